// Grouped expert GEMMs on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16), fp32
// accumulation, LDS-staged tiles filled by direct global->LDS loads (many rows
// per expert).
//
// Expert FFN of "Mixtral of Experts" (xyznot digest, "Method" section and
// "Key terms"): SwiGLU_e(u) = W2_e (SiLU(W1_e u) (*) W3_e u).  The GeekNews
// summary ("Implementasi dan Efisiensi Inferensi") describes running all
// experts as one grouped product over an uneven number of tokens per expert;
// here the rows of every expert are contiguous after the permutation stage
// and a workgroup owns one output tile of one expert.
//
//   gate/up:  H[p][f] = bf16( SiLU(u_p . W1_e[f]) * (u_p . W3_e[f]) )
//             A rows are gathered, u_p = x[perm[p] / K]; the B tile holds
//             W1 rows and the same W3 rows, so the SiLU*mul epilogue finds
//             both accumulators in the same lane.
//   down:     O[s][p][c] = sum over the K range of split s of H_p . W2_e[c]
//             (fp32; only the tiles of the last round -- rows from R0 on --
//             are split along K, and the combine adds their partial sums).
//
// Tile shapes.  Gate/up and down: four waves, each holding a 128 x 128 fp32
// accumulator (4 x 4 MFMA tiles of 32 x 32, 256 accumulators per lane, in
// AGPRs, one wave per SIMD); per 16-deep K sub-step a wave reads 4 A and 4 B
// fragments from LDS for 16 MFMAs.  The backward's K-row products run eight
// waves of 128 x 64 (two per SIMD).  A workgroup owns 256 token rows x 256 B
// rows (waves 2 x 2 or 2 x 4), or -- for an expert's last row tile when it
// has at most 128 rows -- 128 token rows x 512 B rows (waves 1 x 4 or
// 1 x 8), the same MFMA work over twice the columns, so a short tail costs
// half a tile instead of a whole one.  Both operands are K-contiguous
// ([out][in] weights), the per-lane 8-element K
// run each MFMA operand wants; the weights are the MFMA's first operand, so
// a lane ends up owning 4 contiguous output columns.
//
// Pipeline.  Two LDS stages of 64-deep A and B tiles (rows of 128 bytes, the
// 16-byte chunk XOR-swizzled by (row / 2) % 8 so that the fragment reads of
// 16 consecutive rows hit distinct banks).  Gate/up and the backward fill a
// stage with buffer loads with the LDS flag (global -> LDS, no registers, no
// LDS write instructions), issued one step ahead among the MFMAs of the first
// two sub-steps of a step; one barrier per step waits for them (four-wave
// square gate/up tiles also prefetch their weight rows into L2 two steps
// ahead).  The down projection's four-wave tiles stage through registers
// instead: loads in address order two steps ahead, LDS writes to the
// swizzled slots one step ahead, spread over three sub-steps.  Rows past the tile are clamped
// to a valid row (never stored); a K tail and the step past the end load
// through an out-of-range offset, which writes zeros.  Outputs leave through
// LDS as whole 16-byte
// chunks of rows, with non-temporal stores.
//
// The same tile body also runs the backward's products with K-row operands
// ([K][cols] tiles read with the transposing LDS read): r = dy W2_e, the dx
// product and the weight gradients.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int BK = 64;              // K per step
constexpr int ROW_BYTES = BK * 2;   // one LDS row
constexpr int CH = ROW_BYTES / 16;  // 16-byte chunks per row
constexpr int RPB = 256 / ROW_BYTES;  // rows per 256-byte bank sweep
constexpr int KSUB = BK / 16;       // MFMA sub-steps per K step
constexpr int ROWS_LD = 1024 / ROW_BYTES;  // LDS rows per load instruction

template <int BM_, int BN_, int WM_, int WN_>
struct Shape {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int STAGE_BYTES = (BM + BN) * ROW_BYTES;
};
// NWV waves per workgroup: 4 (one per SIMD, 128 x 128 each) or 8 (two per
// SIMD, 128 x 64 each).
template <int NWV>
using Square = Shape<256, 256, 2, NWV / 2>;  // full row tiles
template <int NWV>
using Wide = Shape<128, 512, 1, NWV>;        // an expert's last row tile of <= 128 rows
template <int NWV>
using Narrow = Shape<64, 512, 1, NWV>;       // ... of <= 64 rows: half the MFMA work
constexpr int STAGE_MAX = (128 + 512) * ROW_BYTES;  // the larger (wide) stage

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                             0x00020000);
}

// s_waitcnt immediate: vector-memory count vm (6 bits, split), LDS count lgkm,
// export count left at its maximum.
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8);
}

struct TileArgs {
    const uint16_t* A;
    int64_t A_src_rows;
    const int32_t* perm;
    int K;
    const uint16_t* B1;  // this expert's weights
    const uint16_t* B3;
    int Kdim, N;
    void* Cout;           // already offset to this split's partial sums
    void* Cout2 = nullptr;  // [a | b] rows (gate/up that stores H and [a | b])
    int row0, rows, n0;   // tile rows [row0, row0 + rows), first output column
    int k_begin, k_end;   // K steps of this split
    // K-row operands (stored [K][columns], the tile's M or N columns
    // contiguous): row stride in elements, the K row of step 0, the first K
    // row that loads zeros, and the K row where B continues in B3 (row -
    // b_split) instead of B1.
    int64_t a_stride = 0, b_stride = 0;
    int krow0 = 0, klim = 0, b_split = 0;
};

typedef short v4i16_t __attribute__((ext_vector_type(4)));

// Transposing LDS read (ds_read_b64_tr_b16).  In each group of 16 lanes,
// source lane 4 r + q points at 4 consecutive bf16 of row r; result lane j
// receives element j of the 16 elements of rows r = 0..3 (r-th value from
// row r).  With rows = 4 consecutive K and the 4 lanes of a row covering 16
// consecutive columns, lane j gets 4 consecutive K of column j: the MFMA
// operand layout, read from a [K][columns] tile.
__device__ __forceinline__ v4i16_t lds_read_tr(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16_t*)(p));
}

// One output tile: loads, MFMA main loop and epilogue.  S0 and S1 are the two
// LDS stages (separate objects, so the compiler can tell the stage being read
// from the stage being filled).
// EPI 2 (plain products): the fp32 sums are stored rounded to bf16.
// EPI 3 (gate/up): H into Cout and the rows [a | b] into Cout2.
// EPI (gate/up): 0 stores H = bf16(SiLU(a) * b); 1 stores the
// pre-activations themselves, a and b in bf16, as rows [a | b] of 2 N columns
// (the backward pass needs them).
// AKR / BKR: the A / B operand is a K-row operand ([K][M] / [K][N], rows of
// K; see TileArgs), staged as [64][BM] / [64][BN] tiles and read with the
// transposing LDS read; otherwise it is K-contiguous as described above.
// KD: K depth of a step (64; 32 only when both operands are K-row).
template <bool GATEUP, bool KTAIL, class SH, int STG, int EPI = 0, bool AKR = false,
          bool BKR = false, int KD = BK>
__device__ __forceinline__ void tile_body(const TileArgs& t, uint8_t* S0, uint8_t* S1) {
    constexpr int BM = SH::BM, BN = SH::BN, WM = SH::WM, WN = SH::WN, NW = WM * WN;
    constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile (accumulator space)
    constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 MFMA tiles per wave
    constexpr int A_BYTES = BM * KD * 2;          // A tile of one stage
    constexpr int STAGE_BYTES = (BM + BN) * KD * 2;
    constexpr int KS = KD / 16;                   // MFMA sub-steps per step
    static_assert((TM == 4 || TM == 2) && (TN == 4 || TN == 2),
                  "waves of 128 or 64 rows x 128 or 64 columns");
    static_assert(STAGE_BYTES <= STG, "stage fits (STG: bytes of each stage object)");
    static_assert(!(GATEUP && (AKR || BKR)), "K-row operands only in plain products");
    static_assert(KD == BK || (KD == 32 && AKR && BKR), "32-deep steps: K-row operands only");
    // the K-row swizzle XORs the chunk index with up to 12: rows of >= 16 chunks
    static_assert((!AKR || BM >= 128) && (!BKR || BN >= 128), "K-row tiles of >= 128 columns");

    const int Kdim = t.Kdim, N = t.N, rows = t.rows, n0 = t.n0;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = wid % WM, wn = wid / WM;

    // ---- loader: global -> LDS (directly, or through staging registers) -------
    // A buffer load with the LDS flag writes lane l's 16 bytes at LDS address
    // M0 + 16 l, so one instruction fills 1 KB = ROWS_LD consecutive LDS rows.
    // Lane l serves row ROWS_LD q + l / CH and physical chunk l % CH, i.e. the
    // logical chunk (l % CH) ^ swizzle(row): it fetches exactly the 16 bytes
    // that belong there, and the CH lanes of a row together read its 128-byte
    // K slice.  Each wave issues A_LD + B_LD such loads per K step.
    constexpr int A_LD = BM * KD * 2 / 1024 / NW;  // A loads per wave per K step
    constexpr int B_LD = BN * KD * 2 / 1024 / NW;
    constexpr int NLD = A_LD + B_LD;
    static_assert(A_LD * 1024 * NW == BM * KD * 2 && B_LD * 1024 * NW == BN * KD * 2,
                  "loader split");
    static_assert(!GATEUP || B_LD % 2 == 0, "W1 and W3 halves of the B tile");
    // Register-staged loads (the down projection's four-wave tiles): each
    // lane loads its chunk in natural order (lane l: row l / CH, chunk l % CH,
    // so the CH lanes of a row read its 128 bytes in address order) into
    // VGPRs two K steps ahead, and writes it to its swizzled LDS slot one
    // step later.  Measured A/B in one process, bitwise-identical output:
    // down -9..-12% (prefill, skew, stack layer).  On gate/up it was neutral
    // (within 1.5%), and gate/up keeps the direct loads and the L2 touch.
    constexpr bool RSTAGE = !GATEUP && !AKR && !BKR && NW == 4;
    // The lane's loader coordinates are recomputed for every tile from an
    // opaque copy of the lane id: hoisted out of the kernel's tile loop they
    // stayed live across the K loop and the epilogue, and the register
    // allocator parked them in scratch (gate/up, 12 bytes per lane).
    int lane_t = lane;
    __asm__ __volatile__("" : "+v"(lane_t));
    const int rr = lane_t / CH, pc = lane_t % CH;
    const uint32_t src_row_bytes = (uint32_t)Kdim * 2u;
    const __amdgpu_buffer_rsrc_t a_rs = rsrc(t.A, t.A_src_rows * (int64_t)Kdim * 2);
    const int64_t wbytes = (int64_t)N * Kdim * 2;
    const __amdgpu_buffer_rsrc_t b1_rs = rsrc(t.B1, wbytes);
    const __amdgpu_buffer_rsrc_t b3_rs = GATEUP ? rsrc(t.B3, wbytes) : b1_rs;
    const __amdgpu_buffer_rsrc_t null_rs = rsrc(t.A, 0);
    // first LDS row of load i (A, B)
    auto a_lrow = [&](int i) { return (wid * A_LD + i) * ROWS_LD; };
    auto b_lrow = [&](int i) {
        if (!GATEUP) return (wid * B_LD + i) * ROWS_LD;
        constexpr int H = B_LD / 2;  // loads i < H: W1 rows, i >= H: the matching W3 rows
        return (i < H ? 0 : BN / 2) + (wid * H + (i < H ? i : i - H)) * ROWS_LD;
    };
    uint32_t a_off[A_LD], b_off[B_LD];
    int a_k8[A_LD], b_k8[B_LD];  // first K element of the lane's chunk (tails only)
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = a_lrow(i) + rr;
        const int c = RSTAGE ? pc : pc ^ ((r / RPB) % CH);
        const int p = t.row0 + min(r, rows - 1);  // rows past the tile: a valid row, never stored
        const uint32_t src = GATEUP ? (uint32_t)(t.perm[p] / t.K) : (uint32_t)p;
        a_off[i] = src * src_row_bytes + (uint32_t)c * 16u;
        a_k8[i] = c * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = b_lrow(i) + rr;
        const int c = RSTAGE ? pc : pc ^ ((r / RPB) % CH);
        const int col = n0 + (GATEUP && r >= BN / 2 ? r - BN / 2 : r);
        b_off[i] = (uint32_t)min(col, N - 1) * src_row_bytes + (uint32_t)c * 16u;
        b_k8[i] = c * 8;
    }
    // K-row operands: a load instruction fills 1 KB = KR_RPI rows of a
    // [64][BX] tile (BX / 8 chunks per row); lane l serves tile row
    // KR_RPI q + l / (BX / 8) and physical chunk l % (BX / 8), the logical
    // chunk (l % (BX / 8)) ^ 4 (row % 4).  The XOR moves the four rows a
    // 16-lane group reads to four different 64-byte blocks of a 256-byte bank
    // sweep (see read_frags).  Columns past the operand's last one are
    // clamped to it (never stored); K rows at or past klim load zeros.
    constexpr int A_CPR = BM / 8, B_CPR = BN / 8;      // chunks per K row
    constexpr int A_RPI = 64 / A_CPR, B_RPI = 64 / B_CPR;  // K rows per instruction
    int a_kr[AKR ? A_LD : 1], b_kr[BKR ? B_LD : 1];      // tile K row of the lane
    uint32_t a_colb[AKR ? A_LD : 1], b_colb[BKR ? B_LD : 1];  // column byte offset
    if constexpr (AKR) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int kr = (wid * A_LD + i) * A_RPI + lane / A_CPR;
            const int c = (lane % A_CPR) ^ (4 * (kr & 3));
            a_kr[i] = kr;
            a_colb[i] = (uint32_t)(t.row0 + min(8 * c, rows - 8)) * 2u;
        }
    }
    if constexpr (BKR) {
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int kr = (wid * B_LD + i) * B_RPI + lane / B_CPR;
            const int c = (lane % B_CPR) ^ (4 * (kr & 3));
            b_kr[i] = kr;
            b_colb[i] = (uint32_t)(n0 + min(8 * c, N - n0 - 8)) * 2u;
        }
    }
    // (descriptors are built per load from a selected base and size: a select
    // between descriptor values is lowered through scratch memory)
    const uint32_t a_rowb = (uint32_t)t.a_stride * 2u, b_rowb = (uint32_t)t.b_stride * 2u;
    const int64_t akr_bytes = AKR ? (int64_t)t.klim * t.a_stride * 2 : 0;
    const int b1_rows = min(t.b_split, t.klim);
    const int64_t bkr1_bytes = BKR ? (int64_t)b1_rows * t.b_stride * 2 : 0;
    const int64_t bkr3_bytes = BKR && t.B3 ? (int64_t)(t.klim - b1_rows) * t.b_stride * 2 : 0;
    const uint16_t* bkr3_base = t.B3 ? t.B3 : t.B1;
    const int k_end = t.k_end;
    // Loads of K step kt into stage `st`.  A step past the end goes through a
    // zero-size resource: every load is out of range and writes zeros, so the
    // issue pattern and the load count stay the same.  K tails: chunks past
    // Kdim get an out-of-range offset.
    // Register staging: loads lo .. hi - 1 of K step kt into the staging
    // registers (a step past the end reads zeros through the zero-size
    // resource), and the staged loads lo .. hi - 1 written to stage `st` at
    // the swizzled slot of their (row, chunk).
    u32x4_t ra[RSTAGE ? A_LD : 1], rb[RSTAGE ? B_LD : 1];
    auto gload = [&](int kt, int lo, int hi) {
        if constexpr (RSTAGE) {
            const bool live = kt < k_end;
            const int k0 = live ? kt * BK : 0;
            const __amdgpu_buffer_rsrc_t ars = live ? a_rs : null_rs;
            const __amdgpu_buffer_rsrc_t brs = live ? b1_rs : null_rs;
#pragma unroll
            for (int i = 0; i < A_LD; ++i) {
                if (i < lo || i >= hi) continue;
                const uint32_t off = KTAIL && k0 + a_k8[i] >= Kdim ? 0x80000000u : a_off[i];
                ra[i] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ars, (int)off, k0 * 2, 0));
            }
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                if (A_LD + i < lo || A_LD + i >= hi) continue;
                const uint32_t off = KTAIL && k0 + b_k8[i] >= Kdim ? 0x80000000u : b_off[i];
                rb[i] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(brs, (int)off, k0 * 2, 0));
            }
        }
    };
    auto sstore = [&](uint8_t* st, int lo, int hi) {
        if constexpr (RSTAGE) {
#pragma unroll
            for (int i = 0; i < A_LD; ++i) {
                if (i < lo || i >= hi) continue;
                const int r = a_lrow(i) + rr;
                *reinterpret_cast<u32x4_t*>(st + r * ROW_BYTES + ((pc ^ ((r / RPB) % CH)) << 4)) =
                    ra[i];
            }
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                if (A_LD + i < lo || A_LD + i >= hi) continue;
                const int r = b_lrow(i) + rr;
                *reinterpret_cast<u32x4_t*>(st + A_BYTES + r * ROW_BYTES +
                                            ((pc ^ ((r / RPB) % CH)) << 4)) = rb[i];
            }
        }
    };
    // Loads lo .. hi - 1 of the step's NLD (A loads first, then B loads).
    auto issue = [&](uint8_t* st, int kt, int lo = 0, int hi = 1 << 30) {
        const bool live = kt < k_end;
        const int k0 = live ? kt * BK : 0;
        const uint32_t kb = (uint32_t)k0 * 2u;
        const __amdgpu_buffer_rsrc_t ars = live ? a_rs : null_rs;
        const __amdgpu_buffer_rsrc_t brs1 = live ? b1_rs : null_rs;
        const __amdgpu_buffer_rsrc_t brs3 = live ? b3_rs : null_rs;
        const int krow = t.krow0 + (live ? kt : 0) * KD;  // K row of tile row 0
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            if (i < lo || i >= hi) continue;
            if constexpr (AKR) {
                const int r = krow + a_kr[i];
                const uint32_t off =
                    r < t.klim ? (uint32_t)r * a_rowb + a_colb[i] : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc(t.A, live ? akr_bytes : 0),
                    (__attribute__((address_space(3))) void*)(st + (wid * A_LD + i) * 1024), 16,
                    off, 0, 0, 0);
            } else {
                const uint32_t off = KTAIL && k0 + a_k8[i] >= Kdim ? 0x80000000u : a_off[i];
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ars, (__attribute__((address_space(3))) void*)(st + a_lrow(i) * ROW_BYTES),
                    16, off, kb, 0, 0);
            }
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            if (A_LD + i < lo || A_LD + i >= hi) continue;
            if constexpr (BKR) {
                // the instruction's first row decides B1 or B3 (b_split is a
                // multiple of the rows per instruction)
                const int r0 = krow + (wid * B_LD + i) * B_RPI;
                const bool in3 = r0 >= t.b_split;
                const int r = krow + b_kr[i] - (in3 ? t.b_split : 0);
                const int lim = in3 ? t.klim - t.b_split : b1_rows;
                const uint32_t off = r < lim ? (uint32_t)r * b_rowb + b_colb[i] : 0x80000000u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc(in3 ? bkr3_base : t.B1, live ? (in3 ? bkr3_bytes : bkr1_bytes) : 0),
                    (__attribute__((address_space(3))) void*)(st + A_BYTES +
                                                              (wid * B_LD + i) * 1024),
                    16, off, 0, 0, 0);
            } else {
                const uint32_t off = KTAIL && k0 + b_k8[i] >= Kdim ? 0x80000000u : b_off[i];
                const bool second = GATEUP && i >= B_LD / 2;  // compile-time
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    second ? brs3 : brs1,
                    (__attribute__((address_space(3))) void*)(st + A_BYTES +
                                                              b_lrow(i) * ROW_BYTES),
                    16, off, kb, 0, 0);
            }
        }
    };

    // Weight rows of four-wave square tiles are prefetched into L2 two K
    // steps ahead.  Each weight panel's K slice comes from HBM the first time
    // a tile reaches it, and one step of LDS prefetch leaves that latency
    // exposed (waiting on the B loads took ~19% of a wave's loop at
    // T = 4096).  One 4-byte load per B row (one 128-byte line of the row's K
    // slice) goes out after all stage loads of the step, into a register
    // consumed a step later; loads complete in issue order, so the barrier's
    // vmcnt(1) leaves exactly that load outstanding.  Measured: gate/up 2-4%
    // faster, the four-wave down projection 4-5% (on the eight-wave one it
    // was slower).
    constexpr bool TOUCH = SH::BM == 256 && SH::BN == 256 && NW == 4 && !AKR && !BKR && !RSTAGE;
    auto touch = [&](int kt2) -> uint32_t {
        if constexpr (TOUCH) {
            const int r = wid * 64 + lane;  // B tile row (gate/up: W1 rows, then W3 rows)
            const bool w3 = GATEUP && wid >= 2;  // wave-uniform
            const int col = n0 + (GATEUP ? (r & (BN / 2 - 1)) : r);
            const uint32_t off =
                KTAIL && kt2 * BK >= Kdim
                    ? 0x80000000u
                    : (uint32_t)min(col, N - 1) * src_row_bytes + (uint32_t)kt2 * BK * 2u;
            return __builtin_amdgcn_raw_buffer_load_b32(
                rsrc(w3 ? t.B3 : t.B1, kt2 < k_end ? wbytes : 0), off, 0, 0);
        }
        return 0u;
    };
    uint32_t touched = 0;  // the previous step's prefetch load, consumed a step later

    // ---- MFMA read coordinates ----------------------------------------------
    // Every row a lane reads is congruent to l32 modulo 32, so its swizzle is
    // the lane's own constant: fragment (i, sub-step kk) sits at a per-lane
    // base plus kofs[kk] plus a compile-time row offset.
    const int l32 = lane & 31, khalf = lane >> 5;
    const int sw = (l32 / RPB) % CH;
    uint32_t kofs[KSUB];
#pragma unroll
    for (int kk = 0; kk < KSUB; ++kk) kofs[kk] = (uint32_t)(((kk * 2 + khalf) ^ sw) << 4);
    const uint32_t a_rd = (uint32_t)(wm * WTM + l32) * ROW_BYTES;
    const uint32_t b_rd = A_BYTES + (uint32_t)(wn * (GATEUP ? WTN / 2 : WTN) + l32) * ROW_BYTES;
    auto b_frag_row = [](int j) {  // first B row of fragment j, relative to the wave's rows
        if (!GATEUP) return j * 32;
        constexpr int half = TN / 2;
        return (j < half ? 0 : BN / 2) + (j < half ? j : j - half) * 32;
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // K-row fragments: lane l = 16 g + i16 of fragment f (32 columns from
    // wave column c0 + 32 f) points at tile row 8 (g / 2) + i16 / 4 (+ 16 kk,
    // + 4 for the second read) and column c0 + 32 f + 16 (g % 2) + 4 (i16 % 4),
    // so lane l receives column c0 + 32 f + l % 32 at K rows 16 kk + 8 (l / 32)
    // + 0..7.  Row % 4 = i16 / 4, so the swizzle is the lane's own constant.
    // The 32 lanes of a half wave read 4 rows x 64 bytes, one 64-byte block
    // per row, spread over a 256-byte bank sweep by the swizzle.
    auto kr_off = [&](int c0, int f, int pitch) {
        const int g = lane >> 4, i16 = lane & 15;
        const int row = 8 * (g >> 1) + (i16 >> 2);
        const int chunk = ((c0 + 32 * f) >> 3) + 2 * (g & 1) + ((i16 & 3) >> 1);
        return (uint32_t)(row * pitch + ((chunk ^ (4 * (row & 3))) << 4) + (i16 & 1) * 8);
    };
    constexpr int A_PITCH = BM * 2, B_PITCH = BN * 2;
    uint32_t a_fr[AKR ? TM : 1], b_fr[BKR ? TN : 1];
    if constexpr (AKR) {
#pragma unroll
        for (int i = 0; i < TM; ++i) a_fr[i] = kr_off(wm * WTM, i, A_PITCH);
    }
    if constexpr (BKR) {
#pragma unroll
        for (int j = 0; j < TN; ++j) b_fr[j] = A_BYTES + kr_off(wn * WTN, j, B_PITCH);
    }
    auto tr_frag = [](const uint8_t* p, int pitch) {
        const v4i16_t lo = lds_read_tr(p), hi = lds_read_tr(p + 4 * pitch);
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    auto read_frags = [&](const uint8_t* st, int kk, bf16x8_t(&av)[TM], bf16x8_t(&bv)[TN]) {
        const uint8_t* pa = st + a_rd + kofs[kk];
        const uint8_t* pb = st + b_rd + kofs[kk];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            if constexpr (AKR)
                av[i] = tr_frag(st + a_fr[i] + kk * 16 * A_PITCH, A_PITCH);
            else
                av[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(pa + i * 32 * ROW_BYTES));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            if constexpr (BKR)
                bv[j] = tr_frag(st + b_fr[j] + kk * 16 * B_PITCH, B_PITCH);
            else
                bv[j] = as_bf16x8(
                    *reinterpret_cast<const u32x4_t*>(pb + b_frag_row(j) * ROW_BYTES));
        }
    };
    auto mfmas = [&](const bf16x8_t(&av)[TM], const bf16x8_t(&bv)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i], acc[i][j], 0,
                                                                    0, 0);
    };
    // Scheduling hints (group masks: 0x008 MFMA, 0x020 VMEM read, 0x100 LDS
    // read): the LDS reads of the next sub-step go out one per MFMA at the
    // start of a sub-step, so their latency hides behind the remaining MFMAs;
    // the first sub-step of a step also carries the next step's loads (LPM
    // per MFMA).  Register staging instead puts one LDS write, then one load,
    // on every third MFMA: bunched writes filled the LDS data FIFO and
    // stalled the wave (every third MFMA measured 2-3% faster than every
    // other, and 7-11% faster than one per MFMA).
    constexpr int NRD = (AKR ? 2 : 1) * TM + (BKR ? 2 : 1) * TN;  // LDS reads per sub-step
    auto interleave = [&](int nloads, int nwrites = 0) {
        constexpr int LPM = (NLD + TM * TN - 1) / (TM * TN);
        constexpr int RPM = (NRD + TM * TN - 1) / (TM * TN);
#pragma unroll
        for (int q = 0; q < TM * TN; ++q) {
#pragma unroll
            for (int r = 0; r < RPM; ++r)
                if (q * RPM + r < NRD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (nwrites > 0) {
                if (q % 3 == 0 && q / 3 < nwrites) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
                if (q % 3 == 2 && q / 3 < nloads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            } else {
#pragma unroll
                for (int r = 0; r < LPM; ++r)
                    if (q * LPM + r < nloads) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
    };
    // Block-wide barrier that waits for this wave's loads (the step about to
    // be read) and its own LDS reads (the stage they read is refilled next);
    // the youngest load, an L2 prefetch, may stay in flight.
    // With register staging nothing of the step about to be read is in
    // flight (its data went through VGPRs), and the staged loads stay in
    // flight across the barrier.
    auto barrier = [&]() {
        if constexpr (RSTAGE)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(TOUCH ? 1 : 0, 0));
        __builtin_amdgcn_s_barrier();
        __asm__ __volatile__("" ::: "memory");
    };

    // One K step kt from stage X: while the MFMAs of sub-step s - 1 run, the
    // fragments of sub-step s are read (and, in the first sub-step, the
    // loads of step kt + 1 go into stage Y, free since the last barrier);
    // then the barrier publishes Y, whose first fragments are read while the
    // last MFMAs of X run.
    // Four-wave tiles spread the step's loads over sub-steps 1 and 2: bunched
    // into one sub-step (one load per MFMA) they fill the texture units'
    // address and command FIFOs and stall the SIMD's only wave between its
    // MFMAs (FIFO-full stall counters 10x those of hipBLASLt's kernel on the
    // same product).  Measured: gate/up 3.3-6.7% faster; the eight-wave
    // tiles, whose SIMDs hold a second wave, were not.
    // Register staging spreads over sub-steps 1 .. KS - 1 instead: in each,
    // part of stage Y is written from the staging registers (step kt + 1,
    // loaded during step kt - 1), and the same registers are then reloaded
    // with that part of step kt + 2.
    constexpr int SPREAD = RSTAGE ? KS - 1 : NW == 4 && KS > 2 ? 2 : 1;
    bf16x8_t fa[2][TM], fb[2][TN];
    auto step = [&](const uint8_t* X, uint8_t* Y, int kt) {
        uint32_t touch_now = 0;
#pragma unroll
        for (int sub = 1; sub < KS; ++sub) {
            const int lo = sub <= SPREAD ? (sub - 1) * NLD / SPREAD : NLD;
            const int hi = sub <= SPREAD ? sub * NLD / SPREAD : NLD;
            if constexpr (RSTAGE) {
                if (hi > lo) {
                    sstore(Y, lo, hi);
                    gload(kt + 2, lo, hi);
                }
            } else if (hi > lo) {
                issue(Y, kt + 1, lo, hi);
            }
            read_frags(X, sub, fa[sub & 1], fb[sub & 1]);
            mfmas(fa[(sub - 1) & 1], fb[(sub - 1) & 1]);
            interleave(hi - lo, RSTAGE ? hi - lo : 0);
            __builtin_amdgcn_sched_barrier(0);
            if (TOUCH && sub == SPREAD) {  // after every stage load of the step
                touch_now = touch(kt + 2);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (TOUCH) __asm__ __volatile__("" ::"v"(touched));
        barrier();
        touched = touch_now;
        __builtin_amdgcn_sched_barrier(0);
        read_frags(Y, 0, fa[0], fb[0]);  // past the last step: unused
        mfmas(fa[1], fb[1]);
        interleave(0);
        __builtin_amdgcn_sched_barrier(0);
    };

    if constexpr (RSTAGE) {
        gload(t.k_begin, 0, NLD);
        sstore(S0, 0, NLD);
        gload(t.k_begin + 1, 0, NLD);
    } else {
        issue(S0, t.k_begin);
    }
    if constexpr (TOUCH) {
        __builtin_amdgcn_sched_barrier(0);
        touched = touch(t.k_begin + 1);
        __builtin_amdgcn_sched_barrier(0);
    }
    barrier();
    read_frags(S0, 0, fa[0], fb[0]);
    for (int kt = t.k_begin; kt < k_end; kt += 2) {
        step(S0, S1, kt);
        step(S1, S0, kt + 1);
    }
    // Drain: the loads past the last step are out of range but still write
    // LDS (or staging registers); wait for them before the stages are reused
    // for staging.
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    if constexpr (TOUCH) __asm__ __volatile__("" ::"v"(touched));

    // ---- epilogue -------------------------------------------------------------
    // The MFMAs ran with the weights as the first operand, so the 32x32
    // accumulator of lane l, register r holds token row l%32 of the i-tile
    // and output column 8*(r/4) + 4*(l/32) + r%4 of the j-tile: a lane owns 4
    // contiguous columns per group of 4 registers.  Each wave stages one
    // i-tile at a time (32 rows x its WTN (down) or WTN/2 (gate/up) columns)
    // in its own LDS slot, padded by 16 bytes per row against bank
    // conflicts, and writes it back as whole 16-byte chunks of output rows.
    constexpr int OCOLS = GATEUP ? WTN / 2 : WTN;           // output columns per wave
    constexpr int ES = GATEUP || EPI == 2 ? 2 : 4;           // output element bytes
    constexpr int RSTRIDE = OCOLS * ES + 16;                 // LDS row stride (bytes)
    constexpr int SLOT = 32 * RSTRIDE;                       // one wave's staging slot
    static_assert(SLOT * (NW / 2) <= STG, "half the waves stage in each stage buffer");
    __syncthreads();  // every wave is done with the K-loop LDS
    // the epilogue's lane coordinates, likewise from an opaque lane id (not
    // kept from before the K loop)
    int lane_e = lane;
    __asm__ __volatile__("" : "+v"(lane_e));
    const int l32e = lane_e & 31, khalfe = lane_e >> 5;
    uint8_t* slot = (wid < NW / 2 ? S0 : S1) + (wid % (NW / 2)) * (STG / (NW / 2));
    const int col_w = n0 + wn * OCOLS;  // first output column of this wave
    constexpr int CPR = OCOLS * ES / 16;      // 16-byte chunks per staged row
    constexpr int RPI = kWave / CPR;          // rows per store instruction
    // Gate/up passes: EPI 0 stores H; EPI 1 stores a then b into rows
    // [a | b] of t.Cout; EPI 3 stores H into t.Cout and then a, b into t.Cout2.
    constexpr int PASSES = !GATEUP ? 1 : EPI == 1 ? 2 : EPI == 3 ? 3 : 1;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int pass = 0; pass < PASSES; ++pass) {
            // pass writes H (h_pass) or the pre-activation half ab_half of [a | b]
            const bool h_pass = GATEUP && (EPI == 0 || (EPI == 3 && pass == 0));
            const int ab_half = EPI == 3 ? pass - 1 : pass;
            // stage rows wm*WTM + 32i .. +31
#pragma unroll
            for (int j = 0; j < (GATEUP ? TN / 2 : TN); ++j) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int c = j * 32 + 8 * q + 4 * khalfe;  // column within the wave
                    uint8_t* dst = slot + l32e * RSTRIDE + c * ES;
                    if (GATEUP && !h_pass) {
                        const f32x16_t& v = acc[i][j + ab_half * (TN / 2)];
                        u32x2_t h;
                        h.x = pack_bf16x2(v[4 * q + 0], v[4 * q + 1]);
                        h.y = pack_bf16x2(v[4 * q + 2], v[4 * q + 3]);
                        *reinterpret_cast<u32x2_t*>(dst) = h;
                    } else if (GATEUP) {
                        const f32x16_t& g = acc[i][j];
                        const f32x16_t& u = acc[i][j + TN / 2];
                        u32x2_t h;
                        h.x = pack_bf16x2(silu_bf16out(g[4 * q + 0]) * u[4 * q + 0],
                                          silu_bf16out(g[4 * q + 1]) * u[4 * q + 1]);
                        h.y = pack_bf16x2(silu_bf16out(g[4 * q + 2]) * u[4 * q + 2],
                                          silu_bf16out(g[4 * q + 3]) * u[4 * q + 3]);
                        *reinterpret_cast<u32x2_t*>(dst) = h;
                    } else if (EPI == 2) {
                        const f32x16_t& a = acc[i][j];
                        u32x2_t h;
                        h.x = pack_bf16x2(a[4 * q + 0], a[4 * q + 1]);
                        h.y = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
                        *reinterpret_cast<u32x2_t*>(dst) = h;
                    } else {
                        const f32x16_t& a = acc[i][j];
                        *reinterpret_cast<f32x4_t*>(dst) =
                            f32x4_t{a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                    }
                }
            }
            // write back: lane -> (row, 16-byte chunk).  The slot is the wave's
            // own and LDS operations of one wave complete in order: no barrier
            // needed (also before the second half overwrites the slot).
#pragma unroll
            for (int rr2 = 0; rr2 < 32; rr2 += RPI) {
                const int r = rr2 + lane_e / CPR, ch = lane_e % CPR;
                const int row = wm * WTM + i * 32 + r;
                const int col = col_w + ch * (16 / ES);
                const u32x4_t v =
                    *reinterpret_cast<const u32x4_t*>(slot + r * RSTRIDE + ch * 16);
                if (row < rows && col < N) {
                    uint8_t* out;
                    if (GATEUP && !h_pass)  // [a | b] rows of 2 N columns
                        out = static_cast<uint8_t*>(EPI == 3 ? t.Cout2 : t.Cout) +
                              ((int64_t)(t.row0 + row) * 2 * N + ab_half * N + col) * ES;
                    else
                        out = static_cast<uint8_t*>(t.Cout) +
                              ((int64_t)(t.row0 + row) * N + col) * ES;
                    // Streaming stores: the output is not read again by this
                    // kernel, and its lines need not displace operand panels
                    // from L2 (weight gradients 4-6% faster, the stack layer's
                    // forward 0.5%).  The 32-deep weight-gradient tiles (a few
                    // rows per expert: a pure write) measured 2% slower so.
                    if constexpr (KD == 32)
                        *reinterpret_cast<u32x4_t*>(out) = v;
                    else
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(out));
                }
            }
        }
    }
}

// BKR (plain products only): B1 / B3 are K-row weights [n][b_split][N]; K
// rows [0, b_split) of the product come from B1_e, [b_split, Kdim) from B3_e.
template <bool GATEUP, bool KTAIL, int NWV, int EPI, bool BKR = false>
__global__ __launch_bounds__(NWV * 64) __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4)))
void gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t A_src_rows,
                      const int32_t* __restrict__ perm, int K, const uint16_t* __restrict__ B1,
                      const uint16_t* __restrict__ B3, const int32_t* __restrict__ offsets,
                      int n, int Kdim, int N, void* __restrict__ Cout, int GM, int splits,
                      int64_t split_stride, int b_split = 0, void* __restrict__ Cout2 = nullptr,
                      int down_wide_max = 0, int cus = 0, int* __restrict__ split_meta = nullptr) {
    // gate/up and the down projection may run wide tiles (larger stages)
    using SQ = Square<NWV>;
    using WD = Wide<NWV>;
    constexpr bool WIDE_OK = true;
    constexpr int STG = WIDE_OK ? STAGE_MAX : SQ::STAGE_BYTES;
    __shared__ __attribute__((aligned(1024))) uint8_t S0[STG];
    __shared__ __attribute__((aligned(1024))) uint8_t S1[STG];

    // ---- tile coordinates -------------------------------------------------
    // Expert e with m rows has m / 256 full row tiles; a remainder of more
    // than 128 rows is one more (partial) square row tile, one of at most 128
    // rows a wide row tile.  The real tiles (per K split) are known only here,
    // from the expert offsets; the grid is an upper bound and blocks past the
    // real tiles exit.  Block b runs on XCD b % 8, and each XCD takes one
    // contiguous eighth of the real tiles, so every XCD gets the same number
    // of tiles and the 32 tiles its CUs run together are neighbours in the
    // order below, sharing token and weight tiles in its L2.
    //
    // Order: (split,) expert, row group (GM square row tiles; the wide row tile
    // joins the last group), column pair, then inside a column pair the
    // group's square tiles of both columns followed by the wide tile that
    // spans them -- all tiles reading one weight panel run back to back.
    constexpr int BNO_S = GATEUP ? SQ::BN / 2 : SQ::BN;  // output columns per tile
    const int ntn_s = (N + BNO_S - 1) / BNO_S;  // square column tiles
    const int npair = (ntn_s + 1) / 2;           // column pairs = wide column tiles
    // Wide tail tiles: gate/up for every tail of at most 128 rows; the plain
    // products for tails of at most down_wide_max rows.
    const int WIDE_MAX = GATEUP ? WD::BM : down_wide_max;
    auto expert_tiles = [&](int m, int& nsq, int& nwide) {
        const int rem = m % SQ::BM;
        nsq = m / SQ::BM + (rem > WIDE_MAX ? 1 : 0);
        nwide = rem > 0 && rem <= WIDE_MAX ? 1 : 0;
        return nsq * ntn_s + nwide * npair;
    };
    int tiles = 0;
    for (int q = 0; q < n; ++q) {
        int a, c;
        tiles += expert_tiles(offsets[q + 1] - offsets[q], a, c);
    }
    // This block's tile L among the tiles of rows [lo, hi), and its K split
    // ks of nsplit.
    int lo = offsets[0], hi = offsets[n], ks = 0, nsplit = splits, L = 0;
    int64_t part0 = 0;  // this block writes output row p at row part0 + p of Cout
    if (cus > 0) {
        // Split only the remainder (the down projection): the tiles fill
        // tiles / cus whole rounds of the CUs, plus r = tiles % cus left over.
        // The last row tiles in expert order (at least r tiles, whole rows of
        // tiles, from row R0 on) run as Sr K splits each, Sr = cus / their
        // count at most, so they make one short round instead of a mostly
        // idle full one; every other tile runs its whole K once.  Rows >= R0
        // hold Sr partial sums, the rest one: buffer 0 holds every row's
        // first ([A][N]), and split s >= 1 of row p >= R0 sits at row
        // A + (s - 1)(A - R0) + p - R0.  (R0, Sr) go to split_meta for the
        // combine.
        int R0 = offsets[n], Sr = 1, Trem = 0;
        const int r = tiles % cus;
        if (r > 0 && splits > 1) {
            for (int q = n - 1; q >= 0 && Trem < r; --q) {
                int nsq_q, nw_q;
                const int s0 = offsets[q];
                expert_tiles(offsets[q + 1] - s0, nsq_q, nw_q);
                if (nw_q) {  // the tail tile (its squares are all full)
                    Trem += npair;
                    R0 = s0 + nsq_q * SQ::BM;
                }
                if (Trem >= r) break;
                const int take = min((r - Trem + ntn_s - 1) / ntn_s, nsq_q);
                Trem += take * ntn_s;
                if (take > 0) R0 = s0 + (nsq_q - take) * SQ::BM;
            }
            // Partial sums past the first are stored for rows >= R0 only,
            // (A - R0) rows per split, in the (splits - 1) A rows of buffers
            // the workspace holds beyond buffer 0: that bounds Sr, as do the
            // K steps (and 16, so each split keeps several).
            const int64_t rows_rem = (int64_t)offsets[n] - R0;
            const int64_t fit = 1 + (int64_t)(splits - 1) * offsets[n] / max((int64_t)1, rows_rem);
            const int nk = (Kdim + BK - 1) / BK;
            Sr = (int)min((int64_t)min(min(cus / Trem, nk), 16), fit);
            if (Sr < 2) {
                Sr = 1;
                R0 = offsets[n];
                Trem = 0;
            }
        }
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            split_meta[0] = R0;
            split_meta[1] = Sr;
        }
        // blocks [0, 8 per_xcd): the whole-K tiles, a contiguous eighth per
        // XCD as below; then the split tiles, consecutive ones on different
        // XCDs (block b runs on XCD b % 8)
        const int Tdp = tiles - Trem;
        const int per_xcd = (Tdp + 7) / 8;
        if ((int)blockIdx.x < 8 * per_xcd) {
            L = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
            if (L >= Tdp) return;
            hi = R0;
            nsplit = 1;
        } else {
            const int u = (int)blockIdx.x - 8 * per_xcd;
            if (u >= Trem * Sr) return;
            ks = u / Trem;
            L = u - ks * Trem;
            lo = R0;
            nsplit = Sr;
            // split ks >= 1 writes row p to row A + (ks - 1)(A - R0) + p - R0
            if (ks > 0)
                part0 = (int64_t)offsets[n] + (int64_t)(ks - 1) * (offsets[n] - R0) - R0;
        }
    } else {
        const int per_xcd = (tiles * splits + 7) / 8;
        const int jx = (int)(blockIdx.x >> 3);
        const int L0 = (int)(blockIdx.x & 7) * per_xcd + jx;
        if (jx >= per_xcd || L0 >= tiles * splits) return;
        ks = L0 / tiles;  // K split of this block
        L = L0 - ks * tiles;
        part0 = split_stride / N * ks;  // buffer ks: rows A ks ..
    }
    // the expert of tile L, over the rows of [lo, hi) (R0 is a row-tile
    // boundary of its expert, so both sides keep the expert's own tiling)
    int e = 0, start = 0, end = 0, nsq = 0, nwide = 0;
    for (;; ++e) {  // ends: L < the tiles of [lo, hi)
        start = max(offsets[e], lo);
        end = min(offsets[e + 1], hi);
        const int cnt = expert_tiles(max(0, end - start), nsq, nwide);
        if (L < cnt) break;
        L -= cnt;
    }
    // row group: all but the last hold GM square row tiles and no wide tile
    const int ngroups = max(1, (nsq + GM - 1) / GM);
    int g = min(L / (GM * ntn_s), ngroups - 1);
    L -= g * GM * ntn_s;
    const int gm = min(GM, nsq - g * GM);  // square row tiles of this group (may be 0)
    const int w = g == ngroups - 1 ? nwide : 0;
    // column pair: 2 gm + w tiles (gm + w in a last, single-column pair)
    const int c = min(L / (2 * gm + w), npair - 1);
    L -= c * (2 * gm + w);
    const int ncol = min(2, ntn_s - 2 * c);  // square columns in this pair

    TileArgs t;
    t.A = A;
    t.A_src_rows = A_src_rows;
    t.perm = perm;
    t.K = K;
    if constexpr (BKR) {
        t.B1 = B1 + (int64_t)e * b_split * N;
        t.B3 = B3 ? B3 + (int64_t)e * b_split * N : nullptr;
        t.b_stride = N;
        t.krow0 = 0;
        t.klim = Kdim;
        t.b_split = B3 ? b_split : Kdim;
    } else {
        t.B1 = B1 + (int64_t)e * N * Kdim;
        t.B3 = GATEUP ? B3 + (int64_t)e * N * Kdim : nullptr;
    }
    t.Kdim = Kdim;
    t.N = N;
    t.Cout = static_cast<uint8_t*>(Cout) + part0 * N * (GATEUP || EPI == 2 ? 2 : 4);
    t.Cout2 = Cout2;
    const int nk_all = (Kdim + BK - 1) / BK;
    const int per_split = (nk_all + nsplit - 1) / nsplit;
    t.k_begin = min(nk_all, ks * per_split);
    t.k_end = min(nk_all, t.k_begin + per_split);
    if (L < gm * ncol) {
        const int mt = g * GM + L % gm;
        t.row0 = start + mt * SQ::BM;
        t.rows = min(SQ::BM, end - t.row0);
        t.n0 = (2 * c + L / gm) * BNO_S;
        tile_body<GATEUP, KTAIL, SQ, STG, EPI, false, BKR>(t, S0, S1);
    } else if constexpr (WIDE_OK) {
        t.row0 = start + nsq * SQ::BM;
        t.rows = end - t.row0;
        t.n0 = 2 * c * BNO_S;
        // the same tile slot; a tail of at most 64 rows runs on 64-row waves
        if (t.rows <= Narrow<NWV>::BM)
            tile_body<GATEUP, KTAIL, Narrow<NWV>, STG, EPI, false, BKR>(t, S0, S1);
        else
            tile_body<GATEUP, KTAIL, WD, STG, EPI, false, BKR>(t, S0, S1);
    }
}

template <bool GATEUP, int NWV = 4, int EPI = 0>
hipError_t launch_tiled(const uint16_t* A, int64_t A_src_rows, const int32_t* perm, int K,
                        const uint16_t* B1, const uint16_t* B3, const int32_t* offsets, int n,
                        int64_t A_rows, int Kdim, int N, void* C, int GM, int splits,
                        hipStream_t s, void* C2 = nullptr, int down_wide_max = 0, int cus = 0,
                        int* split_meta = nullptr) {
    using SQ = Square<NWV>;
    constexpr int BNO = GATEUP ? SQ::BN / 2 : SQ::BN;
    // upper bound of the tiles: each expert's last row tile may be partial
    // (a wide tile never has more column tiles than a square one); with the
    // remainder split (cus > 0), the whole-K tiles plus at most cus split ones
    const int64_t mslots = A_rows / SQ::BM + n;
    const int64_t ntn = (N + BNO - 1) / BNO;
    const int64_t blocks =
        cus > 0 ? (mslots * ntn + 7) / 8 * 8 + (cus + 7) / 8 * 8 : (mslots * ntn * splits + 7) / 8 * 8;
    if (cus > 0 && (GATEUP || !split_meta)) return hipErrorInvalidValue;
    if (blocks > 0x7fffffff || splits < 1 || (GATEUP && splits != 1))
        return hipErrorInvalidConfiguration;
    const bool ktail = Kdim % BK != 0;
    const int64_t stride = A_rows * (int64_t)N;
    if (ktail)
        hipLaunchKernelGGL((gemm_bf16_kernel<GATEUP, true, NWV, EPI>), dim3((unsigned)blocks),
                           dim3(NWV * 64), 0, s, A, A_src_rows, perm, K, B1, B3, offsets, n, Kdim,
                           N, C, GM, splits, stride, 0, C2, down_wide_max, cus, split_meta);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<GATEUP, false, NWV, EPI>), dim3((unsigned)blocks),
                           dim3(NWV * 64), 0, s, A, A_src_rows, perm, K, B1, B3, offsets, n, Kdim,
                           N, C, GM, splits, stride, 0, C2, down_wide_max, cus, split_meta);
    return hipGetLastError();
}

// Weight gradients of the grouped products.  For every expert e,
//   C_e[r][c] = sum over the expert's assignment rows p of A[p][r] B[p][c],
// with A [A_rows][a_stride] and B [A_rows][b_stride] in expert order (rows
// offsets[e] .. offsets[e+1] - 1 of both): a product over K rows, both
// operands K-row (no transposed copies).  C_e = C + e N1 N2, fp32, every
// element written (zero for an expert without rows).
// SH: tile shape; KD: K depth of a step; WPE: waves per SIMD the registers
// are budgeted for (two workgroups of 4 waves share a CU with 128 x 256
// tiles and 32-deep steps, so one's epilogue overlaps the other's MFMAs).
template <class SH, int KD, int WPE>
__global__ __launch_bounds__(SH::WM * SH::WN * 64)
__attribute__((amdgpu_waves_per_eu(WPE, WPE)))
void gemm_wgrad_kernel(const uint16_t* __restrict__ A, int64_t a_stride,
                       const uint16_t* __restrict__ B, int64_t b_stride,
                       const int32_t* __restrict__ offsets, int n, int N1, int N2,
                       float* __restrict__ C, int GM) {
    using SQ = SH;
    constexpr int STG = (SH::BM + SH::BN) * KD * 2;
    __shared__ __attribute__((aligned(1024))) uint8_t S0[STG];
    __shared__ __attribute__((aligned(1024))) uint8_t S1[STG];
    const int mtn = (N1 + SQ::BM - 1) / SQ::BM, ntn = (N2 + SQ::BN - 1) / SQ::BN;
    const int per_e = mtn * ntn;
    const int tiles = n * per_e;
    // Tile L runs as block L, on XCD L % 8: every XCD gets an equal share of
    // every expert's tiles.  A tile's K length is its expert's row count, so
    // a contiguous share per XCD (as in the forward) would load the XCD that
    // holds the largest expert with its whole work (four times the mean under
    // the skewed routing where one expert takes half the rows).  Inside an
    // expert, groups of GM row tiles, and inside a group the row tile varies
    // fastest.
    const int L0 = (int)blockIdx.x;
    if (L0 >= tiles) return;
    const int e = L0 / per_e, rem = L0 - e * per_e;
    const int pbeg = offsets[e], pend = offsets[e + 1];
    TileArgs t;
    t.A = A;
    t.A_src_rows = 0;
    t.perm = nullptr;
    t.K = 1;
    t.B1 = B;
    t.B3 = nullptr;
    t.Kdim = 0;
    t.N = N2;
    t.Cout = C + (int64_t)e * N1 * N2;
    const int g = rem / (GM * ntn);
    const int gm = min(GM, mtn - g * GM);
    const int r2 = rem - g * GM * ntn;
    const int mt = g * GM + r2 % gm, nt = r2 / gm;
    t.row0 = mt * SQ::BM;
    t.rows = min(SQ::BM, N1 - t.row0);
    t.n0 = nt * SQ::BN;
    t.k_begin = 0;
    t.k_end = (pend - pbeg + KD - 1) / KD;
    t.a_stride = a_stride;
    t.b_stride = b_stride;
    t.krow0 = pbeg;
    t.klim = pend;
    t.b_split = pend;
    tile_body<false, false, SQ, STG, 0, true, true, KD>(t, S0, S1);
}

}  // namespace

bool tiled_fits(int64_t A_src_rows, int64_t Kdim, int64_t N) {
    // buffer offsets are 32-bit: every operand range below 2^31 bytes
    const int64_t lim = int64_t(1) << 31;
    return A_src_rows * Kdim * 2 < lim && N * Kdim * 2 < lim;
}

hipError_t launch_gemm_bf16_tiled(bool gateup, const uint16_t* A, int64_t A_src_rows,
                                  const int32_t* perm, int K, const uint16_t* B1,
                                  const uint16_t* B3, const int32_t* offsets, int n,
                                  int64_t A_rows, int Kdim, int N, void* C, int splits,
                                  int cus, int* split_meta, hipStream_t s) {
    if (!tiled_fits(A_src_rows, Kdim, N) || (!gateup && (cus < 1 || !split_meta)))
        return hipErrorInvalidValue;
    // Four waves of 128 x 128 for both (measured against eight waves of
    // 128 x 64 for the down projection: 4-5% faster once the loads were
    // spread and its weight rows prefetched into L2; it now stages its loads
    // through registers instead, 10-12% faster again).
    const int GM = 8;
    if (gateup)
        return launch_tiled<true, 4>(A, A_src_rows, perm, K, B1, B3, offsets, n, A_rows, Kdim, N,
                                     C, GM, 1, s);
    // Down tails of at most 128 rows run wide as on gate/up (measured: 1%
    // faster on the 32-layer stack at T = 2048, unchanged at T = 4096).  Up
    // to `splits` K splits for the last round's tiles only (see the kernel).
    return launch_tiled<false, 4>(A, A_src_rows, perm, K, B1, B3, offsets, n, A_rows, Kdim, N,
                                  C, GM, splits, s, nullptr, 128, cus, split_meta);
}

}  // namespace moe

namespace moe {

hipError_t launch_gemm_bf16_gateup_ab(const uint16_t* A, int64_t A_src_rows, const int32_t* perm,
                                      int K, const uint16_t* B1, const uint16_t* B3,
                                      const int32_t* offsets, int n, int64_t A_rows, int Kdim,
                                      int N, uint16_t* AB, hipStream_t s) {
    if (!tiled_fits(A_src_rows, Kdim, N)) return hipErrorInvalidValue;
    return launch_tiled<true, 4, 1>(A, A_src_rows, perm, K, B1, B3, offsets, n, A_rows, Kdim, N,
                                    AB, 8, 1, s);
}

hipError_t launch_gemm_bf16_gateup_save(const uint16_t* A, int64_t A_src_rows,
                                        const int32_t* perm, int K, const uint16_t* B1,
                                        const uint16_t* B3, const int32_t* offsets, int n,
                                        int64_t A_rows, int Kdim, int N, uint16_t* H,
                                        uint16_t* AB, hipStream_t s) {
    if (!tiled_fits(A_src_rows, Kdim, N) || !H || !AB) return hipErrorInvalidValue;
    return launch_tiled<true, 4, 3>(A, A_src_rows, perm, K, B1, B3, offsets, n, A_rows, Kdim, N,
                                    H, 8, 1, s, AB);
}

hipError_t launch_gemm_bf16_wgrad(const uint16_t* A, int64_t a_stride, const uint16_t* B,
                                  int64_t b_stride, const int32_t* offsets, int n,
                                  int64_t A_rows, int N1, int N2, float* C, int GM,
                                  hipStream_t s) {
    const int64_t lim = int64_t(1) << 31;
    if (N1 % 8 || N2 % 8 || A_rows * a_stride * 2 >= lim || A_rows * b_stride * 2 >= lim ||
        GM < 1)
        return hipErrorInvalidValue;
    // Few rows per expert (a K step or two per tile): each tile is mostly its
    // 256 KB fp32 write, so two workgroups of 128 x 256 tiles share a CU and
    // one's stores overlap the other's work (measured 7% faster at 4 rows per
    // expert, 14% slower at 1024).
    if (A_rows <= 128 * (int64_t)n) {
        using SH = Shape<128, 256, 1, 4>;
        const int64_t tiles = (int64_t)n * ((N1 + SH::BM - 1) / SH::BM) *
                              ((N2 + SH::BN - 1) / SH::BN);
        const int64_t blocks = (tiles + 7) / 8 * 8;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((gemm_wgrad_kernel<SH, 32, 2>), dim3((unsigned)blocks), dim3(256), 0,
                           s, A, a_stride, B, b_stride, offsets, n, N1, N2, C, 2 * GM);
        return hipGetLastError();
    }
    using SH = Square<8>;
    const int64_t tiles = (int64_t)n * ((N1 + SH::BM - 1) / SH::BM) * ((N2 + SH::BN - 1) / SH::BN);
    const int64_t blocks = (tiles + 7) / 8 * 8;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_wgrad_kernel<SH, 64, 2>), dim3((unsigned)blocks), dim3(512), 0, s, A,
                       a_stride, B, b_stride, offsets, n, N1, N2, C, GM);
    return hipGetLastError();
}

template <int NWV, int EPI>
hipError_t launch_krow(const uint16_t* A, int64_t A_rows, const uint16_t* B1, const uint16_t* B3,
                       int b_split, const int32_t* offsets, int n, int Kdim, int N, void* C,
                       int splits, int cus, int* split_meta, hipStream_t s) {
    using SQ = Square<NWV>;
    const int64_t mslots = A_rows / SQ::BM + n;
    const int64_t ntn = (N + SQ::BN - 1) / SQ::BN;
    // with split_meta: whole-K tiles plus at most cus split ones (see the kernel)
    const int64_t blocks = split_meta ? (mslots * ntn + 7) / 8 * 8 + (cus + 7) / 8 * 8
                                      : (mslots * ntn * splits + 7) / 8 * 8;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (split_meta && cus < 1) return hipErrorInvalidValue;
    if (!split_meta) cus = 0;
    const int64_t stride = A_rows * (int64_t)N;
    // expert tails of at most 64 rows run as 64 x 512 tiles (a square tile
    // would leave three quarters of its MFMA rows idle); 128 x 512 tiles for
    // tails of 65..128 rows measured no faster here than square ones
    if (Kdim % BK)
        hipLaunchKernelGGL((gemm_bf16_kernel<false, true, NWV, EPI, true>),
                           dim3((unsigned)blocks), dim3(NWV * 64), 0, s, A, A_rows, nullptr, 1, B1,
                           B3, offsets, n, Kdim, N, C, 8, splits, stride, b_split, nullptr, 64,
                           cus, split_meta);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<false, false, NWV, EPI, true>),
                           dim3((unsigned)blocks), dim3(NWV * 64), 0, s, A, A_rows, nullptr, 1, B1,
                           B3, offsets, n, Kdim, N, C, 8, splits, stride, b_split, nullptr, 64,
                           cus, split_meta);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16_krow(const uint16_t* A, int64_t A_rows, const uint16_t* B1,
                                 const uint16_t* B3, int b_split, const int32_t* offsets, int n,
                                 int Kdim, int N, void* C, bool bf16_out, int splits,
                                 int cus, int* split_meta, hipStream_t s) {
    const int64_t lim = int64_t(1) << 31;
    if (N % 8 || Kdim % 8 || (B3 ? 2 * b_split != Kdim : b_split != Kdim) ||
        A_rows * Kdim * 2 >= lim || (int64_t)b_split * N * 2 >= lim || splits < 1 ||
        (bf16_out && (splits != 1 || split_meta)))
        return hipErrorInvalidValue;
    // eight waves of 128 x 64 (measured 10% faster than four of 128 x 128 here)
    if (bf16_out)
        return launch_krow<8, 2>(A, A_rows, B1, B3, b_split, offsets, n, Kdim, N, C, splits,
                                 cus, nullptr, s);
    return launch_krow<8, 0>(A, A_rows, B1, B3, b_split, offsets, n, Kdim, N, C, splits, cus,
                             split_meta, s);
}

}  // namespace moe
