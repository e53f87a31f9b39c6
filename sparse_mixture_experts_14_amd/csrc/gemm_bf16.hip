// Grouped expert GEMMs on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16), fp32
// accumulation, LDS-staged double-buffered tiles (many rows per expert).
//
// Expert FFN of "Mixtral of Experts" (xyznot digest, "Method" section and
// "Key terms"): SwiGLU_e(u) = W2_e (SiLU(W1_e u) (*) W3_e u).  The GeekNews
// summary ("Implementasi dan Efisiensi Inferensi") describes running all
// experts as one grouped product over an uneven number of tokens per expert;
// here the rows of every expert are contiguous after the permutation stage
// and a workgroup owns one BM x BN tile of one expert.
//
//   gate/up:  H[p][f] = bf16( SiLU(u_p . W1_e[f]) * (u_p . W3_e[f]) )
//             A rows are gathered, u_p = x[perm[p] / K]; the B tile holds
//             BN/2 rows of W1 and the same BN/2 rows of W3, so the SiLU*mul
//             epilogue finds both accumulators in the same lane.
//   down:     O[p][c] = H_p . W2_e[c]   (fp32 out)
//
// Tile shape.  256 x 256 accumulator tile, 4 waves, each 128 x 128 (4 x 4
// MFMA tiles of 32 x 32, 256 fp32 accumulators per lane): per 16-element K
// sub-step a wave reads 4 A and 4 B fragments from LDS for 16 MFMAs, and a
// workgroup fetches 64 KB from L2 per 64-element K step for 2 * 256^3 / 4 =
// 8.4 Mflop -- the arithmetic intensity that keeps the L2 ahead of the MFMAs.
// Both operands are K-contiguous ([out][in] weights), which is the per-lane
// 8-element K run each MFMA operand wants; LDS rows are 64 bf16 (8 chunks of
// 16 bytes) with the chunk index XOR-swizzled by (row >> 1) & 7, so the
// 16-byte LDS reads of 16 consecutive rows and the row-wise writes hit
// distinct banks.
//
// Pipeline.  Two LDS stages plus one register stage: the global loads of K
// step k+1 are issued before the MFMAs of step k and land in LDS after them.
// Loads go through buffer resources with 32-bit offsets and are
// unconditional (rows past the tile are clamped to a valid row, never
// stored); a K tail (rare shapes) zeroes the chunks past the end.
//
// Tile order: the 1-D grid is first spread over the 8 XCDs (block b runs on
// XCD b % 8, so consecutive logical tiles go to one XCD and share its L2),
// then walked in groups of GM row tiles: inside a group the row tile varies
// fastest, so a weight tile is fetched once for GM row tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int BK = 64;  // K per LDS stage (8 chunks of 8 bf16)
constexpr int CHUNKS = BK / 8;

// Two 128-byte rows span the 64 banks; XOR-ing the chunk with (row >> 1) & 7
// gives the 16 rows read by one 16-lane group 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * BK + ((chunk ^ ((row >> 1) & 7)) << 3);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                             0x00020000);
}

template <bool GATEUP, bool KTAIL, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN* kWave) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_kernel(const uint16_t* __restrict__ A, int64_t A_src_rows,
                      const int32_t* __restrict__ perm, int K, const uint16_t* __restrict__ B1,
                      const uint16_t* __restrict__ B3, const int32_t* __restrict__ offsets,
                      int n, int Kdim, int N, void* __restrict__ Cout, int mslots, int GM) {
    constexpr int NTH = WM * WN * kWave;
    constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile (accumulator space)
    constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 MFMA tiles per wave
    constexpr int BNO = GATEUP ? BN / 2 : BN;     // output columns per tile
    constexpr int A_LD = BM * CHUNKS / NTH;       // 16-byte chunks per thread
    constexpr int B_LD = BN * CHUNKS / NTH;
    constexpr int ROWS_PER_PASS = NTH / CHUNKS;   // rows a loader pass covers
    static_assert(A_LD * NTH == BM * CHUNKS && B_LD * NTH == BN * CHUNKS, "tile/threads");
    static_assert(!GATEUP || (TN % 2 == 0), "gate/up needs W1 and W3 tiles in pairs");
    static_assert(!GATEUP || ((BN / 2) % ROWS_PER_PASS == 0), "W1/W3 split on a pass boundary");

    __shared__ __attribute__((aligned(16))) uint16_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][BN * BK];

    // ---- tile coordinates -------------------------------------------------
    const int G = gridDim.x;  // a multiple of 8
    const int b = blockIdx.x;
    const int L = (b & 7) * (G >> 3) + (b >> 3);
    const int ntiles_n = (N + BNO - 1) / BNO;
    const int group = L / (GM * ntiles_n);
    const int first_m = group * GM;
    if (first_m >= mslots) return;
    const int gm = min(GM, mslots - first_m);
    const int local = L - group * GM * ntiles_n;
    const int mt = first_m + local % gm;
    const int nt = local / gm;
    if (nt >= ntiles_n) return;  // padding block of the last group
    int e, row0, rows;
    if (!locate_tile<BM>(offsets, n, mt, e, row0, rows)) return;
    const int n0 = nt * BNO;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int wm = wid % WM, wn = wid / WM;

    // ---- loader setup: rows r0 + ROWS_PER_PASS * i, one 16-byte chunk -------
    const int lr0 = tid / CHUNKS, lc = tid % CHUNKS;
    const uint32_t row_bytes = (uint32_t)Kdim * 2u;
    const __amdgpu_buffer_rsrc_t a_rs = rsrc(A, A_src_rows * (int64_t)Kdim * 2);
    const int64_t wbytes = (int64_t)N * Kdim * 2;
    const __amdgpu_buffer_rsrc_t b1_rs = rsrc(B1 + (int64_t)e * N * Kdim, wbytes);
    const __amdgpu_buffer_rsrc_t b3_rs = GATEUP ? rsrc(B3 + (int64_t)e * N * Kdim, wbytes) : b1_rs;
    uint32_t a_off[A_LD], b_off[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = lr0 + ROWS_PER_PASS * i;
        const int p = row0 + min(r, rows - 1);  // rows past the tile: a valid row, never stored
        const uint32_t src = GATEUP ? (uint32_t)(perm[p] / K) : (uint32_t)p;
        a_off[i] = src * row_bytes + (uint32_t)lc * 16u;
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = lr0 + ROWS_PER_PASS * i;
        const int col = n0 + (GATEUP && r >= BN / 2 ? r - BN / 2 : r);
        b_off[i] = (uint32_t)min(col, N - 1) * row_bytes + (uint32_t)lc * 16u;
    }

    auto load_global = [&](int k0, u32x4_t(&ra)[A_LD], u32x4_t(&rb)[B_LD]) {
        const bool ok = !KTAIL || (k0 + lc * 8 < Kdim);
        const uint32_t kb = (uint32_t)(ok ? k0 : 0) * 2u;  // clamped in range
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_off[i] + kb, 0, 0);
            ra[i] = ok ? v : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            // compile-time: passes i >= (BN/2) / ROWS_PER_PASS hold the W3 rows
            constexpr int W3_FROM = (BN / 2) / ROWS_PER_PASS;
            const bool second = GATEUP && i >= W3_FROM;
            const u32x4_t v =
                __builtin_amdgcn_raw_buffer_load_b128(second ? b3_rs : b1_rs, b_off[i] + kb, 0, 0);
            rb[i] = ok ? v : u32x4_t{0, 0, 0, 0};
        }
    };
    auto store_lds = [&](int st, const u32x4_t(&ra)[A_LD], const u32x4_t(&rb)[B_LD]) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            *reinterpret_cast<u32x4_t*>(&As[st][swz(lr0 + ROWS_PER_PASS * i, lc)]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            *reinterpret_cast<u32x4_t*>(&Bs[st][swz(lr0 + ROWS_PER_PASS * i, lc)]) = rb[i];
    };

    // ---- MFMA read coordinates ----------------------------------------------
    const int l32 = lane & 31, khalf = lane >> 5;
    int a_row[TM], b_row[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) a_row[i] = wm * WTM + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        if (GATEUP) {
            const int half = TN / 2;
            const int jj = j < half ? j : j - half;
            b_row[j] = (j < half ? 0 : BN / 2) + wn * (WTN / 2) + jj * 32 + l32;
        } else {
            b_row[j] = wn * WTN + j * 32 + l32;
        }
    }

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nk = (Kdim + BK - 1) / BK;
    auto read_frags = [&](int st, int kk, bf16x8_t(&av)[TM], bf16x8_t(&bv)[TN]) {
        const int ch = kk * 2 + khalf;
#pragma unroll
        for (int i = 0; i < TM; ++i)
            av[i] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&As[st][swz(a_row[i], ch)]));
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bv[j] = as_bf16x8(*reinterpret_cast<const u32x4_t*>(&Bs[st][swz(b_row[j], ch)]));
    };
    auto mfmas = [&](const bf16x8_t(&av)[TM], const bf16x8_t(&bv)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[j], av[i], acc[i][j], 0,
                                                                    0, 0);
    };
    // Scheduling hints (group masks: 0x008 MFMA, 0x020 global read, 0x100
    // LDS read, 0x200 LDS write): spread each sub-step's fragment reads for
    // the next sub-step between its MFMAs so LDS latency hides behind them.
    // The reads go out during the first MFMAs, leaving the rest of the
    // sub-step to cover their latency.
    auto interleave_reads = [&]() {
#pragma unroll
        for (int q = 0; q < TM + TN; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, TM * TN - (TM + TN), 0);
    };

    u32x4_t ra[A_LD], rb[B_LD];
    load_global(0, ra, rb);
    store_lds(0, ra, rb);
    __syncthreads();
    bf16x8_t a0[TM], b0[TN], a1[TM], b1[TN];
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        // next step's loads (the last iteration re-reads its own step:
        // harmless), issued first so they fly during this step's MFMAs
        load_global(min(kt + 1, nk - 1) * BK, ra, rb);
        read_frags(cur, 0, a0, b0);
        __builtin_amdgcn_sched_barrier(0);
        // sub-steps 0..2: read the next sub-step's fragments among the MFMAs
        read_frags(cur, 1, a1, b1);
        mfmas(a0, b0);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(cur, 2, a0, b0);
        mfmas(a1, b1);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
        read_frags(cur, 3, a1, b1);
        mfmas(a0, b0);
        interleave_reads();
        __builtin_amdgcn_sched_barrier(0);
        // sub-step 3, with the next stage's LDS writes among its MFMAs
        mfmas(a1, b1);
        store_lds(cur ^ 1, ra, rb);
#pragma unroll
        for (int q = 0; q < A_LD + B_LD; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------------
    // The MFMAs ran with the weights as the first operand, so the 32x32
    // accumulator of lane l, register r holds token row l%32 of the i-tile
    // and output column 8*(r/4) + 4*(l/32) + r%4 of the j-tile: a lane owns 4
    // contiguous columns per group of 4 registers.  Each wave stages one
    // i-tile at a time (32 rows x its WTN (down) or WTN/2 (gate/up) columns)
    // in its own LDS slot, padded by 16 bytes per row against bank
    // conflicts, and writes it back as whole 16-byte chunks of output rows.
    constexpr int OCOLS = GATEUP ? WTN / 2 : WTN;           // output columns per wave
    constexpr int ES = GATEUP ? 2 : 4;                       // output element bytes
    constexpr int RSTRIDE = OCOLS * ES + 16;                 // LDS row stride (bytes)
    constexpr int SLOT = 32 * RSTRIDE;                       // one wave's staging slot
    static_assert(WM * WN * SLOT <= 2 * (BM + BN) * BK * 2, "staging fits in the stage LDS");
    __syncthreads();  // every wave is done with the K-loop LDS
    uint8_t* slot = reinterpret_cast<uint8_t*>(&As[0][0]) + wid * SLOT;
    const int col_w = n0 + wn * OCOLS;  // first output column of this wave
    constexpr int CPR = OCOLS * ES / 16;      // 16-byte chunks per staged row
    constexpr int RPI = kWave / CPR;          // rows per store instruction
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        // stage rows wm*WTM + 32i .. +31
#pragma unroll
        for (int j = 0; j < (GATEUP ? TN / 2 : TN); ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int c = j * 32 + 8 * q + 4 * khalf;  // column within the wave
                uint8_t* dst = slot + l32 * RSTRIDE + c * ES;
                if (GATEUP) {
                    const f32x16_t& g = acc[i][j];
                    const f32x16_t& u = acc[i][j + TN / 2];
                    u32x2_t h;
                    h.x = pack_bf16x2(silu_bf16out(g[4 * q + 0]) * u[4 * q + 0],
                                      silu_bf16out(g[4 * q + 1]) * u[4 * q + 1]);
                    h.y = pack_bf16x2(silu_bf16out(g[4 * q + 2]) * u[4 * q + 2],
                                      silu_bf16out(g[4 * q + 3]) * u[4 * q + 3]);
                    *reinterpret_cast<u32x2_t*>(dst) = h;
                } else {
                    const f32x16_t& a = acc[i][j];
                    *reinterpret_cast<f32x4_t*>(dst) =
                        f32x4_t{a[4 * q + 0], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
                }
            }
        }
        // write back: lane -> (row, 16-byte chunk).  The slot is the wave's own
        // and LDS operations of one wave complete in order: no barrier needed.
#pragma unroll
        for (int rr = 0; rr < 32; rr += RPI) {
            const int r = rr + lane / CPR, ch = lane % CPR;
            const int row = wm * WTM + i * 32 + r;
            const int col = col_w + ch * (16 / ES);
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(slot + r * RSTRIDE + ch * 16);
            if (row < rows && col < N) {
                uint8_t* out = static_cast<uint8_t*>(Cout) +
                               ((int64_t)(row0 + row) * N + col) * ES;
                *reinterpret_cast<u32x4_t*>(out) = v;
            }
        }
    }
}

template <bool GATEUP, int BM, int BN, int WM, int WN>
hipError_t launch_tiled(const uint16_t* A, int64_t A_src_rows, const int32_t* perm, int K,
                        const uint16_t* B1, const uint16_t* B3, const int32_t* offsets, int n,
                        int64_t A_rows, int Kdim, int N, void* C, int GM, hipStream_t s) {
    constexpr int BNO = GATEUP ? BN / 2 : BN;
    const int64_t mslots = A_rows / BM + n;
    const int64_t ntn = (N + BNO - 1) / BNO;
    int64_t blocks = mslots * ntn;
    blocks = (blocks + 7) / 8 * 8;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    const bool ktail = Kdim % BK != 0;
    if (ktail)
        hipLaunchKernelGGL((gemm_bf16_kernel<GATEUP, true, BM, BN, WM, WN>), dim3((unsigned)blocks),
                           dim3(WM * WN * kWave), 0, s, A, A_src_rows, perm, K, B1, B3, offsets,
                           n, Kdim, N, C, (int)mslots, GM);
    else
        hipLaunchKernelGGL((gemm_bf16_kernel<GATEUP, false, BM, BN, WM, WN>),
                           dim3((unsigned)blocks), dim3(WM * WN * kWave), 0, s, A, A_src_rows,
                           perm, K, B1, B3, offsets, n, Kdim, N, C, (int)mslots, GM);
    return hipGetLastError();
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
                                  int64_t A_rows, int Kdim, int N, void* C, hipStream_t s) {
    if (!tiled_fits(A_src_rows, Kdim, N)) return hipErrorInvalidValue;
    const int GM = 4;
    if (gateup)
        return launch_tiled<true, 256, 256, 2, 2>(A, A_src_rows, perm, K, B1, B3, offsets, n,
                                                  A_rows, Kdim, N, C, GM, s);
    return launch_tiled<false, 256, 256, 2, 2>(A, A_src_rows, perm, K, B1, B3, offsets, n,
                                               A_rows, Kdim, N, C, GM, s);
}

}  // namespace moe
