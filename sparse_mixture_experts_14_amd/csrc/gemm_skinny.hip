// Grouped expert GEMMs for few rows per expert (decode): a weight stream.
//
// Same products as the tiled kernels (xyznot digest of "Mixtral of Experts",
// "Method" section: SwiGLU_e(u) = W2_e (SiLU(W1_e u) (*) W3_e u)), but with a
// handful of tokens per expert the layer is bound by reading the touched
// experts' weights from HBM once; everything here serves that stream.
//
// * Work split.  An item is a 16-row slice of weights (16 output columns)
//   over one K range: gate/up -- rows f..f+15 of W1_e, then the same rows of
//   W3_e (the SiLU*mul epilogue needs both); down -- rows c..c+15 of W2_e over
//   one of S K-splits (partial sums go to O + s * A_rows * N and the combine
//   stage adds the S splits in order).  Items of experts with no rows do not
//   exist (an expert whose gate is 0 is never read).  The grid is
//   persistent: one workgroup of W (7 or 8) waves per CU (its LDS keeps a
//   second one off the CU) and wave g takes items g, g + NW, ...; the host
//   picks W and S so that items divide evenly over the waves, preferring
//   fewer splits (longer runs along each weight row).
// * Weight loads.  HBM streams best in long runs per row, so every load
//   instruction reads 1 KB of one weight row (lane l: elements 8l..8l+7 of a
//   512-element step), non-temporal, into registers; the wave then writes the
//   16 rows x 512 elements to its own 16 KB LDS tile and reads MFMA A
//   fragments (v_mfma_f32_16x16x32_bf16, weights as the 16-row operand) back
//   out of it.  The LDS chunk index is XOR-swizzled by the row, so both the
//   row-wise writes and the fragment reads hit distinct banks.  Token rows
//   (the B operand, <= 16 per pass, padding lanes read nothing) come from L2
//   straight in fragment layout.
// * K map.  Fragment c of a step takes chunk 4c + g (g = lane/16) for both
//   operands, so weights and tokens agree on k and the products are unchanged.
// * Buffer instructions.  Loads and stores go through buffer resources (one
//   per expert matrix, per activation array, per output), so offsets are
//   32-bit and a store at an out-of-range offset is dropped by the hardware.
//   The epilogue store is issued on every step with no branch (only its
//   offset decides whether it lands), which keeps the instruction stream
//   fixed so that the compiler counts outstanding loads exactly.
// * Tables.  At start the workgroup copies the touched experts' row ranges
//   and the activation row of every expert-ordered row into LDS; the step
//   loop reads only LDS besides the streams, so no table lookup drains the
//   loads in flight.
// * Pipeline, per step s: MFMAs of step s from LDS; write step s+1's rows
//   (loaded one step earlier) into LDS; load step s+1's token fragments;
//   load step s+2's weight rows; store.  One step of weights stays in flight
//   per wave while it computes.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {


constexpr int KSTEP = 512;         // k per step: 64 lanes x 8 elements of one row
constexpr int MAX_ROWS = 2048;     // row-source table in LDS (the host keeps A <= this)
constexpr int TILE_U4 = 16 * 64;   // one wave's LDS tile: 16 rows x 64 chunks of 16 bytes

struct Shape {
    int Kdim, N, nsplit, ksplit, tiles, groups, steps, total_items, NW;
};

struct Tables {  // per-workgroup copies in LDS, so the step loop never waits on memory
    int t_expert[64], t_start[64], t_end[64];
    int src[MAX_ROWS];  // activation row feeding expert-ordered row p
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Everything an item implies (recomputed only when the cursor changes item).
struct Where {
    int expert, end, col0, split, kbeg, kend;
};

// A cursor over the wave's flat step sequence: items gw, gw + NW, ...; each
// item in 16-row passes; each pass streams its weight slices (tiles) one
// after the other, each in `steps` K steps.  Plain scalars only.
struct Cursor {
    int item, row0, tile, step;
    bool valid;
    Where w;
};

__device__ __forceinline__ Where where(const Tables& tb, const Shape& S, int item) {
    Where w;
    const int per_expert = S.groups * S.nsplit;
    const int ti = item / per_expert;
    const int rem = item - ti * per_expert;
    const int grp = rem / S.nsplit;
    w.split = rem - grp * S.nsplit;
    w.expert = uni(tb.t_expert[ti]);
    w.end = uni(tb.t_end[ti]);
    w.col0 = grp * 16;
    w.kbeg = w.split * S.ksplit;
    w.kend = min(S.Kdim, w.kbeg + S.ksplit);
    return w;
}

__device__ __forceinline__ Cursor start_cursor(const Tables& tb, const Shape& S, int item) {
    Cursor c;
    c.item = item;
    c.row0 = uni(tb.t_start[item / (S.groups * S.nsplit)]);
    c.tile = 0;
    c.step = 0;
    c.valid = true;
    c.w = where(tb, S, item);
    return c;
}

// One step on: next K step, next tile, next 16-row pass, or the wave's next
// item.  Past the end the cursor stays on its last step with valid = false.
__device__ __forceinline__ void step_on(const Tables& tb, const Shape& S, Cursor& c) {
    if (!c.valid) return;
    if (++c.step < S.steps) return;
    c.step = 0;
    if (c.tile + 1 < S.tiles) {
        ++c.tile;
    } else if (c.row0 + 16 < c.w.end) {
        c.tile = 0;
        c.row0 += 16;
    } else if (c.item + S.NW < S.total_items) {
        c = start_cursor(tb, S, c.item + S.NW);
    } else {
        c.valid = false;
        c.step = S.steps - 1;
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr uint32_t OOB = 0x80000000u;  // a buffer offset past every range: load 0, store dropped
constexpr int NT_AUX = 2;              // non-temporal cache policy

// LDS position (in 16-byte units) of chunk q of tile row r.
__device__ __forceinline__ int lds_pos(int r, int q) { return r * 64 + (q ^ r); }

// SAVE (gate/up only): also store the pre-activation rows AB[p] = [a | b]
// (bf16, 2 N columns); a NULL Cout then skips H (its stores fall out of a
// zero-size range).
template <bool GATEUP, bool KTAIL, int WAVES, bool SAVE = false>
__global__ __launch_bounds__(WAVES* kWave) void gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm, int K,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int32_t* __restrict__ offsets, int n, int Kdim, int N, void* __restrict__ Cout,
    int64_t A_rows, int64_t A_src_rows, int nsplit, int ksplit,
    uint16_t* __restrict__ AB = nullptr) {
    __shared__ Tables tb;
    __shared__ int s_touched;
    __shared__ u32x4_t tiles_lds[WAVES * TILE_U4];
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    // the wave index is uniform across the wave: keep the cursors in SGPRs
    const int gw = uni(blockIdx.x * WAVES + wv);
    const int j16 = lane & 15, g = lane >> 4;
    u32x4_t* tile = tiles_lds + wv * TILE_U4;

    if (threadIdx.x == 0) {
        int t = 0;
        for (int e = 0; e < n; ++e) {
            const int s0 = offsets[e], s1 = offsets[e + 1];
            if (s1 > s0) {
                tb.t_expert[t] = e;
                tb.t_start[t] = s0;
                tb.t_end[t] = s1;
                ++t;
            }
        }
        s_touched = t;
    }
    for (int p = threadIdx.x; p < A_rows; p += blockDim.x)
        tb.src[p] = GATEUP ? perm[p] / K : p;
    __syncthreads();

    Shape S;
    S.Kdim = Kdim;
    S.N = N;
    S.nsplit = nsplit;
    S.ksplit = ksplit;
    S.tiles = GATEUP ? 2 : 1;
    S.groups = (N + 15) / 16;
    S.steps = (ksplit + KSTEP - 1) / KSTEP;
    S.total_items = uni(s_touched) * S.groups * nsplit;
    S.NW = gridDim.x * WAVES;
    if (gw >= S.total_items) return;

    const uint32_t row_bytes = (uint32_t)Kdim * 2u;
    const __amdgpu_buffer_rsrc_t a_rs = rsrc(A, (uint32_t)(A_src_rows * Kdim * 2));
    const uint32_t w_bytes = (uint32_t)N * row_bytes;  // one expert's matrix
    const uint32_t out_bytes = (uint32_t)((GATEUP ? 2 : 4) * (int64_t)nsplit * A_rows * N);
    const __amdgpu_buffer_rsrc_t o_rs = rsrc(Cout, Cout ? out_bytes : 0u);
    const __amdgpu_buffer_rsrc_t ab_rs =
        rsrc(AB, SAVE ? (uint32_t)(2 * A_rows * (int64_t)N * 2) : 0u);

    // ---- weight rows: instruction i loads 1 KB of tile row i ------------------
    Cursor bc = start_cursor(tb, S, gw);  // position of the rows being loaded
    u32x4_t wq[16];
    auto load_rows = [&]() {
        const Where& w = bc.w;
        const int k = w.kbeg + bc.step * KSTEP + lane * 8;
        const bool ok = !KTAIL || k < w.kend;
        const int kc = ok ? k : w.kend - 8;  // clamped, in range
        const uint16_t* base = (GATEUP && bc.tile == 1) ? B3 : B1;
        const __amdgpu_buffer_rsrc_t w_rs = rsrc(base + (int64_t)w.expert * N * Kdim, w_bytes);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int col = min(w.col0 + i, N - 1);  // columns past N are never stored
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(
                w_rs, (uint32_t)col * row_bytes + (uint32_t)kc * 2u, 0, NT_AUX);
            wq[i] = ok ? v : u32x4_t{0, 0, 0, 0};
        }
        step_on(tb, S, bc);
    };
    auto rows_to_lds = [&]() {
#pragma unroll
        for (int i = 0; i < 16; ++i) tile[lds_pos(i, lane)] = wq[i];
    };

    // ---- token fragments: fragment c, lane (token j16, group g) -> chunk 4c+g --
    Cursor ac = start_cursor(tb, S, gw);  // position of the token fragments loaded
    u32x4_t tq[16];
    auto load_tokens = [&]() {
        const Where& w = ac.w;
        const int k0 = w.kbeg + ac.step * KSTEP;
        const int p = min(ac.row0 + j16, w.end - 1);
        // padding token lanes (past the expert's rows) read nothing: out of range -> 0
        const uint32_t a_row = ac.row0 + j16 < w.end ? (uint32_t)tb.src[p] * row_bytes : OOB;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int k = k0 + (4 * c + g) * 8;
            const bool ok = !KTAIL || k < w.kend;
            const int kc = ok ? k : w.kend - 8;
            const u32x4_t v =
                __builtin_amdgcn_raw_buffer_load_b128(a_rs, a_row + (uint32_t)kc * 2u, 0, 0);
            tq[c] = ok ? v : u32x4_t{0, 0, 0, 0};
        }
        step_on(tb, S, ac);
    };

    // ---- compute -----------------------------------------------------------------
    // Weights are the MFMA A operand, tokens the B operand: the 16x16
    // accumulator of lane l, register r is output column 4*(l/16) + r of the
    // slice for token row l%16, so a lane owns 4 contiguous output columns.
    // gate/up: the W1 tile streams first; its sums move to `prev` while the
    // W3 tile accumulates.  Four independent accumulation chains.
    Cursor cc = start_cursor(tb, S, gw);
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    f32x4_t acc4[4] = {z, z, z, z}, prev = z;
    auto mfma = [&]() {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const u32x4_t wf = tile[lds_pos(j16, 4 * c + g)];
            acc4[c & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wf), as_bf16x8(tq[c]),
                                                                  acc4[c & 3], 0, 0, 0);
        }
    };
    auto finish = [&]() {
        const Where& w = cc.w;
        const f32x4_t acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
        const bool tile_end = cc.valid && cc.step == S.steps - 1;
        const bool last = tile_end && cc.tile == S.tiles - 1;
        const int row = cc.row0 + j16;
        const int col = w.col0 + 4 * g;
        const bool ok = last && row < w.end && col < N;
        if (GATEUP) {
            u32x2_t h;
            h.x = pack_bf16x2(silu_bf16out(prev[0]) * acc[0], silu_bf16out(prev[1]) * acc[1]);
            h.y = pack_bf16x2(silu_bf16out(prev[2]) * acc[2], silu_bf16out(prev[3]) * acc[3]);
            const uint32_t off = ok ? (uint32_t)(((int64_t)row * N + col) * 2) : OOB;
            __builtin_amdgcn_raw_buffer_store_b64(h, o_rs, off, 0, 0);
            if (SAVE) {
                u32x2_t va, vb;
                va.x = pack_bf16x2(prev[0], prev[1]);
                va.y = pack_bf16x2(prev[2], prev[3]);
                vb.x = pack_bf16x2(acc[0], acc[1]);
                vb.y = pack_bf16x2(acc[2], acc[3]);
                const uint32_t oa = ok ? (uint32_t)(((int64_t)row * 2 * N + col) * 2) : OOB;
                const uint32_t ob = ok ? oa + (uint32_t)N * 2u : OOB;
                __builtin_amdgcn_raw_buffer_store_b64(va, ab_rs, oa, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b64(vb, ab_rs, ob, 0, 0);
            }
        } else {
            const int64_t o = ((int64_t)w.split * A_rows + row) * N + col;
            const uint32_t off = ok ? (uint32_t)(o * 4) : OOB;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, acc), o_rs, off, 0,
                                                   0);
        }
        prev = tile_end ? acc : prev;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc4[i] = tile_end ? z : acc4[i];
        step_on(tb, S, cc);
    };

    // Steps in this wave's sequence (extra steps past the end repeat the last
    // loads and store nothing: the cursors are no longer valid).
    int nsteps = 0;
    for (int it = gw; it < S.total_items; it += S.NW) {
        const int ti = it / (S.groups * S.nsplit);
        const int rows = uni(tb.t_end[ti]) - uni(tb.t_start[ti]);
        nsteps += (rows + 15) / 16 * S.tiles * S.steps;
    }
    load_rows();      // step 0 rows
    load_tokens();    // step 0 tokens
    rows_to_lds();    // (waits for step 0 rows)
    load_rows();      // step 1 rows in flight
    for (int q = 0; q < nsteps; ++q) {  // one back edge, no early exit
        mfma();         // step q (LDS + token fragments)
        rows_to_lds();  // step q+1 rows, loaded during step q
        load_tokens();  // step q+1 tokens (issued before the rows of q+2)
        load_rows();    // step q+2 rows stay in flight through step q+1
        finish();       // epilogue store of step q (fixed instruction stream)
    }
}

}  // namespace

bool skinny_fits(int64_t A_src_rows, int64_t A_rows, int64_t Kdim, int64_t N, int splits) {
    // (the saved [a | b] rows of the gate/up are 2 A_rows N bf16 = the fp32
    // partial sums of one split, covered below)
    // every buffer range must stay below 2^31 bytes (32-bit buffer offsets)
    const int64_t lim = int64_t(1) << 31;
    return A_rows <= MAX_ROWS && A_src_rows * Kdim * 2 < lim && N * Kdim * 2 < lim &&
           (int64_t)splits * A_rows * N * 4 < lim;
}

hipError_t launch_gemm_bf16_skinny(bool gateup, const uint16_t* A, int64_t A_src_rows,
                                   const int32_t* perm, int K, const uint16_t* B1,
                                   const uint16_t* B3, const int32_t* offsets, int n,
                                   int64_t A_rows, int Kdim, int N, void* C, int splits,
                                   int waves, int cus, hipStream_t s, uint16_t* AB) {
    const int ksplit = (((Kdim + splits - 1) / splits) + 7) / 8 * 8;
    const int nsplit = (Kdim + ksplit - 1) / ksplit;
    if (!skinny_fits(A_src_rows, A_rows, Kdim, N, nsplit)) return hipErrorInvalidValue;
    if (waves != 7 && waves != 8) return hipErrorInvalidValue;
    if (AB && !gateup) return hipErrorInvalidValue;
    const dim3 grid((unsigned)cus), block((unsigned)(waves * kWave));
    // every K split a whole number of steps: no partial chunks to zero
    const bool ktail = (ksplit % KSTEP) != 0 || (Kdim % ksplit) != 0;
#define MOE_SKINNY(GU, KT, W, SV)                                                         \
    hipLaunchKernelGGL((gemm_skinny_kernel<GU, KT, W, SV>), grid, block, 0, s, A, perm, K, \
                       B1, B3, offsets, n, Kdim, N, C, A_rows, A_src_rows, nsplit, ksplit, AB)
#define MOE_SKINNY_W(GU, KT, SV) \
    if (waves == 7) MOE_SKINNY(GU, KT, 7, SV); else MOE_SKINNY(GU, KT, 8, SV)
#define MOE_SKINNY_WS(GU, KT) \
    if (AB) { MOE_SKINNY_W(GU, KT, true); } else { MOE_SKINNY_W(GU, KT, false); }
    if (gateup) {
        if (ktail) { MOE_SKINNY_WS(true, true); }
        else { MOE_SKINNY_WS(true, false); }
    } else {
        if (ktail) { MOE_SKINNY_W(false, true, false); }
        else { MOE_SKINNY_W(false, false, false); }
    }
#undef MOE_SKINNY_WS
#undef MOE_SKINNY_W
#undef MOE_SKINNY
    return hipGetLastError();
}

int skinny_splits_used(int Kdim, int splits) {
    const int ksplit = (((Kdim + splits - 1) / splits) + 7) / 8 * 8;
    return (Kdim + ksplit - 1) / ksplit;
}

}  // namespace moe
