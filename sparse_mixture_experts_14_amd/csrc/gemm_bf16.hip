// Grouped expert GEMMs on bf16 MFMA (gfx950 v_mfma_f32_32x32x16_bf16), fp32
// accumulation, LDS-staged double-buffered tiles.
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
// Both operands are K-contiguous ([out][in] weights), which is exactly the
// per-lane 8-element K run each MFMA operand wants; LDS rows are 64 bf16
// (8 chunks of 16 bytes) with the chunk index XOR-swizzled by (row & 7) so
// that the 16-byte LDS reads of 8 consecutive rows hit distinct banks.
//
// Tile order: the 1-D grid is first spread over the 8 XCDs (block b runs on
// XCD b % 8, so consecutive logical tiles are given to one XCD and share its
// L2), then walked in groups of GM row tiles: inside a group the row tile
// varies fastest, so a weight tile is fetched once for GM row tiles.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int BK = 64;              // K per LDS stage (8 chunks of 8 bf16)
constexpr int CHUNKS = BK / 8;

__device__ __forceinline__ int swz(int row, int chunk) {
    return row * BK + ((chunk ^ (row & 7)) << 3);
}

template <bool GATEUP, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM* WN* kWave) void gemm_bf16_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm, int K,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int32_t* __restrict__ offsets, int n, int Kdim, int N, void* __restrict__ Cout,
    int mslots, int GM) {
    constexpr int NTH = WM * WN * kWave;
    constexpr int WTM = BM / WM, WTN = BN / WN;   // wave tile (accumulator space)
    constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 MFMA tiles per wave
    constexpr int BNO = GATEUP ? BN / 2 : BN;     // output columns per tile
    constexpr int A_LD = BM * CHUNKS / NTH;       // 16-byte chunks per thread
    constexpr int B_LD = BN * CHUNKS / NTH;
    static_assert(A_LD * NTH == BM * CHUNKS && B_LD * NTH == BN * CHUNKS, "tile/threads");
    static_assert(!GATEUP || (TN % 2 == 0), "gate/up needs W1 and W3 tiles in pairs");

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

    // ---- loader setup: fixed rows per thread for the whole K loop ----------
    const uint16_t* a_ptr[A_LD];
    bool a_ok[A_LD];
    int a_lds[A_LD], a_ch[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int q = tid + i * NTH;
        const int r = q / CHUNKS, c = q % CHUNKS;
        a_ok[i] = r < rows;
        const int p = row0 + (a_ok[i] ? r : 0);
        const int64_t src = GATEUP ? (int64_t)(perm[p] / K) : (int64_t)p;
        a_ptr[i] = A + src * Kdim + c * 8;
        a_lds[i] = swz(r, c);
        a_ch[i] = c * 8;
    }
    const uint16_t* b_ptr[B_LD];
    bool b_ok[B_LD];
    int b_lds[B_LD], b_ch[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int q = tid + i * NTH;
        const int r = q / CHUNKS, c = q % CHUNKS;
        int col;
        const uint16_t* base;
        if (GATEUP) {
            const bool second = r >= BN / 2;
            col = n0 + (second ? r - BN / 2 : r);
            base = second ? B3 : B1;
        } else {
            col = n0 + r;
            base = B1;
        }
        b_ok[i] = col < N;
        b_ptr[i] = base + ((int64_t)e * N + (b_ok[i] ? col : 0)) * Kdim + c * 8;
        b_lds[i] = swz(r, c);
        b_ch[i] = c * 8;
    }

    uint4 ra[A_LD], rb[B_LD];
    auto load_global = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const bool ok = a_ok[i] && (k0 + a_ch[i] < Kdim);
            ra[i] = ok ? *reinterpret_cast<const uint4*>(a_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const bool ok = b_ok[i] && (k0 + b_ch[i] < Kdim);
            rb[i] = ok ? *reinterpret_cast<const uint4*>(b_ptr[i] + k0) : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_lds = [&](int st) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) *reinterpret_cast<uint4*>(&As[st][a_lds[i]]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_LD; ++i) *reinterpret_cast<uint4*>(&Bs[st][b_lds[i]]) = rb[i];
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
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load_global((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = kk * 2 + khalf;
            bf16x8_t av[TM], bv[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                av[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&As[cur][swz(a_row[i], ch)]));
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bv[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&Bs[cur][swz(b_row[j], ch)]));
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (kt + 1 < nk) store_lds(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------------
    // 32x32 accumulator layout: lane l, register r holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the MFMA tile.
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = wm * WTM + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
            if (row >= rows) continue;
            const int64_t orow = (int64_t)(row0 + row) * N;
            if (GATEUP) {
                uint16_t* H = static_cast<uint16_t*>(Cout);
#pragma unroll
                for (int j = 0; j < TN / 2; ++j) {
                    const int col = n0 + wn * (WTN / 2) + j * 32 + l32;
                    if (col < N) {
                        const float g = acc[i][j][r], u = acc[i][j + TN / 2][r];
                        H[orow + col] = f32_to_bf16_bits(silu(g) * u);
                    }
                }
            } else {
                float* O = static_cast<float*>(Cout);
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int col = n0 + wn * WTN + j * 32 + l32;
                    if (col < N) O[orow + col] = acc[i][j][r];
                }
            }
        }
    }
}

template <bool GATEUP, int BM, int BN, int WM, int WN>
hipError_t launch_tiled(const uint16_t* A, const int32_t* perm, int K, const uint16_t* B1,
                        const uint16_t* B3, const int32_t* offsets, int n, int64_t A_rows,
                        int Kdim, int N, void* C, int GM, hipStream_t s) {
    constexpr int BNO = GATEUP ? BN / 2 : BN;
    const int64_t mslots = A_rows / BM + n;
    const int64_t ntn = (N + BNO - 1) / BNO;
    int64_t blocks = mslots * ntn;
    blocks = (blocks + 7) / 8 * 8;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((gemm_bf16_kernel<GATEUP, BM, BN, WM, WN>), dim3((unsigned)blocks),
                       dim3(WM * WN * kWave), 0, s, A, perm, K, B1, B3, offsets, n, Kdim, N,
                       C, (int)mslots, GM);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_bf16_tiled(bool gateup, const uint16_t* A, const int32_t* perm, int K,
                                  const uint16_t* B1, const uint16_t* B3,
                                  const int32_t* offsets, int n, int64_t A_rows, int Kdim,
                                  int N, void* C, hipStream_t s) {
    const int GM = 8;
    if (gateup)
        return launch_tiled<true, 128, 128, 2, 2>(A, perm, K, B1, B3, offsets, n, A_rows,
                                                  Kdim, N, C, GM, s);
    return launch_tiled<false, 128, 128, 2, 2>(A, perm, K, B1, B3, offsets, n, A_rows, Kdim,
                                               N, C, GM, s);
}

}  // namespace moe
