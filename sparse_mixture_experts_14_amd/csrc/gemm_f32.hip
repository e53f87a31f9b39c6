// Grouped expert GEMMs for fp32 storage (small layers; plain FMA, no MFMA).
//
// Expert FFN of "Mixtral of Experts" (xyznot digest, "Method" section and
// "Key terms"): SwiGLU_e(u) = W2_e (SiLU(W1_e u) (*) W3_e u).
//   gate/up:  H[p][f] = SiLU(sum_k u_p[k] W1_e[f][k]) * sum_k u_p[k] W3_e[f][k]
//             for every row p of expert e, u_p = x[perm[p] / K]
//   down:     O[p][c] = sum_f H[p][f] W2_e[c][f]
// Rows of one expert are contiguous (offsets[e] .. offsets[e+1]); a workgroup
// owns a 64 x 64 output tile of one expert and exits when its tile slot is
// past the last tile, so the grid can be sized without knowing the routing.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int BM = 64, BN = 64, BK = 16;

template <bool GATEUP>
__global__ __launch_bounds__(256) void gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ perm, int K,
    const float* __restrict__ B1, const float* __restrict__ B3,
    const int32_t* __restrict__ offsets, int n, int Kdim, int N,
    float* __restrict__ C) {
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs1[BK][BN + 4];
    __shared__ float Bs3[GATEUP ? BK : 1][BN + 4];

    int e, row0, rows;
    if (!locate_tile<BM>(offsets, n, blockIdx.y, e, row0, rows)) return;
    const int n0 = blockIdx.x * BN;
    const int tid = threadIdx.x;
    const int tx = tid % 16, ty = tid / 16;

    // loader coordinates: one row (or weight row) and 4 consecutive k
    const int lr = tid / 4, lk = (tid % 4) * 4;
    const bool a_ok = lr < rows;
    const float* a_row;
    if (GATEUP) {
        const int p = row0 + (a_ok ? lr : 0);
        a_row = A + (int64_t)(perm[p] / K) * Kdim;
    } else {
        a_row = A + (int64_t)(row0 + (a_ok ? lr : 0)) * Kdim;
    }
    const bool b_ok = n0 + lr < N;
    const int64_t bofs = ((int64_t)e * N + (b_ok ? n0 + lr : 0)) * Kdim;
    const float* b1_row = B1 + bofs;
    const float* b3_row = GATEUP ? B3 + bofs : nullptr;

    float acc1[4][4] = {}, acc3[4][4] = {};
    for (int k0 = 0; k0 < Kdim; k0 += BK) {
        const int k = k0 + lk;
        const bool k_ok = k < Kdim;  // Kdim % 4 == 0: a float4 is all in or all out
        float4 av = make_float4(0.f, 0.f, 0.f, 0.f), bv1 = av, bv3 = av;
        if (a_ok && k_ok) av = *reinterpret_cast<const float4*>(a_row + k);
        if (b_ok && k_ok) {
            bv1 = *reinterpret_cast<const float4*>(b1_row + k);
            if (GATEUP) bv3 = *reinterpret_cast<const float4*>(b3_row + k);
        }
        As[lk + 0][lr] = av.x;
        As[lk + 1][lr] = av.y;
        As[lk + 2][lr] = av.z;
        As[lk + 3][lr] = av.w;
        Bs1[lk + 0][lr] = bv1.x;
        Bs1[lk + 1][lr] = bv1.y;
        Bs1[lk + 2][lr] = bv1.z;
        Bs1[lk + 3][lr] = bv1.w;
        if (GATEUP) {
            Bs3[lk + 0][lr] = bv3.x;
            Bs3[lk + 1][lr] = bv3.y;
            Bs3[lk + 2][lr] = bv3.z;
            Bs3[lk + 3][lr] = bv3.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b1[4], b3[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b1[j] = Bs1[kk][tx + 16 * j];
                if (GATEUP) b3[j] = Bs3[kk][tx + 16 * j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc1[i][j] = fmaf(a[i], b1[j], acc1[i][j]);
                    if (GATEUP) acc3[i][j] = fmaf(a[i], b3[j], acc3[i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = ty + 16 * i;
        if (r >= rows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = n0 + tx + 16 * j;
            if (c >= N) continue;
            const float v = GATEUP ? silu(acc1[i][j]) * acc3[i][j] : acc1[i][j];
            C[(int64_t)(row0 + r) * N + c] = v;
        }
    }
}

}  // namespace

hipError_t launch_gemm_f32(bool gateup, const float* A, const int32_t* perm, int K,
                           const float* B1, const float* B3, const int32_t* offsets, int n,
                           int64_t A_rows, int Kdim, int N, float* C, hipStream_t s) {
    const int64_t mslots = A_rows / BM + n;
    const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)mslots);
    if (gateup)
        hipLaunchKernelGGL((gemm_f32_kernel<true>), grid, dim3(256), 0, s, A, perm, K, B1,
                           B3, offsets, n, Kdim, N, C);
    else
        hipLaunchKernelGGL((gemm_f32_kernel<false>), grid, dim3(256), 0, s, A, perm, K, B1,
                           B3, offsets, n, Kdim, N, C);
    return hipGetLastError();
}

}  // namespace moe
