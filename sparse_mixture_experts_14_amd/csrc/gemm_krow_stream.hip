// Grouped products with K-row weights for few rows per expert (the backward
// pass at decode sizes): a weight stream.
//
//   C[s][p][c] = sum over k in K split s of A[p][k] W_e[k][c]
//
// for the rows p of each expert e.  W_e is read along its rows (K rows of N
// contiguous columns): W_e[k] = B1_e[k] for k < b_split, else
// B3_e[k - b_split], with B_e = B + e b_split N -- the r = W2_e^T dy product
// (W2_e [d][d_ff]) and the dx = [W1_e ; W3_e]^T [da | db] product of the
// backward of "Mixtral of Experts" (xyznot digest, "Method": the SwiGLU
// experts).  With a handful of rows per expert the work is reading the
// weights once, so everything serves that stream:
// * An item is one touched expert x 512 columns x one K split; lane l owns
//   columns 8 l .. 8 l + 7 of the item and every weight load is 16 bytes of
//   one row, so a wave reads 1 KB runs.  The persistent grid (one workgroup
//   of WAVES waves per CU) deals items round robin to the waves; the host
//   picks WAVES and the splits so that they divide evenly.
// * A chunk is 16 K rows: its 16 loads are issued together (non-temporal),
//   then the expert's A values for those 16 k (bf16 pairs, up to 16 rows) go
//   to the wave's own LDS, then the wave computes.  Other waves' loads are in
//   flight meanwhile.
// * Rows k and k + 1 of a column are packed into one bf16 pair, so one
//   v_dot2_f32_bf16 adds both products: acc += W[k] A[k] + W[k+1] A[k+1].
//   Passes of 16 expert rows; rows past the expert's skip their dot products
//   (a wave-uniform branch).
// * Rows past the K split load zeros (out-of-range offset) and their A
//   values are zero; columns past N are clamped and not stored.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int CB = 512;   // columns per item: 64 lanes x 8
constexpr int PMAX = 16;  // expert rows per pass
constexpr int KC = 16;    // K rows per chunk
constexpr uint32_t OOB_K = 0x80000000u;  // buffer offset past every range: loads 0


__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_k(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                             0x00020000);
}

__device__ __forceinline__ int uni_k(int v) { return __builtin_amdgcn_readfirstlane(v); }

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void krow_stream_kernel(
    const uint16_t* __restrict__ A, int64_t A_rows, int Kdim, const uint16_t* __restrict__ B1,
    const uint16_t* __restrict__ B3, int b_split, const int32_t* __restrict__ offsets, int n,
    int N, float* __restrict__ C, int nsplit, int ksplit) {
    __shared__ int t_e[64], t_s[64], t_end[64];
    __shared__ int s_touched;
    __shared__ uint32_t a_lds[WAVES][PMAX][KC / 2];  // bf16 pairs (k, k + 1) per row
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int gw = uni_k(blockIdx.x * WAVES + wv);
    if (threadIdx.x == 0) {
        int t = 0;
        for (int e = 0; e < n; ++e) {
            const int s0 = offsets[e], s1 = offsets[e + 1];
            if (s1 > s0) {
                t_e[t] = e;
                t_s[t] = s0;
                t_end[t] = s1;
                ++t;
            }
        }
        s_touched = t;
    }
    __syncthreads();
    const int ncb = (N + CB - 1) / CB;
    const int total = uni_k(s_touched) * ncb * nsplit;
    const int NW = gridDim.x * WAVES;
    const __amdgpu_buffer_rsrc_t a_rs = rsrc_k(A, A_rows * (int64_t)Kdim * 2);
    const int64_t wbytes1 = (int64_t)b_split * N * 2;                 // one B1_e
    const int64_t wbytes3 = B3 ? (int64_t)(Kdim - b_split) * N * 2 : 0;  // one B3_e rows used
    uint32_t(*al)[KC / 2] = a_lds[wv];

    for (int it = gw; it < total; it += NW) {
        const int ti = it / (ncb * nsplit);
        const int rem = it - ti * (ncb * nsplit);
        const int cb = rem / nsplit, s = rem - cb * nsplit;
        const int e = uni_k(t_e[ti]), start = uni_k(t_s[ti]), end = uni_k(t_end[ti]);
        const int k0 = s * ksplit, k1 = min(Kdim, k0 + ksplit);
        const int col = cb * CB + lane * 8;
        const int colc = min(col, N - 8);  // columns past N: a valid column, never stored
        const uint16_t* w1_base = B1 + (int64_t)e * b_split * N;
        const uint16_t* w3_base = B3 ? B3 + (int64_t)e * b_split * N : w1_base;
        for (int row0 = start; row0 < end; row0 += PMAX) {
            const int P = min(PMAX, end - row0);
            float acc[PMAX][8];
#pragma unroll
            for (int p = 0; p < PMAX; ++p)
#pragma unroll
                for (int c = 0; c < 8; ++c) acc[p][c] = 0.0f;
            for (int kc = k0; kc < k1; kc += KC) {
                // A values (issued first, so that staging them waits for this
                // load only): lane l -> expert row l / 4, k = kc + 4 (l % 4) .. + 3
                const int pr = lane >> 2, kq = kc + (lane & 3) * 4;
                u32x2_t av;
                {
                    uint32_t off = OOB_K;
                    if (pr < P && kq < k1)
                        off = (uint32_t)((int64_t)(row0 + pr) * Kdim + kq) * 2u;
                    av = __builtin_bit_cast(
                        u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(a_rs, off, 0, 0));
                }
                // weight rows kc .. kc + 15 of this lane's 8 columns
                u32x4_t w[KC];
#pragma unroll
                for (int r = 0; r < KC; ++r) {
                    const int k = kc + r;
                    const bool in3 = B3 && k >= b_split;
                    const uint32_t off =
                        k < k1 ? (uint32_t)(in3 ? k - b_split : k) * (uint32_t)N * 2u +
                                     (uint32_t)colc * 2u
                               : OOB_K;
                    // (a descriptor built from a selected base and size: a select
                    // between descriptor values is lowered through scratch memory)
                    w[r] = __builtin_amdgcn_raw_buffer_load_b128(
                        rsrc_k(in3 ? w3_base : w1_base, in3 ? wbytes3 : wbytes1), off, 0, 2);
                }
                // a K tail inside these 4 k: zero the values past k1
                if (kq + 1 >= k1) av.x &= 0x0000ffffu;
                if (kq + 2 >= k1) av.y = 0u;
                if (kq + 3 >= k1) av.y &= 0x0000ffffu;
                al[pr][(lane & 3) * 2] = av.x;
                al[pr][(lane & 3) * 2 + 1] = av.y;
                // the wave reads what its other lanes wrote: LDS operations of a
                // wave complete in order; keep the compiler from reordering
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_wave_barrier();
#pragma unroll
                for (int r = 0; r < KC; r += 2) {
                    // pairs (W[k][c], W[k+1][c]) for the 8 columns
                    uint32_t wp[8];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint32_t lo = w[r][q], hi = w[r + 1][q];
                        wp[2 * q] = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
                        wp[2 * q + 1] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
                    }
#pragma unroll
                    for (int p = 0; p < PMAX; ++p) {
                        if (p < P) {
                            const bf16x2_t ap = __builtin_bit_cast(bf16x2_t, al[p][r / 2]);
#pragma unroll
                            for (int c = 0; c < 8; ++c)
                                acc[p][c] = __builtin_amdgcn_fdot2_f32_bf16(
                                    __builtin_bit_cast(bf16x2_t, wp[c]), ap, acc[p][c], false);
                        }
                    }
                }
                __asm__ __volatile__("" ::: "memory");
                __builtin_amdgcn_wave_barrier();
            }
            if (col < N) {
#pragma unroll
                for (int p = 0; p < PMAX; ++p) {
                    if (p < P) {
                        float* o = C + ((int64_t)s * A_rows + row0 + p) * N + col;
                        *reinterpret_cast<f32x4_t*>(o) =
                            f32x4_t{acc[p][0], acc[p][1], acc[p][2], acc[p][3]};
                        *reinterpret_cast<f32x4_t*>(o + 4) =
                            f32x4_t{acc[p][4], acc[p][5], acc[p][6], acc[p][7]};
                    }
                }
            }
        }
    }
}

}  // namespace

int krow_stream_splits_used(int Kdim, int splits) {
    const int ksplit = ((Kdim + splits - 1) / splits + KC - 1) / KC * KC;
    return (Kdim + ksplit - 1) / ksplit;
}

hipError_t launch_gemm_bf16_krow_stream(const uint16_t* A, int64_t A_rows, const uint16_t* B1,
                                        const uint16_t* B3, int b_split,
                                        const int32_t* offsets, int n, int Kdim, int N,
                                        float* C, int splits, int waves, int cus,
                                        hipStream_t s) {
    const int64_t lim = int64_t(1) << 31;
    if (N % 8 || Kdim % 8 || (B3 ? 2 * b_split != Kdim : b_split != Kdim) || splits < 1 ||
        A_rows * Kdim * 2 >= lim || (int64_t)b_split * N * 2 >= lim || n > 64)
        return hipErrorInvalidValue;
    const int ksplit = ((Kdim + splits - 1) / splits + KC - 1) / KC * KC;
    const int nsplit = (Kdim + ksplit - 1) / ksplit;
    const dim3 grid((unsigned)cus);
    if (waves == 8)
        hipLaunchKernelGGL((krow_stream_kernel<8>), grid, dim3(512), 0, s, A, A_rows, Kdim, B1,
                           B3, b_split, offsets, n, N, C, nsplit, ksplit);
    else if (waves == 7)
        hipLaunchKernelGGL((krow_stream_kernel<7>), grid, dim3(448), 0, s, A, A_rows, Kdim, B1,
                           B3, b_split, offsets, n, N, C, nsplit, ksplit);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace moe
