// Elementwise, reduction and layout kernels of the backward pass (bf16 data,
// fp32 arithmetic).  The grouped products themselves run on the MFMA kernels
// of gemm_bf16.hip.
//
// Gradients of L = sum_t dy_t . y_t through the layer of "Mixtral of
// Experts" (xyznot digest, "Method" section: gate equation and output
// equation; "Key terms": SwiGLU experts).  For token t, kept experts s_j with
// gates g_j, e = s_j, a = W1_e x, b = W3_e x, h = SiLU(a) b, o = W2_e h:
//   dg_j = dy . o,  do = g_j dy,  dh = W2_e^T do,
//   da = dh b SiLU'(a),  db = dh SiLU(a),
//   dx = sum_j (W1_e^T da + W3_e^T db) + W_g dl,
//   dl_{s_j} = g_j (dg_j - sum_k g_k dg_k)  (softmax over the kept logits;
//   the other logits get 0: TopK is constant away from ties),
//   dW_g = sum_t x_t dl_t^T.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float bf(uint16_t v) { return bf16_bits_to_f32(v); }

// H[p][f] = bf16(SiLU(a) * b) from rows AB[p] = [a | b] (8 elements per thread).
__global__ __launch_bounds__(256) void bwd_h_kernel(const uint16_t* __restrict__ AB, int64_t A,
                                                    int dff, uint16_t* __restrict__ H) {
    const int64_t chunks = A * (dff / 8);
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < chunks; q += (int64_t)gridDim.x * 256) {
        const int64_t p = q / (dff / 8);
        const int c = (int)(q % (dff / 8)) * 8;
        const uint4 av = *reinterpret_cast<const uint4*>(AB + p * 2 * dff + c);
        const uint4 bv = *reinterpret_cast<const uint4*>(AB + p * 2 * dff + dff + c);
        float a[8], b[8], h[8];
        unpack_bf16x8(av, a);
        unpack_bf16x8(bv, b);
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = silu(a[i]) * b[i];
        uint4 o;
        o.x = pack_bf16x2(h[0], h[1]);
        o.y = pack_bf16x2(h[2], h[3]);
        o.z = pack_bf16x2(h[4], h[5]);
        o.w = pack_bf16x2(h[6], h[7]);
        *reinterpret_cast<uint4*>(H + p * dff + c) = o;
    }
}

// Per assignment row p (expert order), a = perm[p], t = a / K:
// dg[a] = dy_t . O[p] (fixed-order block sum) and DO[p] = bf16(gate[a] dy_t).
__global__ __launch_bounds__(256) void bwd_gates_kernel(
    const uint16_t* __restrict__ dy, const float* __restrict__ O,
    const int32_t* __restrict__ perm, const float* __restrict__ gate, int K, int d,
    float* __restrict__ dg, uint16_t* __restrict__ DO) {
    __shared__ float part[4];
    const int64_t p = blockIdx.x;
    const int a = perm[p];
    const int64_t t = a / K;
    const float g = gate[a];
    float s = 0.0f;
    for (int c = threadIdx.x * 4; c < d; c += 1024) {
        const uint2 yv = *reinterpret_cast<const uint2*>(dy + t * d + c);
        const float y0 = __uint_as_float(yv.x << 16), y1 = __uint_as_float(yv.x & 0xffff0000u);
        const float y2 = __uint_as_float(yv.y << 16), y3 = __uint_as_float(yv.y & 0xffff0000u);
        const float4 o = *reinterpret_cast<const float4*>(O + p * d + c);
        s = fmaf(y0, o.x, s);
        s = fmaf(y1, o.y, s);
        s = fmaf(y2, o.z, s);
        s = fmaf(y3, o.w, s);
        uint2 w;
        w.x = pack_bf16x2(g * y0, g * y1);
        w.y = pack_bf16x2(g * y2, g * y3);
        *reinterpret_cast<uint2*>(DO + p * d + c) = w;
    }
    s = wave_sum(s);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = s;
    __syncthreads();
    if (threadIdx.x == 0) dg[a] = (part[0] + part[1]) + (part[2] + part[3]);
}

// SwiGLU backward: DADB[p] = [da | db] (bf16) from AB[p] = [a | b] and the
// fp32 upstream gradient DH[p] of h = SiLU(a) b.
__global__ __launch_bounds__(256) void bwd_swiglu_kernel(const uint16_t* __restrict__ AB,
                                                         const float* __restrict__ DH,
                                                         int64_t A, int dff,
                                                         uint16_t* __restrict__ DADB) {
    const int64_t chunks = A * (dff / 4);
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < chunks; q += (int64_t)gridDim.x * 256) {
        const int64_t p = q / (dff / 4);
        const int c = (int)(q % (dff / 4)) * 4;
        const uint2 av = *reinterpret_cast<const uint2*>(AB + p * 2 * dff + c);
        const uint2 bv = *reinterpret_cast<const uint2*>(AB + p * 2 * dff + dff + c);
        const float4 dh = *reinterpret_cast<const float4*>(DH + p * dff + c);
        const float a[4] = {__uint_as_float(av.x << 16), __uint_as_float(av.x & 0xffff0000u),
                            __uint_as_float(av.y << 16), __uint_as_float(av.y & 0xffff0000u)};
        const float b[4] = {__uint_as_float(bv.x << 16), __uint_as_float(bv.x & 0xffff0000u),
                            __uint_as_float(bv.y << 16), __uint_as_float(bv.y & 0xffff0000u)};
        const float g[4] = {dh.x, dh.y, dh.z, dh.w};
        float da[4], db[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float s = 1.0f / (1.0f + expf(-a[i]));
            db[i] = g[i] * a[i] * s;
            da[i] = g[i] * b[i] * (s + a[i] * s * (1.0f - s));
        }
        uint2 o;
        o.x = pack_bf16x2(da[0], da[1]);
        o.y = pack_bf16x2(da[2], da[3]);
        *reinterpret_cast<uint2*>(DADB + p * 2 * dff + c) = o;
        o.x = pack_bf16x2(db[0], db[1]);
        o.y = pack_bf16x2(db[2], db[3]);
        *reinterpret_cast<uint2*>(DADB + p * 2 * dff + dff + c) = o;
    }
}

// Per token: the router-logit gradient dl (thread 0, written to dl[t][n]),
// then dx_t = W_g dl + sum_j DX[inv[t K + j]] in fp32, rounded once to bf16.
__global__ __launch_bounds__(256) void bwd_token_kernel(
    const uint16_t* __restrict__ wg, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dg, const float* __restrict__ DX,
    const int32_t* __restrict__ inv, int K, int n, int d, float* __restrict__ dl,
    uint16_t* __restrict__ dx) {
    __shared__ float sdl[64];
    const int64_t t = blockIdx.x;
    if (threadIdx.x < 64) sdl[threadIdx.x] = 0.0f;
    __syncthreads();
    if (threadIdx.x == 0) {
        float gdg = 0.0f;
        for (int j = 0; j < K; ++j) gdg = fmaf(gate[t * K + j], dg[t * K + j], gdg);
        for (int j = 0; j < K; ++j)
            sdl[idx[t * K + j]] = gate[t * K + j] * (dg[t * K + j] - gdg);
    }
    __syncthreads();
    if (threadIdx.x < n) dl[t * n + threadIdx.x] = sdl[threadIdx.x];
    for (int k = threadIdx.x; k < d; k += 256) {
        float s = 0.0f;
        for (int i = 0; i < n; ++i) s = fmaf(bf(wg[(int64_t)k * n + i]), sdl[i], s);
        for (int j = 0; j < K; ++j) s += DX[(int64_t)inv[t * K + j] * d + k];
        dx[t * d + k] = (uint16_t)f32_to_bf16_bits(s);
    }
}

// dW_g partial sums: block (kb, ch) covers rows [256 kb, 256 kb + 256) of
// W_g and tokens [ch tpc, (ch + 1) tpc); part[ch][k][i] = sum_t x[t][k] dl[t][i].
template <int NE>
__global__ __launch_bounds__(256) void bwd_dwg_partial_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ dl,
                                                             int64_t T, int d, int n, int tpc,
                                                             float* __restrict__ part) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * tpc;
    const int64_t t1 = min(T, t0 + tpc);
    float acc[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = 0.0f;
    if (k < d) {
        for (int64_t t = t0; t < t1; ++t) {
            const float xv = bf(x[t * d + k]);
#pragma unroll
            for (int i = 0; i < NE; ++i)
                if (i < n) acc[i] = fmaf(xv, dl[t * n + i], acc[i]);
        }
        float* o = part + ((int64_t)blockIdx.y * d + k) * n;
#pragma unroll
        for (int i = 0; i < NE; ++i)
            if (i < n) o[i] = acc[i];
    }
}

// dW_g[k][i] = sum over chunks (in order) of the partial sums.
__global__ __launch_bounds__(256) void bwd_dwg_final_kernel(const float* __restrict__ part,
                                                            int chunks, int64_t dn,
                                                            float* __restrict__ dwg) {
    const int64_t q = blockIdx.x * 256ll + threadIdx.x;
    if (q >= dn) return;
    float s = 0.0f;
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * dn + q];
    dwg[q] = s;
}

// Batched transpose through LDS: for batch b, out[c][ooff + r] (row stride
// ostride) = in[r][icol0 + c] (row stride istride), r < R, c < C.
__global__ __launch_bounds__(256) void transpose_kernel(const uint16_t* __restrict__ in,
                                                        int64_t R, int C, int64_t istride,
                                                        int icol0, int64_t ibatch,
                                                        uint16_t* __restrict__ out,
                                                        int64_t ostride, int64_t ooff,
                                                        int64_t obatch) {
    __shared__ uint16_t tile[64][65];
    in += (int64_t)blockIdx.z * ibatch;
    out += (int64_t)blockIdx.z * obatch;
    const int64_t r0 = (int64_t)blockIdx.y * 64;
    const int c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
    for (int i = ty; i < 64; i += 4) {
        const int64_t r = r0 + i;
        const int c = c0 + tx;
        tile[i][tx] = (r < R && c < C) ? in[r * istride + icol0 + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {
        const int c = c0 + i;
        const int64_t r = r0 + tx;
        if (c < C && r < R) out[(int64_t)c * ostride + ooff + r] = tile[tx][i];
    }
}

// Expert-padded transpose of assignment rows: out[c][q] for q < Kp, where
// column q of expert e (padded offsets: each expert's run rounded up to 64)
// is assignment row p = offsets[e] + (q - poff[e]) if that is inside the
// expert's rows, else 0.  The source row is perm[p] / K (gathered tokens) when
// perm is given, else p; value = in[src][icol0 + c].
__global__ __launch_bounds__(256) void transpose_pad_kernel(
    const uint16_t* __restrict__ in, int C, int64_t istride, int icol0,
    const int32_t* __restrict__ offsets, int n, const int32_t* __restrict__ perm, int K,
    int64_t Kp, uint16_t* __restrict__ out) {
    __shared__ uint16_t tile[64][65];
    __shared__ int64_t src_row[64];
    const int64_t q0 = (int64_t)blockIdx.x * 64;
    const int c0 = blockIdx.y * 64;
    if (threadIdx.x < 64) {
        const int64_t q = q0 + threadIdx.x;
        int64_t src = -1;
        int64_t poff = 0;
        for (int e = 0; e < n; ++e) {
            const int64_t m = offsets[e + 1] - offsets[e];
            const int64_t mp = (m + 63) / 64 * 64;
            if (q < poff + mp) {
                const int64_t local = q - poff;
                if (local < m) {
                    const int64_t p = offsets[e] + local;
                    src = perm ? perm[p] / K : p;
                }
                break;
            }
            poff += mp;
        }
        src_row[threadIdx.x] = src;
    }
    __syncthreads();
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int i = ty; i < 64; i += 4) {  // i: column q, tx: channel c
        const int64_t src = src_row[i];
        const int c = c0 + tx;
        tile[i][tx] = (src >= 0 && c < C) ? in[src * istride + icol0 + c] : (uint16_t)0;
    }
    __syncthreads();
    for (int i = ty; i < 64; i += 4) {  // i: channel, tx: column
        const int c = c0 + i;
        const int64_t q = q0 + tx;
        if (c < C && q < Kp) out[(int64_t)c * Kp + q] = tile[tx][i];
    }
}

unsigned grid_for(int64_t work, int64_t per_block) {
    const int64_t b = (work + per_block - 1) / per_block;
    return (unsigned)(b < 1 ? 1 : (b > 65535 * 16 ? 65535 * 16 : b));
}

}  // namespace

hipError_t launch_bwd_h(const uint16_t* AB, int64_t A, int dff, uint16_t* H, hipStream_t s) {
    hipLaunchKernelGGL(bwd_h_kernel, dim3(grid_for(A * (dff / 8), 256)), dim3(256), 0, s, AB, A,
                       dff, H);
    return hipGetLastError();
}

hipError_t launch_bwd_gates(const uint16_t* dy, const float* O, const int32_t* perm,
                            const float* gate, int64_t A, int K, int d, float* dg, uint16_t* DO,
                            hipStream_t s) {
    if (A > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_gates_kernel, dim3((unsigned)A), dim3(256), 0, s, dy, O, perm, gate,
                       K, d, dg, DO);
    return hipGetLastError();
}

hipError_t launch_bwd_swiglu(const uint16_t* AB, const float* DH, int64_t A, int dff,
                             uint16_t* DADB, hipStream_t s) {
    hipLaunchKernelGGL(bwd_swiglu_kernel, dim3(grid_for(A * (dff / 4), 256)), dim3(256), 0, s,
                       AB, DH, A, dff, DADB);
    return hipGetLastError();
}

hipError_t launch_bwd_token(const uint16_t* wg, const int32_t* idx, const float* gate,
                            const float* dg, const float* DX, const int32_t* inv, int64_t T,
                            int K, int n, int d, float* dl, uint16_t* dx, hipStream_t s) {
    if (T > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_token_kernel, dim3((unsigned)T), dim3(256), 0, s, wg, idx, gate, dg,
                       DX, inv, K, n, d, dl, dx);
    return hipGetLastError();
}

int bwd_dwg_chunks(int64_t T) { return (int)((T + 255) / 256 < 64 ? (T + 255) / 256 : 64); }

hipError_t launch_bwd_dwg(const uint16_t* x, const float* dl, int64_t T, int d, int n,
                          float* part, float* dwg, hipStream_t s) {
    const int chunks = bwd_dwg_chunks(T);
    const int tpc = (int)((T + chunks - 1) / chunks);
    const dim3 grid((unsigned)((d + 255) / 256), (unsigned)chunks);
    if (n <= 8)
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<8>), grid, dim3(256), 0, s, x, dl, T, d, n,
                           tpc, part);
    else if (n <= 16)
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<16>), grid, dim3(256), 0, s, x, dl, T, d, n,
                           tpc, part);
    else if (n <= 32)
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<32>), grid, dim3(256), 0, s, x, dl, T, d, n,
                           tpc, part);
    else
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<64>), grid, dim3(256), 0, s, x, dl, T, d, n,
                           tpc, part);
    const int64_t dn = (int64_t)d * n;
    hipLaunchKernelGGL(bwd_dwg_final_kernel, dim3(grid_for(dn, 256)), dim3(256), 0, s, part,
                       chunks, dn, dwg);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* in, int64_t R, int C, int64_t istride, int icol0,
                            int64_t ibatch, uint16_t* out, int64_t ostride, int64_t ooff,
                            int64_t obatch, int batches, hipStream_t s) {
    const int64_t rb = (R + 63) / 64;
    if (rb > 65535 || batches > 65535) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((C + 63) / 64), (unsigned)rb, (unsigned)batches);
    hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, in, R, C, istride, icol0, ibatch,
                       out, ostride, ooff, obatch);
    return hipGetLastError();
}

hipError_t launch_transpose_pad(const uint16_t* in, int C, int64_t istride, int icol0,
                                const int32_t* offsets, int n, const int32_t* perm, int K,
                                int64_t Kp, uint16_t* out, hipStream_t s) {
    const int64_t qb = Kp / 64;
    if (Kp % 64 || qb > 0x7fffffff || (C + 63) / 64 > 65535)
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)qb, (unsigned)((C + 63) / 64));
    hipLaunchKernelGGL(transpose_pad_kernel, grid, dim3(256), 0, s, in, C, istride, icol0, offsets,
                       n, perm, K, Kp, out);
    return hipGetLastError();
}

}  // namespace moe
