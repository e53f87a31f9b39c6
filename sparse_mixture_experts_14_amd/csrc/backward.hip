// Elementwise, reduction and gather kernels of the backward pass (bf16 data,
// fp32 arithmetic).  The grouped products themselves run on the MFMA kernels
// of gemm_bf16.hip, which read the weights and the per-expert activation rows
// in their stored layouts (no transposed copies).
//
// Gradients of L = sum_t dy_t . y_t through the layer of "Mixtral of
// Experts" (xyznot digest, "Method" section: gate equation and output
// equation; "Key terms": SwiGLU experts).  For token t, kept experts s_j with
// gates g_j, e = s_j, a = W1_e x, b = W3_e x, h = SiLU(a) b, o = W2_e h:
//   r = W2_e^T dy  (the gradient of h through the ungated output),
//   dg_j = dy . o = h . r,  dh = g_j r,
//   da = dh b SiLU'(a),  db = dh SiLU(a),
//   dx = sum_j (W1_e^T da + W3_e^T db) + W_g dl,
//   dl_{s_j} = g_j (dg_j - sum_k g_k dg_k)  (softmax over the kept logits;
//   the other logits get 0: TopK is constant away from ties),
//   dW_g = sum_t x_t dl_t^T,  dW2_e = sum dy (g_j h)^T,
//   dW1_e = sum da x^T,  dW3_e = sum db x^T.
// Taking dg_j as h . r needs no recomputed expert output o.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float bf(uint16_t v) { return bf16_bits_to_f32(v); }

// One block per assignment row p (a = perm[p], g = gate[a]); 8 elements of
// [a | b] and of r = DH[p] (bf16) per thread and step:
//   h = bf16(SiLU(a) b) (the forward's rounding point), dg[a] = sum h r
//   (fixed-order block sum), dh = g r, da = dh b SiLU'(a), db = dh SiLU(a),
//   DADB[p] = bf16([da | db]), GH[p] = bf16(g h).
// PART: r arrives as S fp32 K-split partial sums (split stride sstride
// elements), added in split order, instead of one bf16 row.
template <bool PART>
__global__ __launch_bounds__(256) void bwd_swiglu_kernel(
    const uint16_t* __restrict__ AB, const void* __restrict__ DH, int S, int64_t sstride,
    const int32_t* __restrict__ perm, const float* __restrict__ gate, int dff,
    float* __restrict__ dg, uint16_t* __restrict__ DADB, uint16_t* __restrict__ GH) {
    __shared__ float part[4];
    const int64_t p = blockIdx.x;
    const int a_idx = perm[p];
    const float g = gate[a_idx];
    const uint16_t* ab = AB + p * 2 * dff;
    const uint16_t* r = static_cast<const uint16_t*>(DH) + p * dff;
    const float* rp = static_cast<const float*>(DH) + p * dff;
    uint16_t* dadb = DADB + p * 2 * dff;
    float acc = 0.0f;
    for (int c = threadIdx.x * 8; c < dff; c += 256 * 8) {
        float av[8], bv[8], h[8], da[8], db[8], gh[8];
        unpack_bf16x8(*reinterpret_cast<const uint4*>(ab + c), av);
        unpack_bf16x8(*reinterpret_cast<const uint4*>(ab + dff + c), bv);
        float rv[8];
        if (PART) {
#pragma unroll
            for (int i = 0; i < 8; ++i) rv[i] = 0.0f;
            for (int q = 0; q < S; ++q) {
                const float4 r0 = *reinterpret_cast<const float4*>(rp + q * sstride + c);
                const float4 r1 = *reinterpret_cast<const float4*>(rp + q * sstride + c + 4);
                rv[0] += r0.x; rv[1] += r0.y; rv[2] += r0.z; rv[3] += r0.w;
                rv[4] += r1.x; rv[5] += r1.y; rv[6] += r1.z; rv[7] += r1.w;
            }
        } else {
            unpack_bf16x8(*reinterpret_cast<const uint4*>(r + c), rv);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sg = 1.0f / (1.0f + expf(-av[i]));
            const float si = av[i] * sg;
            h[i] = bf16_bits_to_f32(f32_to_bf16_bits(si * bv[i]));
            acc = fmaf(h[i], rv[i], acc);
            const float dh = g * rv[i];
            db[i] = dh * si;
            da[i] = dh * bv[i] * (sg + si * (1.0f - sg));
            gh[i] = g * h[i];
        }
        uint4 o;
        o.x = pack_bf16x2(da[0], da[1]);
        o.y = pack_bf16x2(da[2], da[3]);
        o.z = pack_bf16x2(da[4], da[5]);
        o.w = pack_bf16x2(da[6], da[7]);
        *reinterpret_cast<uint4*>(dadb + c) = o;
        o.x = pack_bf16x2(db[0], db[1]);
        o.y = pack_bf16x2(db[2], db[3]);
        o.z = pack_bf16x2(db[4], db[5]);
        o.w = pack_bf16x2(db[6], db[7]);
        *reinterpret_cast<uint4*>(dadb + dff + c) = o;
        o.x = pack_bf16x2(gh[0], gh[1]);
        o.y = pack_bf16x2(gh[2], gh[3]);
        o.z = pack_bf16x2(gh[4], gh[5]);
        o.w = pack_bf16x2(gh[6], gh[7]);
        *reinterpret_cast<uint4*>(GH + p * dff + c) = o;
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = acc;
    __syncthreads();
    if (threadIdx.x == 0) dg[a_idx] = (part[0] + part[1]) + (part[2] + part[3]);
}

// Per token: the router-logit gradient dl (thread 0, written to dl[t][n]),
// then dx_t = W_g dl + sum_j sum_s DX[s][inv[t K + j]] in fp32 (in that
// order), rounded once to bf16 (RNE) -- or kept in fp32 (dx32, when given:
// the gradient with respect to a stack layer's normalised input).
__global__ __launch_bounds__(256) void bwd_token_kernel(
    const uint16_t* __restrict__ wg, const int32_t* __restrict__ idx,
    const float* __restrict__ gate, const float* __restrict__ dg, const float* __restrict__ DX,
    int S, int64_t split_stride, const int32_t* __restrict__ inv, int K, int n, int d,
    float* __restrict__ dl, uint16_t* __restrict__ dx, float* __restrict__ dx32,
    const int* __restrict__ split_meta) {
    // rows from R0 on hold Sr partial sums, the rows before it one
    const int R0 = split_meta ? split_meta[0] : 0;
    const int Sr = split_meta ? split_meta[1] : S;
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
    if (threadIdx.x < n && blockIdx.y == 0) dl[t * n + threadIdx.x] = sdl[threadIdx.x];
    // four columns per thread (16-byte loads of the partial sums); block y
    // takes columns [1024 y, 1024 y + 1024) of every 1024 gridDim.y
    for (int k = blockIdx.y * 1024 + threadIdx.x * 4; k < d; k += 1024 * gridDim.y) {
        float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        if (n == 8) {  // a W_g row is one 16-byte load; the same sums in the same order
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                float w[8];
                unpack_bf16x8(*reinterpret_cast<const uint4*>(wg + (int64_t)(k + u) * 8), w);
#pragma unroll
                for (int i = 0; i < 8; ++i) s[u] = fmaf(w[i], sdl[i], s[u]);
            }
        } else {
            for (int i = 0; i < n; ++i) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    s[u] = fmaf(bf(wg[(int64_t)(k + u) * n + i]), sdl[i], s[u]);
            }
        }
        for (int j = 0; j < K; ++j) {
            const int pos = inv[t * K + j];
            const int np = pos >= R0 ? Sr : 1;
            // partial q >= 1: row A + (q - 1)(A - R0) + pos - R0 (R0 = 0: q A + pos)
            const int64_t A = split_stride / d;
#pragma unroll 4
            for (int q = 0; q < np; ++q) {
                const int64_t r = q == 0 ? pos : A + (int64_t)(q - 1) * (A - R0) + pos - R0;
                const float4 v = *reinterpret_cast<const float4*>(DX + r * d + k);
                s[0] += v.x;
                s[1] += v.y;
                s[2] += v.z;
                s[3] += v.w;
            }
        }
        if (dx32) {
            *reinterpret_cast<float4*>(dx32 + t * d + k) = float4{s[0], s[1], s[2], s[3]};
        } else {
            uint2 o;
            o.x = pack_bf16x2(s[0], s[1]);
            o.y = pack_bf16x2(s[2], s[3]);
            *reinterpret_cast<uint2*>(dx + t * d + k) = o;
        }
    }
}

// Stack layer y = x + MoE(u), u = x s, s = 1 / sqrt(mean(x^2) + eps): per
// token, from the gradient du (fp32) with respect to u,
//   dx = dy + s (du - u (u . du) / d)   (fp32, rounded once to bf16),
// and the token's scale s for the router weight gradient.
__global__ __launch_bounds__(256) void bwd_rms_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ dy,
                                                      const float* __restrict__ du, int d,
                                                      float eps, uint16_t* __restrict__ dx,
                                                      float* __restrict__ scale) {
    __shared__ float red[2][4];
    const int64_t t = blockIdx.x;
    const uint16_t* xt = x + t * d;
    const float* dut = du + t * d;
    float ss = 0.0f, xd = 0.0f;  // sum x^2, sum x du
    for (int k = threadIdx.x * 4; k < d; k += 1024) {
        const uint2 xv = *reinterpret_cast<const uint2*>(xt + k);
        const float4 g = *reinterpret_cast<const float4*>(dut + k);
        const float a[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xffff0000u),
                            __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xffff0000u)};
        ss = fmaf(a[0], a[0], ss);
        ss = fmaf(a[1], a[1], ss);
        ss = fmaf(a[2], a[2], ss);
        ss = fmaf(a[3], a[3], ss);
        xd = fmaf(a[0], g.x, xd);
        xd = fmaf(a[1], g.y, xd);
        xd = fmaf(a[2], g.z, xd);
        xd = fmaf(a[3], g.w, xd);
    }
    ss = wave_sum(ss);
    xd = wave_sum(xd);
    if ((threadIdx.x & (kWave - 1)) == 0) {
        red[0][threadIdx.x / kWave] = ss;
        red[1][threadIdx.x / kWave] = xd;
    }
    __syncthreads();
    ss = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    xd = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
    const float sc = 1.0f / sqrtf(ss / (float)d + eps);
    // u . du / d = s (x . du) / d
    const float c = sc * xd / (float)d;
    if (threadIdx.x == 0) scale[t] = sc;
    for (int k = threadIdx.x * 4; k < d; k += 1024) {
        const uint2 xv = *reinterpret_cast<const uint2*>(xt + k);
        const uint2 yv = *reinterpret_cast<const uint2*>(dy + t * d + k);
        const float4 g = *reinterpret_cast<const float4*>(dut + k);
        const float a[4] = {__uint_as_float(xv.x << 16), __uint_as_float(xv.x & 0xffff0000u),
                            __uint_as_float(xv.y << 16), __uint_as_float(xv.y & 0xffff0000u)};
        const float r[4] = {__uint_as_float(yv.x << 16), __uint_as_float(yv.x & 0xffff0000u),
                            __uint_as_float(yv.y << 16), __uint_as_float(yv.y & 0xffff0000u)};
        const float gv[4] = {g.x, g.y, g.z, g.w};
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = r[i] + sc * (gv[i] - (a[i] * sc) * c);
        uint2 w;
        w.x = pack_bf16x2(o[0], o[1]);
        w.y = pack_bf16x2(o[2], o[3]);
        *reinterpret_cast<uint2*>(dx + t * d + k) = w;
    }
}

// dW_g partial sums: block (kb, ch) covers rows [256 kb, 256 kb + 256) of
// W_g and tokens [ch tpc, (ch + 1) tpc); part[ch][k][i] = sum_t x[t][k] dl[t][i]
// in token order.  The block's dl rows go through LDS 64 tokens at a time,
// padded to NE columns with zeros, and each thread keeps 8 independent x
// loads in flight.
// scale (nullable): the rows are x[t] scale[t] (a stack layer's u).
template <int NE>
__global__ __launch_bounds__(256) void bwd_dwg_partial_kernel(const uint16_t* __restrict__ x,
                                                             const float* __restrict__ scale,
                                                             const float* __restrict__ dl,
                                                             int64_t T, int d, int n, int tpc,
                                                             float* __restrict__ part) {
    constexpr int TB = 64;  // tokens per LDS batch
    __shared__ float sdl[TB][NE];
    const int k = blockIdx.x * 256 + threadIdx.x;
    const int64_t t0 = (int64_t)blockIdx.y * tpc;
    const int64_t t1 = min(T, t0 + tpc);
    float acc[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = 0.0f;
    const uint16_t* xp = x + (k < d ? k : 0);
    for (int64_t tb = t0; tb < t1; tb += TB) {
        const int cnt = (int)min((int64_t)TB, t1 - tb);
        __syncthreads();
        for (int q = threadIdx.x; q < TB * NE; q += 256) {
            const int tt = q / NE, i = q % NE;
            sdl[tt][i] = (tt < cnt && i < n)
                             ? dl[(tb + tt) * n + i] * (scale ? scale[tb + tt] : 1.0f)
                             : 0.0f;
        }
        __syncthreads();
        if (k < d) {
            int tt = 0;
            for (; tt + 8 <= cnt; tt += 8) {
                float xv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) xv[u] = bf(xp[(tb + tt + u) * d]);
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int i = 0; i < NE; ++i) acc[i] = fmaf(xv[u], sdl[tt + u][i], acc[i]);
            }
            for (; tt < cnt; ++tt) {
                const float xv = bf(xp[(tb + tt) * d]);
#pragma unroll
                for (int i = 0; i < NE; ++i) acc[i] = fmaf(xv, sdl[tt][i], acc[i]);
            }
        }
    }
    if (k < d) {
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
#pragma unroll 8
    for (int c = 0; c < chunks; ++c) s += part[(int64_t)c * dn + q];
    dwg[q] = s;
}

// XG[p] = x[perm[p] / K] and YG[p] = y[perm[p] / K]: the rows of every
// assignment in expert order (16 bytes per thread and array).
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ y,
                                                          const int32_t* __restrict__ perm,
                                                          int K, int64_t A, int d,
                                                          uint16_t* __restrict__ XG,
                                                          uint16_t* __restrict__ YG) {
    const int cpr = d / 8;
    const int64_t chunks = A * cpr;
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < chunks; q += (int64_t)gridDim.x * 256) {
        const int64_t p = q / cpr;
        const int c = (int)(q % cpr) * 8;
        const int64_t src = (int64_t)(perm[p] / K) * d + c;
        *reinterpret_cast<uint4*>(XG + p * d + c) = *reinterpret_cast<const uint4*>(x + src);
        *reinterpret_cast<uint4*>(YG + p * d + c) = *reinterpret_cast<const uint4*>(y + src);
    }
}

// Zero fill, 16 bytes per thread (a kernel, so that a captured graph never
// holds a memset node); bytes is a multiple of 16.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ p, int64_t n16) {
    for (int64_t q = blockIdx.x * 256ll + threadIdx.x; q < n16; q += (int64_t)gridDim.x * 256)
        p[q] = uint4{0u, 0u, 0u, 0u};
}

unsigned grid_for(int64_t work, int64_t per_block) {
    const int64_t b = (work + per_block - 1) / per_block;
    return (unsigned)(b < 1 ? 1 : (b > 65535 * 16 ? 65535 * 16 : b));
}

}  // namespace

hipError_t launch_bwd_swiglu(const uint16_t* AB, const uint16_t* DH, const float* DHP, int S,
                             const int32_t* perm, const float* gate, int64_t A, int dff,
                             float* dg, uint16_t* DADB, uint16_t* GH, hipStream_t s) {
    if (A > 0x7fffffff || dff % 8 || (DHP && S < 1)) return hipErrorInvalidConfiguration;
    if (DHP)
        hipLaunchKernelGGL((bwd_swiglu_kernel<true>), dim3((unsigned)A), dim3(256), 0, s, AB,
                           (const void*)DHP, S, A * dff, perm, gate, dff, dg, DADB, GH);
    else
        hipLaunchKernelGGL((bwd_swiglu_kernel<false>), dim3((unsigned)A), dim3(256), 0, s, AB,
                           (const void*)DH, 1, (int64_t)0, perm, gate, dff, dg, DADB, GH);
    return hipGetLastError();
}

hipError_t launch_bwd_token(const uint16_t* wg, const int32_t* idx, const float* gate,
                            const float* dg, const float* DX, int S, int64_t A,
                            const int32_t* inv, int64_t T, int K, int n, int d, float* dl,
                            uint16_t* dx, float* dx32, const int* split_meta, hipStream_t s) {
    if (T > 0x7fffffff) return hipErrorInvalidConfiguration;
    // few tokens: spread each token's columns over several blocks
    const int ycols = (d + 1023) / 1024;
    const int gy = T >= 1024 ? 1 : ycols;
    hipLaunchKernelGGL(bwd_token_kernel, dim3((unsigned)T, (unsigned)gy), dim3(256), 0, s, wg,
                       idx, gate, dg, DX, S, A * d, inv, K, n, d, dl, dx, dx32, split_meta);
    return hipGetLastError();
}

hipError_t launch_bwd_rms(const uint16_t* x, const uint16_t* dy, const float* du, int64_t T,
                          int d, float eps, uint16_t* dx, float* scale, hipStream_t s) {
    if (T > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_rms_kernel, dim3((unsigned)T), dim3(256), 0, s, x, dy, du, d, eps, dx,
                       scale);
    return hipGetLastError();
}

int bwd_dwg_chunks(int64_t T) { return (int)((T + 63) / 64 < 256 ? (T + 63) / 64 : 256); }

hipError_t launch_bwd_dwg(const uint16_t* x, const float* scale, const float* dl, int64_t T,
                          int d, int n, float* part, float* dwg, hipStream_t s) {
    const int chunks = bwd_dwg_chunks(T);
    const int tpc = (int)((T + chunks - 1) / chunks);
    const dim3 grid((unsigned)((d + 255) / 256), (unsigned)chunks);
    if (n <= 8)
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<8>), grid, dim3(256), 0, s, x, scale, dl, T, d, n,
                           tpc, part);
    else if (n <= 16)
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<16>), grid, dim3(256), 0, s, x, scale, dl, T, d, n,
                           tpc, part);
    else if (n <= 32)
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<32>), grid, dim3(256), 0, s, x, scale, dl, T, d, n,
                           tpc, part);
    else
        hipLaunchKernelGGL((bwd_dwg_partial_kernel<64>), grid, dim3(256), 0, s, x, scale, dl, T, d, n,
                           tpc, part);
    const int64_t dn = (int64_t)d * n;
    hipLaunchKernelGGL(bwd_dwg_final_kernel, dim3(grid_for(dn, 256)), dim3(256), 0, s, part,
                       chunks, dn, dwg);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    if (bytes % 16) return hipErrorInvalidValue;
    if (bytes == 0) return hipSuccess;
    const int64_t n16 = (int64_t)(bytes / 16);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16, 256)), dim3(256), 0, s,
                       static_cast<uint4*>(p), n16);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const uint16_t* x, const uint16_t* y, const int32_t* perm, int K,
                              int64_t A, int d, uint16_t* XG, uint16_t* YG, hipStream_t s) {
    hipLaunchKernelGGL(gather_rows_kernel, dim3(grid_for(A * (d / 8), 256)), dim3(256), 0, s, x,
                       y, perm, K, A, d, XG, YG);
    return hipGetLastError();
}

}  // namespace moe
