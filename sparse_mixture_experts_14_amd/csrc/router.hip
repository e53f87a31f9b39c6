// Router: logits l = x . W_g, TopK, softmax over the kept logits.
//
// "Mixtral of Experts", xyznot digest, section "Method (with core equations)":
// G(x) = Softmax(TopK(x . W_g)); TopK leaves the K largest logits and sets the
// rest to -inf, so the softmax normalises over the K kept logits only.
//
// One workgroup of 256 threads per token.  Thread i reads the 16-byte chunks
// i, i+256, ... of the token's row, multiplies each element with the matching
// row of W_g (n contiguous values), and keeps n fp32 partial sums; a butterfly
// inside each wave and a fixed-order sum of the 4 waves' partials in LDS give
// the n logits (fp32, never rounded to bf16, same order every call).  Thread
// 0 then takes the TopK (ties to the lower index) and the softmax.
//
// The pre-normalised variant (a layer of a residual stack) also accumulates
// sum(x^2), scales the logits by rstd = 1/sqrt(mean(x^2) + eps) -- the same
// logits as those of u = x * rstd, in fp32 -- and writes u in the storage
// dtype for the expert GEMMs.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <typename TIn>
struct Vec;

template <>
struct Vec<uint16_t> {  // bf16 storage: 8 values per 16-byte chunk
    static constexpr int N = 8;
    __device__ static void load(const uint16_t* p, float* f) {
        unpack_bf16x8(*reinterpret_cast<const uint4*>(p), f);
    }
    __device__ static float scalar(const uint16_t* p) { return bf16_bits_to_f32(*p); }
    __device__ static void store(uint16_t* p, const float* f) {
        uint4 v;
        v.x = pack_bf16x2(f[0], f[1]);
        v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]);
        v.w = pack_bf16x2(f[6], f[7]);
        *reinterpret_cast<uint4*>(p) = v;
    }
};

template <>
struct Vec<float> {  // fp32 storage: 4 values per 16-byte chunk
    static constexpr int N = 4;
    __device__ static void load(const float* p, float* f) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        f[0] = v.x;
        f[1] = v.y;
        f[2] = v.z;
        f[3] = v.w;
    }
    __device__ static float scalar(const float* p) { return *p; }
    __device__ static void store(float* p, const float* f) {
        *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    }
};

// acc[e] += xv * W_g[k][e] for e < n.  Fast path: n == NE with NE % 8 == 0
// (bf16) or NE % 4 == 0 (fp32): the row of W_g is read as 16-byte vectors.
template <typename TIn, int NE>
__device__ __forceinline__ void axpy_row(const TIn* __restrict__ w, int n, float xv,
                                         float* acc) {
    constexpr int VN = Vec<TIn>::N;
    if (NE % VN == 0 && n == NE) {
#pragma unroll
        for (int e0 = 0; e0 < NE; e0 += VN) {
            float wf[VN];
            Vec<TIn>::load(w + e0, wf);
#pragma unroll
            for (int j = 0; j < VN; ++j) acc[e0 + j] = fmaf(xv, wf[j], acc[e0 + j]);
        }
    } else {
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (e < n) acc[e] = fmaf(xv, Vec<TIn>::scalar(w + e), acc[e]);
    }
}

template <typename TIn, int NE, bool NORM>
__global__ __launch_bounds__(256) void router_kernel(
    const TIn* __restrict__ x, const TIn* __restrict__ wg, int64_t T, int d, int n,
    int K, float eps, int32_t* __restrict__ idx, float* __restrict__ gate,
    TIn* __restrict__ u_out) {
    constexpr int VN = Vec<TIn>::N;
    constexpr int NTH = 256;
    __shared__ float part[NTH / kWave][NE + 1];
    __shared__ float s_rstd;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;
    const int64_t t = blockIdx.x;
    const TIn* __restrict__ xr = x + t * (int64_t)d;

    float acc[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = 0.0f;
    float ss = 0.0f;

    // d is a multiple of 8, so every chunk is either whole or absent.
    for (int k0 = threadIdx.x * VN; k0 < d; k0 += NTH * VN) {
        float xv[VN];
        Vec<TIn>::load(xr + k0, xv);
#pragma unroll
        for (int j = 0; j < VN; ++j) {
            if (NORM) ss = fmaf(xv[j], xv[j], ss);
            axpy_row<TIn, NE>(wg + (int64_t)(k0 + j) * n, n, xv[j], acc);
        }
    }
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[e] = wave_sum(acc[e]);
    if (NORM) ss = wave_sum(ss);
    if (lane == 0) {
#pragma unroll
        for (int e = 0; e < NE; ++e) part[wv][e] = acc[e];
        part[wv][NE] = ss;
    }
    __syncthreads();

    if (threadIdx.x == 0) {
        float l[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e)
            l[e] = (part[0][e] + part[1][e]) + (part[2][e] + part[3][e]);
        float rstd = 1.0f;
        if (NORM) {
            const float sst = (part[0][NE] + part[1][NE]) + (part[2][NE] + part[3][NE]);
            rstd = 1.0f / sqrtf(sst / (float)d + eps);
#pragma unroll
            for (int e = 0; e < NE; ++e) l[e] *= rstd;
            s_rstd = rstd;
        }
        // TopK: K rounds of "largest logit not yet taken"; a later expert
        // needs a strictly larger logit, so ties go to the lower index.
        uint64_t taken = 0;
        int sel[8];
        float val[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < K) {
                int best = -1;
                float bv = 0.0f;
#pragma unroll
                for (int e = 0; e < NE; ++e) {
                    if (e < n && !((taken >> e) & 1ull)) {
                        if (best < 0 || l[e] > bv) {
                            best = e;
                            bv = l[e];
                        }
                    }
                }
                taken |= 1ull << best;
                sel[j] = best;
                val[j] = bv;
            }
        }
        // Softmax over the kept logits; val[0] is the largest.
        float g[8];
        float z = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < K) {
                g[j] = expf(val[j] - val[0]);
                z += g[j];
            }
        }
        const float rz = 1.0f / z;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (j < K) {
                idx[t * K + j] = sel[j];
                gate[t * K + j] = g[j] * rz;
            }
        }
    }

    if (NORM) {
        __syncthreads();
        const float rstd = s_rstd;
        TIn* __restrict__ ur = u_out + t * (int64_t)d;
        for (int k0 = threadIdx.x * VN; k0 < d; k0 += NTH * VN) {
            float xv[VN];
            Vec<TIn>::load(xr + k0, xv);
#pragma unroll
            for (int j = 0; j < VN; ++j) xv[j] *= rstd;
            Vec<TIn>::store(ur + k0, xv);
        }
    }
}

// Resident-weight variant (bf16, n = 8, d = 256 * ELEMS): thread i keeps
// rows [i ELEMS, (i + 1) ELEMS) of W_g (8 bf16 = 16 bytes per row) in
// registers and walks the tokens blockIdx.x, blockIdx.x + gridDim.x, ...,
// prefetching the next token's slice of x while it reduces the current one.
// W_g is then read once per workgroup instead of once per token.  Per token:
// ELEMS * 8 fp32 FMAs per thread, a wave butterfly and a fixed-order sum of
// the 4 waves' partials in LDS (deterministic), then thread 0 takes TopK
// (ties to the lower index) and the softmax.  The pre-normalised variant
// also sums x^2; every thread forms rstd from the same LDS partials (same
// order, same value) and writes its slice of u.
template <int ELEMS, bool NORM>
__global__ __launch_bounds__(256) void router_resident_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int64_t T, int d, int K,
    float eps, int32_t* __restrict__ idx, float* __restrict__ gate,
    uint16_t* __restrict__ u_out) {
    constexpr int NE = 8;
    constexpr int XV = ELEMS / 8;  // 16-byte chunks of x per thread
    __shared__ float part[2][4][NE + 1];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const int k0 = tid * ELEMS;
    uint4 w[ELEMS];
#pragma unroll
    for (int j = 0; j < ELEMS; ++j) w[j] = *reinterpret_cast<const uint4*>(wg + (int64_t)(k0 + j) * NE);
    auto wget = [&](int j, int e) {
        const uint32_t v = e < 2 ? w[j].x : e < 4 ? w[j].y : e < 6 ? w[j].z : w[j].w;
        return (e & 1) ? __uint_as_float(v & 0xffff0000u) : __uint_as_float(v << 16);
    };
    auto load = [&](uint4(&xv)[XV], int64_t t) {
        const uint4* p = reinterpret_cast<const uint4*>(x + t * (int64_t)d + k0);
#pragma unroll
        for (int c = 0; c < XV; ++c) xv[c] = p[c];
    };
    auto xget = [&](const uint4(&xv)[XV], int j) {
        const uint4& c = xv[j / 8];
        const int e = j % 8;
        const uint32_t v = e < 2 ? c.x : e < 4 ? c.y : e < 6 ? c.z : c.w;
        return (e & 1) ? __uint_as_float(v & 0xffff0000u) : __uint_as_float(v << 16);
    };
    int64_t t = blockIdx.x;
    uint4 xv[XV];
    if (t < T) load(xv, t);
    for (int par = 0; t < T; t += gridDim.x, par ^= 1) {
        uint4 xn[XV];
        const int64_t tn = t + gridDim.x;
        if (tn < T) load(xn, tn);
        float acc[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[e] = 0.0f;
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < ELEMS; ++j) {
            const float xf = xget(xv, j);
            if (NORM) ss = fmaf(xf, xf, ss);
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[e] = fmaf(xf, wget(j, e), acc[e]);
        }
        // Reduce-scatter over the wave: the xor-32/16/8 exchanges halve the
        // values a lane keeps (4 + 2 + 1 shuffles), the xor-4/2/1 butterfly
        // finishes the sums; lane 8 e' then holds logit e' = lane bits 5..3.
        float v4[4], v2[2];
        const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float mine = b5 ? acc[4 + i] : acc[i], other = b5 ? acc[i] : acc[4 + i];
            v4[i] = mine + __shfl_xor(other, 32, kWave);
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const float mine = b4 ? v4[2 + i] : v4[i], other = b4 ? v4[i] : v4[2 + i];
            v2[i] = mine + __shfl_xor(other, 16, kWave);
        }
        float v1 = (b3 ? v2[1] : v2[0]) + __shfl_xor(b3 ? v2[0] : v2[1], 8, kWave);
        v1 += __shfl_xor(v1, 4, kWave);
        v1 += __shfl_xor(v1, 2, kWave);
        v1 += __shfl_xor(v1, 1, kWave);
        if (NORM) ss = wave_sum(ss);
        if ((lane & 7) == 0) part[par][wv][lane >> 3] = v1;
        if (NORM && lane == 0) part[par][wv][NE] = ss;
        __syncthreads();
        float rstd = 1.0f;
        if (NORM) {
            const float sst = (part[par][0][NE] + part[par][1][NE]) +
                              (part[par][2][NE] + part[par][3][NE]);
            rstd = 1.0f / sqrtf(sst / (float)d + eps);
        }
        if (tid == 0) {
            float l[NE];
#pragma unroll
            for (int e = 0; e < NE; ++e)
                l[e] = ((part[par][0][e] + part[par][1][e]) + (part[par][2][e] + part[par][3][e])) *
                       rstd;
            uint32_t taken = 0;
            int sel[8];
            float val[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < K) {
                    int best = -1;
                    float bv = 0.0f;
#pragma unroll
                    for (int e = 0; e < NE; ++e) {
                        if (!((taken >> e) & 1u) && (best < 0 || l[e] > bv)) {
                            best = e;
                            bv = l[e];
                        }
                    }
                    taken |= 1u << best;
                    sel[j] = best;
                    val[j] = bv;
                }
            }
            float g[8];
            float z = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < K) {
                    g[j] = expf(val[j] - val[0]);
                    z += g[j];
                }
            }
            const float rz = 1.0f / z;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (j < K) {
                    idx[t * K + j] = sel[j];
                    gate[t * K + j] = g[j] * rz;
                }
            }
        }
        if (NORM) {
            uint4* up = reinterpret_cast<uint4*>(u_out + t * (int64_t)d + k0);
#pragma unroll
            for (int c = 0; c < XV; ++c) {
                uint4 o;
                o.x = pack_bf16x2(xget(xv, 8 * c + 0) * rstd, xget(xv, 8 * c + 1) * rstd);
                o.y = pack_bf16x2(xget(xv, 8 * c + 2) * rstd, xget(xv, 8 * c + 3) * rstd);
                o.z = pack_bf16x2(xget(xv, 8 * c + 4) * rstd, xget(xv, 8 * c + 5) * rstd);
                o.w = pack_bf16x2(xget(xv, 8 * c + 6) * rstd, xget(xv, 8 * c + 7) * rstd);
                up[c] = o;
            }
        }
#pragma unroll
        for (int c = 0; c < XV; ++c) xv[c] = xn[c];
    }
}

template <bool NORM>
hipError_t launch_router_resident(const void* x, const void* wg, int64_t T, int d, int K,
                                  float eps, int32_t* idx, float* gate, void* u_out,
                                  hipStream_t s) {
    const dim3 grid((unsigned)(T < 512 ? T : 512));
    const dim3 block(256);
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(wg);
    uint16_t* up = static_cast<uint16_t*>(u_out);
    if (d == 2048)
        hipLaunchKernelGGL((router_resident_kernel<8, NORM>), grid, block, 0, s, xp, wp, T, d, K,
                           eps, idx, gate, up);
    else if (d == 4096)
        hipLaunchKernelGGL((router_resident_kernel<16, NORM>), grid, block, 0, s, xp, wp, T, d,
                           K, eps, idx, gate, up);
    else
        hipLaunchKernelGGL((router_resident_kernel<32, NORM>), grid, block, 0, s, xp, wp, T, d,
                           K, eps, idx, gate, up);
    return hipGetLastError();
}

template <typename TIn, bool NORM>
hipError_t launch_router_t(const void* x, const void* wg, int64_t T, int d, int n, int K,
                           float eps, int32_t* idx, float* gate, void* u_out,
                           hipStream_t s) {
    const dim3 grid((unsigned)T);
    const dim3 block(256);
    const TIn* xp = static_cast<const TIn*>(x);
    const TIn* wp = static_cast<const TIn*>(wg);
    TIn* up = static_cast<TIn*>(u_out);
    if (n <= 8)
        hipLaunchKernelGGL((router_kernel<TIn, 8, NORM>), grid, block, 0, s, xp, wp, T, d,
                           n, K, eps, idx, gate, up);
    else if (n <= 16)
        hipLaunchKernelGGL((router_kernel<TIn, 16, NORM>), grid, block, 0, s, xp, wp, T,
                           d, n, K, eps, idx, gate, up);
    else if (n <= 32)
        hipLaunchKernelGGL((router_kernel<TIn, 32, NORM>), grid, block, 0, s, xp, wp, T,
                           d, n, K, eps, idx, gate, up);
    else
        hipLaunchKernelGGL((router_kernel<TIn, 64, NORM>), grid, block, 0, s, xp, wp, T,
                           d, n, K, eps, idx, gate, up);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_router(bool bf16, bool norm, const void* x, const void* wg, int64_t T,
                         int d, int n, int K, float eps, int32_t* idx, float* gate,
                         void* u_out, hipStream_t s) {
    if (bf16 && n == 8 && (d == 2048 || d == 4096 || d == 8192))
        return norm ? launch_router_resident<true>(x, wg, T, d, K, eps, idx, gate, u_out, s)
                    : launch_router_resident<false>(x, wg, T, d, K, eps, idx, gate, u_out, s);
    if (bf16)
        return norm ? launch_router_t<uint16_t, true>(x, wg, T, d, n, K, eps, idx, gate,
                                                      u_out, s)
                    : launch_router_t<uint16_t, false>(x, wg, T, d, n, K, eps, idx, gate,
                                                       u_out, s);
    return norm ? launch_router_t<float, true>(x, wg, T, d, n, K, eps, idx, gate, u_out, s)
                : launch_router_t<float, false>(x, wg, T, d, n, K, eps, idx, gate, u_out,
                                                s);
}

}  // namespace moe
