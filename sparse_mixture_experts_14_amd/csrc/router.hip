// Router: logits l = x . W_g, TopK, softmax over the kept logits.
//
// "Mixtral of Experts", xyznot digest, section "Method (with core equations)":
// G(x) = Softmax(TopK(x . W_g)); TopK leaves the K largest logits and sets the
// rest to -inf, so the softmax normalises over the K kept logits only.
//
// Logits are fp32 sums of exact bf16 (or fp32) products, never rounded to
// bf16, summed in one fixed order (deterministic).  TopK and the softmax run
// across the lanes of one wavefront: a token's logits sit in a group of lanes
// (lane e holds expert e), and each of the K rounds is an argmax butterfly
// over the group on (logit, index) pairs -- the larger logit wins, equal
// logits go to the lower index -- after which the winner's lane drops out.
// The lanes of the group then hold the K selected (index, logit) pairs in
// rank order; lane j < K writes slot j with the softmax weight
// exp(l_j - l_0) / sum_i exp(l_i - l_0).
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

// TopK and softmax of one token whose n <= G logits sit in a group of G
// lanes (G a power of two <= 64; lane e of the group holds expert e's logit,
// lanes e >= n hold nothing).  Every lane of the group ends with the same
// sel / val; lane j < K of the group writes slot j of the token's idx and
// gate rows.
template <int G>
__device__ __forceinline__ void wave_topk_softmax(float l, int e, int n, int K,
                                                  int32_t* __restrict__ idx_row,
                                                  float* __restrict__ gate_row) {
    bool live = e < n;  // still selectable
    int sel[8];
    float val[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j < K) {
            float v = live ? l : -INFINITY;
            int i = live ? e : 0x7fff;
#pragma unroll
            for (int m = 1; m < G; m <<= 1) {
                const float ov = __shfl_xor(v, m, kWave);
                const int oi = __shfl_xor(i, m, kWave);
                if (ov > v || (ov == v && oi < i)) {
                    v = ov;
                    i = oi;
                }
            }
            sel[j] = i;
            val[j] = v;
            if (i == e) live = false;
        }
    }
    // softmax over the kept logits; val[0] is the largest
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
        if (j < K && e == j) {
            idx_row[j] = sel[j];
            gate_row[j] = g[j] * rz;
        }
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

    // Wave 0: lane e < n forms logit e (fixed-order sum of the 4 waves'
    // partials) and the wave takes TopK and the softmax.
    if (wv == 0) {
        float rstd = 1.0f;
        if (NORM) {
            const float sst = (part[0][NE] + part[1][NE]) + (part[2][NE] + part[3][NE]);
            rstd = 1.0f / sqrtf(sst / (float)d + eps);
            if (lane == 0) s_rstd = rstd;
        }
        float l = 0.0f;
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (e == lane) l = ((part[0][e] + part[1][e]) + (part[2][e] + part[3][e])) * rstd;
        wave_topk_softmax<NE>(l, lane, n, K, idx + t * K, gate + t * K);
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

// Halving exchanges over lane bits 5, 4, ..: V = 2^M values per lane in,
// and lane l ends with the wave's full sum of value number l >> (6 - M)
// (the xor-32 exchange halves the values a lane keeps, then xor-16, ...; the
// remaining xor-(32 >> M) .. xor-1 butterfly completes the sums).  A fixed
// order of adds: the result is deterministic.
template <int M>
__device__ __forceinline__ float wave_reduce_scatter(float (&v)[1 << M], int lane) {
#pragma unroll
    for (int st = 0; st < M; ++st) {
        const int mask = 32 >> st;
        const int half = (1 << M) >> (st + 1);
        const bool hi = lane & mask;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            // select values, not array slots (a select of slots becomes a
            // dynamic index into the array)
            const float lo_v = v[i], hi_v = v[half + i];
            const float mine = hi ? hi_v : lo_v;
            const float other = hi ? lo_v : hi_v;
            v[i] = mine + __shfl_xor(other, mask, kWave);
        }
    }
    float r = v[0];
#pragma unroll
    for (int mask = 32 >> M; mask >= 1; mask >>= 1) r += __shfl_xor(r, mask, kWave);
    return r;
}

// Resident-weight variant (bf16, n = 8, d = 256 * ELEMS): thread i keeps
// rows [i ELEMS, (i + 1) ELEMS) of W_g (8 bf16 = 16 bytes per row) in
// registers, so W_g is read once per workgroup, and the workgroup walks
// batches of TB tokens (batch b, b + gridDim.x, ...), prefetching the next
// batch's slices of x while it reduces the current one.  Per batch: ELEMS *
// 4 * TB bf16-pair dot products (fp32 sums) per thread; one wave
// reduce-scatter of the TB * 8
// partial logits; a fixed-order sum of the 4 waves' partials in LDS
// (deterministic); then wave w takes TopK and the softmax of token w of the
// batch in its lanes 0..7.  The pre-normalised variant also reduces the TB
// sums of x^2; every thread forms each token's rstd from the same LDS
// partials (same order, same value) and writes its slices of u.
template <int ELEMS, int TB, bool NORM>
__global__ __launch_bounds__(256) void router_resident_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wg, int64_t T, int d, int K,
    float eps, int32_t* __restrict__ idx, float* __restrict__ gate,
    uint16_t* __restrict__ u_out) {
    constexpr int NE = 8;
    constexpr int XV = ELEMS / 8;  // 16-byte chunks of x per thread and token
    constexpr int M = TB == 4 ? 5 : TB == 2 ? 4 : 3;  // log2(TB * NE)
    constexpr int MS = TB == 4 ? 2 : TB == 2 ? 1 : 0;  // log2(TB)
    static_assert(TB == 1 || TB == 2 || TB == 4, "batches of 1, 2 or 4 tokens");
    __shared__ float part[2][4][TB * NE];
    __shared__ float part_ss[2][4][TB];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wv = tid / kWave;
    const int k0 = tid * ELEMS;
    // W_g rows k0 + 2p and k0 + 2p + 1 packed per expert as bf16 pairs, the
    // operand layout of v_dot2_f32_bf16 (x holds its pairs natively): one
    // dot2 adds both products, and W_g stays packed in 4 ELEMS registers.
    uint32_t wp[ELEMS / 2][NE];
#pragma unroll
    for (int p = 0; p < ELEMS / 2; ++p) {
        const uint4 lo = *reinterpret_cast<const uint4*>(wg + (int64_t)(k0 + 2 * p) * NE);
        const uint4 hi = *reinterpret_cast<const uint4*>(wg + (int64_t)(k0 + 2 * p + 1) * NE);
        const uint32_t l4[4] = {lo.x, lo.y, lo.z, lo.w}, h4[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            wp[p][2 * q] = __builtin_amdgcn_perm(h4[q], l4[q], 0x05040100u);
            wp[p][2 * q + 1] = __builtin_amdgcn_perm(h4[q], l4[q], 0x07060302u);
        }
    }
    // tokens past T read as zeros (their outputs are not written)
    auto load = [&](uint4(&xv)[TB][XV], int64_t t0) {
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            const uint4* p = reinterpret_cast<const uint4*>(x + (t0 + b) * (int64_t)d + k0);
#pragma unroll
            for (int c = 0; c < XV; ++c) xv[b][c] = t0 + b < T ? p[c] : make_uint4(0, 0, 0, 0);
        }
    };
    auto xpair = [&](const uint4(&xv)[XV], int p) {  // elements 2p, 2p + 1 of the slice
        const uint4& c = xv[p / 4];
        const int q = p % 4;
        return __builtin_bit_cast(bf16x2_t, q == 0 ? c.x : q == 1 ? c.y : q == 2 ? c.z : c.w);
    };
    const int64_t nb = (T + TB - 1) / TB;
    int64_t bt = blockIdx.x;
    uint4 xv[TB][XV];
    if (bt < nb) load(xv, bt * TB);
    for (int par = 0; bt < nb; bt += gridDim.x, par ^= 1) {
        const int64_t t0 = bt * TB;
        uint4 xn[TB][XV];
        if (bt + gridDim.x < nb) load(xn, (bt + gridDim.x) * TB);
        float acc[TB * NE];
        float ss[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            ss[b] = 0.0f;
#pragma unroll
            for (int e = 0; e < NE; ++e) acc[b * NE + e] = 0.0f;
#pragma unroll
            for (int p = 0; p < ELEMS / 2; ++p) {
                const bf16x2_t xp2 = xpair(xv[b], p);
                if (NORM) ss[b] = __builtin_amdgcn_fdot2_f32_bf16(xp2, xp2, ss[b], false);
#pragma unroll
                for (int e = 0; e < NE; ++e)
                    acc[b * NE + e] = __builtin_amdgcn_fdot2_f32_bf16(
                        __builtin_bit_cast(bf16x2_t, wp[p][e]), xp2, acc[b * NE + e], false);
            }
        }
        // lane l: the wave's sum of logit (l >> (6 - M)) = token l >> (9 - M),
        // expert (l >> (6 - M)) % 8
        const float lw = wave_reduce_scatter<M>(acc, lane);
        if ((lane & ((1 << (6 - M)) - 1)) == 0) part[par][wv][lane >> (6 - M)] = lw;
        if (NORM) {
            const float sw = wave_reduce_scatter<MS>(ss, lane);
            if ((lane & ((1 << (6 - MS)) - 1)) == 0) part_ss[par][wv][lane >> (6 - MS)] = sw;
        }
        __syncthreads();
        float rstd[TB];
#pragma unroll
        for (int b = 0; b < TB; ++b) {
            rstd[b] = 1.0f;
            if (NORM) {
                const float sst = (part_ss[par][0][b] + part_ss[par][1][b]) +
                                  (part_ss[par][2][b] + part_ss[par][3][b]);
                rstd[b] = 1.0f / sqrtf(sst / (float)d + eps);
            }
        }
        if (wv < TB && t0 + wv < T) {  // wave w: token t0 + w, lane e < 8: expert e
            const int e = lane & 7;
            float rs = rstd[0];
#pragma unroll
            for (int b = 1; b < TB; ++b)
                if (b == wv) rs = rstd[b];
            const int vi = wv * NE + e;
            const float l = ((part[par][0][vi] + part[par][1][vi]) +
                             (part[par][2][vi] + part[par][3][vi])) * rs;
            wave_topk_softmax<8>(l, lane < 8 ? e : NE, NE, K, idx + (t0 + wv) * K,
                                 gate + (t0 + wv) * K);
        }
        if (NORM) {
#pragma unroll
            for (int b = 0; b < TB; ++b) {
                if (t0 + b >= T) continue;
                uint4* up = reinterpret_cast<uint4*>(u_out + (t0 + b) * (int64_t)d + k0);
                const float r = rstd[b];
#pragma unroll
                for (int c = 0; c < XV; ++c) {
                    float f[8];
                    unpack_bf16x8(xv[b][c], f);
                    uint4 o;
                    o.x = pack_bf16x2(f[0] * r, f[1] * r);
                    o.y = pack_bf16x2(f[2] * r, f[3] * r);
                    o.z = pack_bf16x2(f[4] * r, f[5] * r);
                    o.w = pack_bf16x2(f[6] * r, f[7] * r);
                    up[c] = o;
                }
            }
        }
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int c = 0; c < XV; ++c) xv[b][c] = xn[b][c];
    }
}

// Batches of 4 tokens (2 at d = 8192, where W_g alone holds 64 registers
// per thread), at most 512 workgroups; up to 256 tokens, one token per
// workgroup (measured: 4-token batches route T = 4096 in 18.8 us instead of
// 24.9, T = 16384 in 41 instead of 74; at T = 16, 1-token batches take
// 7.1 us, 4-token ones 8.4).
template <int ELEMS, bool NORM>
void launch_router_resident_d(int tb, dim3 grid, hipStream_t s, const uint16_t* xp,
                              const uint16_t* wp, int64_t T, int d, int K, float eps,
                              int32_t* idx, float* gate, uint16_t* up) {
    const dim3 block(256);
    if (tb == 1)
        hipLaunchKernelGGL((router_resident_kernel<ELEMS, 1, NORM>), grid, block, 0, s, xp, wp,
                           T, d, K, eps, idx, gate, up);
    else if (tb == 2)
        hipLaunchKernelGGL((router_resident_kernel<ELEMS, 2, NORM>), grid, block, 0, s, xp, wp,
                           T, d, K, eps, idx, gate, up);
    else if constexpr (ELEMS <= 16)
        hipLaunchKernelGGL((router_resident_kernel<ELEMS, 4, NORM>), grid, block, 0, s, xp, wp,
                           T, d, K, eps, idx, gate, up);
}

template <bool NORM>
hipError_t launch_router_resident(const void* x, const void* wg, int64_t T, int d, int K,
                                  float eps, int32_t* idx, float* gate, void* u_out,
                                  hipStream_t s) {
    const int tb = T <= 256 ? 1 : d == 8192 ? 2 : 4;
    const int64_t nb = (T + tb - 1) / tb;
    const dim3 grid((unsigned)(nb < 512 ? nb : 512));
    const uint16_t* xp = static_cast<const uint16_t*>(x);
    const uint16_t* wp = static_cast<const uint16_t*>(wg);
    uint16_t* up = static_cast<uint16_t*>(u_out);
    if (d == 2048)
        launch_router_resident_d<8, NORM>(tb, grid, s, xp, wp, T, d, K, eps, idx, gate, up);
    else if (d == 4096)
        launch_router_resident_d<16, NORM>(tb, grid, s, xp, wp, T, d, K, eps, idx, gate, up);
    else
        launch_router_resident_d<32, NORM>(tb == 4 ? 2 : tb, grid, s, xp, wp, T, d, K, eps, idx,
                                           gate, up);
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
