// Unpermute and combine: y_t = sum_k gate[t][k] * O[inv[t*K+k]]  (+ x_t).
//
// "Mixtral of Experts", xyznot digest, section "Method (with core equations)":
// the layer output is the gate-weighted sum of the selected experts' outputs.
// GeekNews summary, "Implementasi dan Efisiensi Inferensi": expert outputs go
// back to their tokens' original positions.
//
// One thread per 4 output columns (a workgroup covers 1024 columns of one
// token).  Each token gathers its K expert rows (fp32, possibly split into
// partial sums of the down projection: S for every row, or, after the tiled
// down projection, Sr for the rows from R0 on and one before; partial s >= 1
// of row p at row A + (s - 1)(A - R0) + p - R0) and sums them in a fixed
// order -- partials in split order, then slots in k order -- so the result
// is deterministic and no atomics are needed.  The sum is rounded once into the output dtype (RNE).
// The residual variant adds x_t (fp32) before that single rounding.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

template <typename TOut, bool RESID>
__global__ __launch_bounds__(256) void combine_kernel(
    const float* __restrict__ O, int64_t A, int S, const int32_t* __restrict__ inv,
    const float* __restrict__ gate, int K, int d, const TOut* __restrict__ resid,
    TOut* __restrict__ y, const int* __restrict__ split_meta) {
    const int cb = (d + 1023) / 1024;  // workgroups per token
    const int64_t t = blockIdx.x / cb;
    const int c = (int)(blockIdx.x % cb) * 1024 + threadIdx.x * 4;
    // rows from R0 on hold Sr partial sums, the rows before it one
    const int R0 = split_meta ? split_meta[0] : 0;
    const int Sr = split_meta ? split_meta[1] : S;
    if (c < d) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int k = 0; k < K; ++k) {
            const int64_t pos = inv[t * K + k];
            const float g = gate[t * K + k];
            const float* __restrict__ row = O + pos * (int64_t)d + c;
            float4 o = *reinterpret_cast<const float4*>(row);
            const int np = pos >= R0 ? Sr : 1;
            // partial s >= 1: row A + (s - 1)(A - R0) + pos - R0 (R0 = 0: s A + pos)
            const float* __restrict__ more = O + (A + pos - R0) * (int64_t)d + c;
            for (int s = 1; s < np; ++s) {
                const float4 p = *reinterpret_cast<const float4*>(
                    more + (int64_t)(s - 1) * (A - R0) * d);
                o.x += p.x;
                o.y += p.y;
                o.z += p.z;
                o.w += p.w;
            }
            acc.x = fmaf(g, o.x, acc.x);
            acc.y = fmaf(g, o.y, acc.y);
            acc.z = fmaf(g, o.z, acc.z);
            acc.w = fmaf(g, o.w, acc.w);
        }
        if constexpr (sizeof(TOut) == 2) {
            uint16_t* yp = reinterpret_cast<uint16_t*>(y) + t * (int64_t)d + c;
            if (RESID) {
                const uint2 xv = *reinterpret_cast<const uint2*>(
                    reinterpret_cast<const uint16_t*>(resid) + t * (int64_t)d + c);
                acc.x += __uint_as_float(xv.x << 16);
                acc.y += __uint_as_float(xv.x & 0xffff0000u);
                acc.z += __uint_as_float(xv.y << 16);
                acc.w += __uint_as_float(xv.y & 0xffff0000u);
            }
            uint2 out;
            out.x = pack_bf16x2(acc.x, acc.y);
            out.y = pack_bf16x2(acc.z, acc.w);
            *reinterpret_cast<uint2*>(yp) = out;
        } else {
            float* yp = reinterpret_cast<float*>(y) + t * (int64_t)d + c;
            if (RESID) {
                const float4 xv = *reinterpret_cast<const float4*>(
                    reinterpret_cast<const float*>(resid) + t * (int64_t)d + c);
                acc.x += xv.x;
                acc.y += xv.y;
                acc.z += xv.z;
                acc.w += xv.w;
            }
            *reinterpret_cast<float4*>(yp) = acc;
        }
    }
}

}  // namespace

hipError_t launch_combine(bool bf16, bool resid, const float* O, int64_t A, int S,
                          const int32_t* inv, const float* gate, int64_t T, int K, int d,
                          const void* x, void* y, const int* split_meta, hipStream_t s) {
    const int64_t cb = (d + 1023) / 1024;
    if (T * cb > 0x7fffffff) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)(T * cb));
    const dim3 block(256);
    if (bf16) {
        if (resid)
            hipLaunchKernelGGL((combine_kernel<uint16_t, true>), grid, block, 0, s, O, A, S,
                               inv, gate, K, d, static_cast<const uint16_t*>(x),
                               static_cast<uint16_t*>(y), split_meta);
        else
            hipLaunchKernelGGL((combine_kernel<uint16_t, false>), grid, block, 0, s, O, A,
                               S, inv, gate, K, d, static_cast<const uint16_t*>(x),
                               static_cast<uint16_t*>(y), split_meta);
    } else {
        if (resid)
            hipLaunchKernelGGL((combine_kernel<float, true>), grid, block, 0, s, O, A, S,
                               inv, gate, K, d, static_cast<const float*>(x),
                               static_cast<float*>(y), split_meta);
        else
            hipLaunchKernelGGL((combine_kernel<float, false>), grid, block, 0, s, O, A, S,
                               inv, gate, K, d, static_cast<const float*>(x),
                               static_cast<float*>(y), split_meta);
    }
    return hipGetLastError();
}

}  // namespace moe
