// Device-side helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace moe {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even fp32 -> bf16 (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack_bf16x8(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x << 16);
    f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16);
    f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16);
    f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16);
    f[7] = __uint_as_float(v.w & 0xffff0000u);
}

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t& v) {
    return __builtin_bit_cast(bf16x8_t, v);
}

// SiLU(z) = z / (1 + e^-z) (Swish with beta = 1).
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Same function with the hardware exp2 and reciprocal (a few ulp of fp32),
// for results that are rounded to bf16 (8 mantissa bits) right after.
__device__ __forceinline__ float silu_bf16out(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Sum over the 64 lanes of a wavefront.  Butterfly order: every lane ends with
// the bitwise-identical total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

// Find which expert a tile of BM rows belongs to.  offsets[0..n] are the
// per-expert row offsets; tile t counts tiles expert by expert.  Returns
// false when t is past the last tile.
template <int BM>
__device__ __forceinline__ bool locate_tile(const int32_t* __restrict__ offsets, int n,
                                            int t, int& expert, int& row0, int& rows) {
    int start = offsets[0];
    for (int e = 0; e < n; ++e) {
        const int end = offsets[e + 1];
        const int m = end - start;
        const int tiles = (m + BM - 1) / BM;
        if (t < tiles) {
            expert = e;
            row0 = start + t * BM;
            rows = min(BM, end - row0);
            return true;
        }
        t -= tiles;
        start = end;
    }
    return false;
}

}  // namespace moe
