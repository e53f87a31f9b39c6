// Grouped expert GEMMs for few rows per expert (decode): a weight stream.
//
// Same products as the tiled kernels (xyznot digest of "Mixtral of Experts",
// "Method" section: SwiGLU_e(u) = W2_e (SiLU(W1_e u) (*) W3_e u)), but with a
// handful of tokens per expert the layer is bound by reading the touched
// experts' weights from HBM once.  Each wavefront streams 16-column slices of
// the weight matrices straight from global memory into MFMA B operands
// (v_mfma_f32_16x16x32_bf16; the token rows, zero-padded to 16, are the A
// operand and come from L2), so no LDS round trip sits on the weight path.
//
// K permutation: in one step a lane loads 4 consecutive 16-byte chunks (64
// contiguous bytes) of its weight row; MFMA sub-step c uses chunk c.  Lane
// group g = lane/16 covers k in [k0 + 32g, k0 + 32g + 32), the A operand is
// loaded with the same k map, so the products are unchanged while each row
// is read in 64-byte runs.  The next step's loads are issued before the
// current step's MFMAs (register double buffering).
//
// An expert with no rows exits at once and reads no weights (the pages: an
// expert whose gate is 0 need not be computed).  Down projection: blockIdx.z
// splits K; split s writes its partial sums to O + s * A_rows * N and the
// combine stage adds the splits in order (deterministic, no atomics).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int KSTEP = 128;  // k per step: 4 lane groups x 32

template <bool GATEUP, int NT>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const uint16_t* __restrict__ A, const int32_t* __restrict__ perm, int K,
    const uint16_t* __restrict__ B1, const uint16_t* __restrict__ B3,
    const int32_t* __restrict__ offsets, int Kdim, int N, void* __restrict__ Cout,
    int ksplit, int64_t A_rows) {
    constexpr int CW = GATEUP ? NT / 2 * 16 : NT * 16;  // output columns per wave
    const int e = blockIdx.y;
    const int start = offsets[e];
    const int M = offsets[e + 1] - start;
    if (M <= 0) return;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int col0 = (blockIdx.x * (blockDim.x / kWave) + w) * CW;
    if (col0 >= N) return;
    const int kbeg = blockIdx.z * ksplit;
    const int kend = min(Kdim, kbeg + ksplit);

    const int j = lane & 15, g = lane >> 4;
    const uint16_t* b_ptr[NT];
    bool b_ok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        int col;
        const uint16_t* base;
        if (GATEUP) {
            col = col0 + (t < NT / 2 ? t : t - NT / 2) * 16 + j;
            base = t < NT / 2 ? B1 : B3;
        } else {
            col = col0 + t * 16 + j;
            base = B1;
        }
        b_ok[t] = col < N;
        b_ptr[t] = base + ((int64_t)e * N + (b_ok[t] ? col : 0)) * Kdim + g * 32;
    }

    for (int m0 = 0; m0 < M; m0 += 16) {
        const int i = lane & 15;
        const bool a_ok = m0 + i < M;
        const int p = start + m0 + (a_ok ? i : 0);
        const int64_t src = GATEUP ? (int64_t)(perm[p] / K) : (int64_t)p;
        const uint16_t* a_ptr = A + src * Kdim + g * 32;

        f32x4_t acc[NT];
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        uint4 av0[4], bv0[NT][4], av1[4], bv1[NT][4];
        auto load = [&](uint4(&av)[4], uint4(&bv)[NT][4], int k0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const bool k_ok = k0 + g * 32 + c * 8 < kend;
                av[c] = (a_ok && k_ok) ? *reinterpret_cast<const uint4*>(a_ptr + k0 + c * 8)
                                       : make_uint4(0, 0, 0, 0);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    bv[t][c] = (b_ok[t] && k_ok)
                                   ? *reinterpret_cast<const uint4*>(b_ptr[t] + k0 + c * 8)
                                   : make_uint4(0, 0, 0, 0);
            }
        };
        auto compute = [&](const uint4(&av)[4], const uint4(&bv)[NT][4]) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        as_bf16x8(av[c]), as_bf16x8(bv[t][c]), acc[t], 0, 0, 0);
        };

        // two named register buffers, alternating, so every index is static
        int k0 = kbeg;
        load(av0, bv0, k0);
        while (true) {
            const bool more0 = k0 + KSTEP < kend;
            if (more0) load(av1, bv1, k0 + KSTEP);
            compute(av0, bv0);
            if (!more0) break;
            k0 += KSTEP;
            const bool more1 = k0 + KSTEP < kend;
            if (more1) load(av0, bv0, k0 + KSTEP);
            compute(av1, bv1);
            if (!more1) break;
            k0 += KSTEP;
        }

        // 16x16 accumulator layout: lane l, register r holds row 4*(l/16) + r
        // and column l%16 of the tile.
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 4 * g + r;
            if (m0 + row >= M) continue;
            const int64_t orow = (int64_t)(start + m0 + row) * N;
            if (GATEUP) {
                uint16_t* H = static_cast<uint16_t*>(Cout);
#pragma unroll
                for (int t = 0; t < NT / 2; ++t) {
                    const int col = col0 + t * 16 + j;
                    if (col < N)
                        H[orow + col] = f32_to_bf16_bits(silu(acc[t][r]) * acc[t + NT / 2][r]);
                }
            } else {
                float* O = static_cast<float*>(Cout) + (int64_t)blockIdx.z * A_rows * N;
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const int col = col0 + t * 16 + j;
                    if (col < N) O[orow + col] = acc[t][r];
                }
            }
        }
    }
}

int split_len(int Kdim, int splits) {
    return ((Kdim + splits - 1) / splits + KSTEP - 1) / KSTEP * KSTEP;
}

template <bool GATEUP, int NT>
hipError_t launch_skinny_t(const uint16_t* A, const int32_t* perm, int K, const uint16_t* B1,
                           const uint16_t* B3, const int32_t* offsets, int n, int64_t A_rows,
                           int Kdim, int N, void* C, int splits, hipStream_t s) {
    constexpr int CW = GATEUP ? NT / 2 * 16 : NT * 16;
    const int waves = 4;
    const int ksplit = split_len(Kdim, splits);
    const int zs = (Kdim + ksplit - 1) / ksplit;
    const dim3 grid((unsigned)((N + waves * CW - 1) / (waves * CW)), (unsigned)n, (unsigned)zs);
    hipLaunchKernelGGL((gemm_skinny_kernel<GATEUP, NT>), grid, dim3(waves * kWave), 0, s, A,
                       perm, K, B1, B3, offsets, Kdim, N, C, ksplit, A_rows);
    return hipGetLastError();
}

}  // namespace

int skinny_splits_used(int Kdim, int splits) {
    const int ksplit = split_len(Kdim, splits);
    return (Kdim + ksplit - 1) / ksplit;
}

hipError_t launch_gemm_bf16_skinny(bool gateup, const uint16_t* A, const int32_t* perm, int K,
                                   const uint16_t* B1, const uint16_t* B3,
                                   const int32_t* offsets, int n, int64_t A_rows, int Kdim,
                                   int N, void* C, int splits, hipStream_t s) {
    if (gateup)
        return launch_skinny_t<true, 2>(A, perm, K, B1, B3, offsets, n, A_rows, Kdim, N, C, 1,
                                        s);
    return launch_skinny_t<false, 2>(A, perm, K, B1, B3, offsets, n, A_rows, Kdim, N, C,
                                     splits, s);
}

}  // namespace moe
