// Token permutation: a stable counting sort of the T*K (token, slot)
// assignments by expert.
//
// GeekNews summary of "Mixtral of Experts", sections "Cara Komputasi Layer
// MoE" and "Implementasi dan Efisiensi Inferensi": an expert whose gate is 0
// is not evaluated, and the expert FFNs run as one grouped matrix product that
// copes with a different number of tokens per expert.  This stage produces
// that grouping: offsets[e] (first row of expert e), perm[pos] = assignment,
// inv[assignment] = pos.  Within an expert, rows keep assignment order.
//
// One workgroup of 16 wavefronts; no atomics, so the result is deterministic.
//   pass 1  wave w counts its contiguous segment of assignments per expert
//           with one ballot per expert per 64 assignments (lane e keeps the
//           count of expert e, n <= 64);
//   scan    expert-major, wave-minor exclusive prefix sum in LDS;
//   pass 2  the wave re-reads its segment; an assignment's position is its
//           expert's running base plus the number of lower lanes holding the
//           same expert in this batch (popcount of the ballot below the lane).
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kPermWaves = 16;

__global__ __launch_bounds__(kPermWaves* kWave) void permute_kernel(
    const int32_t* __restrict__ idx, int64_t A, int n, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ counts) {
    __shared__ int32_t cnt[kPermWaves][64];
    __shared__ int32_t base[kPermWaves][64];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    // contiguous segment per wave, a multiple of 64 long
    const int64_t per = ((A + kPermWaves - 1) / kPermWaves + kWave - 1) / kWave * kWave;
    const int64_t beg = min((int64_t)w * per, A);
    const int64_t end = min(beg + per, A);

    int32_t c = 0;  // lane e: count of expert e in this segment
    for (int64_t a0 = beg; a0 < end; a0 += kWave) {
        const int64_t a = a0 + lane;
        const int v = a < end ? idx[a] : -1;
        for (int e = 0; e < n; ++e) {
            const uint64_t m = __ballot(v == e);
            if (lane == e) c += __popcll(m);
        }
    }
    if (lane < 64) cnt[w][lane] = lane < n ? c : 0;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;
        for (int e = 0; e < n; ++e) {
            offsets[e] = run;
            const int32_t start = run;
            for (int ww = 0; ww < kPermWaves; ++ww) {
                base[ww][e] = run;
                run += cnt[ww][e];
            }
            if (counts) counts[e] = run - start;
        }
        offsets[n] = run;
    }
    __syncthreads();

    int32_t rb = lane < n ? base[w][lane] : 0;  // lane e: next position of expert e
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t a0 = beg; a0 < end; a0 += kWave) {
        const int64_t a = a0 + lane;
        int v = a < end ? idx[a] : -1;
        const bool valid = v >= 0 && v < n;  // an out-of-range id is dropped, never written
        if (!valid) v = -1;
        uint64_t mine = 0;
        for (int e = 0; e < n; ++e) {
            const uint64_t m = __ballot(v == e);
            if (v == e) mine = m;
            if (lane == e) rb += __popcll(m);
        }
        // base of my expert before this batch: rb of lane v minus this batch's count
        const int vs = valid ? v : 0;
        const int32_t after = __shfl(rb, vs, kWave);
        if (valid) {
            const int32_t pos = after - __popcll(mine) + __popcll(mine & below);
            perm[pos] = (int32_t)a;
            inv[a] = pos;
        }
    }
}

}  // namespace

hipError_t launch_permute(const int32_t* idx, int64_t A, int n, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* counts, hipStream_t s) {
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermWaves * kWave), 0, s, idx, A, n,
                       offsets, perm, inv, counts);
    return hipGetLastError();
}

}  // namespace moe
