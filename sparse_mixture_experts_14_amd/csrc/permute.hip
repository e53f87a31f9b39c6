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
// Workgroups of 16 wavefronts; no atomics, so the result is deterministic.
//   pass 1  wave w counts its contiguous segment of assignments per expert
//           with one ballot per expert per 64 assignments (lane e keeps the
//           count of expert e, n <= 64);
//   scan    expert-major, wave-minor exclusive prefix sum in LDS;
//   pass 2  the wave re-reads its segment; an assignment's position is its
//           expert's running base plus the number of lower lanes holding the
//           same expert in this batch (popcount of the ballot below the lane).
// Few assignments: one workgroup does all of it.  Many (given scratch for
// the per-block counts): a first kernel counts each block of CH assignments
// per expert; in the second, each block forms its experts' bases from the
// counts of the blocks before it (fixed order), then runs the two passes on
// its own block.  Both give the same, stable order.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

constexpr int kPermWaves = 16;

// Lane e of the calling wave: the number of assignments of expert e among
// [beg, end) (0 for e >= n).
__device__ __forceinline__ int32_t count_segment(const int32_t* __restrict__ idx, int64_t beg,
                                                 int64_t end, int n, int lane) {
    int32_t c = 0;
    for (int64_t a0 = beg; a0 < end; a0 += kWave) {
        const int64_t a = a0 + lane;
        const int v = a < end ? idx[a] : -1;
        for (int e = 0; e < n; ++e) {
            const uint64_t m = __ballot(v == e);
            if (lane == e) c += __popcll(m);
        }
    }
    return lane < n ? c : 0;
}

// The per-block counts: block b counts assignments [b CH, (b + 1) CH) per
// expert into bcnt[b][0..n).
__global__ __launch_bounds__(kPermWaves* kWave) void permute_count_kernel(
    const int32_t* __restrict__ idx, int64_t A, int n, int64_t CH, int32_t* __restrict__ bcnt) {
    __shared__ int32_t cnt[kPermWaves][64];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int64_t b0 = (int64_t)blockIdx.x * CH, b1 = min(b0 + CH, A);
    const int64_t per = ((b1 - b0 + kPermWaves - 1) / kPermWaves + kWave - 1) / kWave * kWave;
    const int64_t beg = min(b0 + (int64_t)w * per, b1);
    cnt[w][lane] = count_segment(idx, beg, min(beg + per, b1), n, lane);
    __syncthreads();
    if (threadIdx.x < n) {
        int32_t s = 0;
        for (int ww = 0; ww < kPermWaves; ++ww) s += cnt[ww][threadIdx.x];
        bcnt[(int64_t)blockIdx.x * n + threadIdx.x] = s;
    }
}

// Passes over assignments [b0, b1): with bcnt (nblocks blocks of CH), the
// block's bases come from the counts of the blocks before it; without, the
// single workgroup covers everything.
__global__ __launch_bounds__(kPermWaves* kWave) void permute_kernel(
    const int32_t* __restrict__ idx, int64_t A, int n, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ inv, int32_t* __restrict__ counts,
    int64_t CH, const int32_t* __restrict__ bcnt, int nblocks) {
    __shared__ int32_t cnt[kPermWaves][64];
    __shared__ int32_t base[kPermWaves][64];
    __shared__ int32_t before[64], total[64];
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int64_t b0 = bcnt ? (int64_t)blockIdx.x * CH : 0;
    const int64_t b1 = bcnt ? min(b0 + CH, A) : A;
    // contiguous segment per wave, a multiple of 64 long
    const int64_t per = ((b1 - b0 + kPermWaves - 1) / kPermWaves + kWave - 1) / kWave * kWave;
    const int64_t beg = min(b0 + (int64_t)w * per, b1);
    const int64_t end = min(beg + per, b1);

    cnt[w][lane] = count_segment(idx, beg, end, n, lane);
    if (threadIdx.x < 64) {  // expert e: this block's base among all blocks
        const int e = threadIdx.x;
        int32_t bef = 0, tot = 0;
        if (bcnt && e < n) {
            for (int b = 0; b < nblocks; ++b) {
                const int32_t c = bcnt[(int64_t)b * n + e];
                if (b < (int)blockIdx.x) bef += c;
                tot += c;
            }
        }
        before[e] = bef;
        total[e] = tot;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;  // first row of expert e (over all blocks)
        for (int e = 0; e < n; ++e) {
            int32_t blk = 0;  // this block's assignments of expert e
            for (int ww = 0; ww < kPermWaves; ++ww) blk += cnt[ww][e];
            const int32_t all = bcnt ? total[e] : blk;
            if (blockIdx.x == 0) {
                offsets[e] = run;
                if (counts) counts[e] = all;
            }
            int32_t r = run + before[e];
            for (int ww = 0; ww < kPermWaves; ++ww) {
                base[ww][e] = r;
                r += cnt[ww][e];
            }
            run += all;
        }
        if (blockIdx.x == 0) offsets[n] = run;
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

int permute_blocks(int64_t A) {
    if (A < kPermSplitMin) return 1;
    const int64_t ch = permute_chunk(A);
    return (int)((A + ch - 1) / ch);
}

// counts[e] (+)= offsets[e + 1] - offsets[e]: the per-expert counts of a call
// that runs its tokens in several chunks, summed chunk after chunk in stream
// order (one thread per expert, no atomics).
__global__ void add_counts_kernel(const int32_t* __restrict__ offsets, int n, int first,
                                  int32_t* __restrict__ counts) {
    const int e = threadIdx.x;
    if (e < n) counts[e] = (first ? 0 : counts[e]) + (offsets[e + 1] - offsets[e]);
}

hipError_t launch_add_counts(const int32_t* offsets, int n, bool first, int32_t* counts,
                             hipStream_t s) {
    hipLaunchKernelGGL(add_counts_kernel, dim3(1), dim3(64), 0, s, offsets, n, first ? 1 : 0,
                       counts);
    return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int64_t A, int n, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* counts, hipStream_t s,
                          int32_t* scratch) {
    const int nb = permute_blocks(A);
    if (!scratch || nb <= 1) {
        hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(kPermWaves * kWave), 0, s, idx, A, n,
                           offsets, perm, inv, counts, (int64_t)0, (const int32_t*)nullptr, 1);
        return hipGetLastError();
    }
    const int64_t ch = permute_chunk(A);
    hipLaunchKernelGGL(permute_count_kernel, dim3((unsigned)nb), dim3(kPermWaves * kWave), 0, s,
                       idx, A, n, ch, scratch);
    hipLaunchKernelGGL(permute_kernel, dim3((unsigned)nb), dim3(kPermWaves * kWave), 0, s, idx,
                       A, n, offsets, perm, inv, counts, ch, (const int32_t*)scratch, nb);
    return hipGetLastError();
}

}  // namespace moe
