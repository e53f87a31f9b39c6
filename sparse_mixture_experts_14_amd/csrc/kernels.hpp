// Host-side launchers of the gfx950 kernels (internal to libmoe.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Router (+ optional fused pre-normalisation writing u_out).
hipError_t launch_router(bool bf16, bool norm, const void* x, const void* wg, int64_t T,
                         int d, int n, int K, float eps, int32_t* idx, float* gate,
                         void* u_out, hipStream_t s);

// Stable counting sort of A = T*K assignments by expert.
hipError_t launch_permute(const int32_t* idx, int64_t A, int n, int32_t* offsets,
                          int32_t* perm, int32_t* inv, int32_t* counts, hipStream_t s);

// fp32 grouped GEMMs (gate/up with SiLU*mul epilogue, or down).
hipError_t launch_gemm_f32(bool gateup, const float* A, const int32_t* perm, int K,
                           const float* B1, const float* B3, const int32_t* offsets, int n,
                           int64_t A_rows, int Kdim, int N, float* C, hipStream_t s);

// bf16 MFMA grouped GEMMs, LDS-tiled (many rows per expert).  A has
// A_src_rows rows of Kdim elements (x, u or H).
// The down projection (gateup false) may split K into `splits` partial sums,
// written `A_rows * N` elements apart; gate/up takes splits = 1.
hipError_t launch_gemm_bf16_tiled(bool gateup, const uint16_t* A, int64_t A_src_rows,
                                  const int32_t* perm, int K, const uint16_t* B1,
                                  const uint16_t* B3, const int32_t* offsets, int n,
                                  int64_t A_rows, int Kdim, int N, void* C, int splits,
                                  hipStream_t s);
// K splits worth using for the tiled down projection on `cus` compute units
// (at most min(max_splits, 4)): the count that minimises tile rounds per split
// plus the cost of the extra fp32 partial sums.  Depends on sizes only.
int tiled_down_splits(int64_t A_rows, int n, int N, int Kdim, int cus, int max_splits);
// Whether the tiled kernels can take these sizes (32-bit buffer offsets).
bool tiled_fits(int64_t A_src_rows, int64_t Kdim, int64_t N);

// bf16 MFMA grouped GEMMs streaming weights (few rows per expert), one
// persistent workgroup of `waves` (7 or 8) waves per CU (`cus` of them).
// The down projection may split K into partial sums; skinny_splits_used()
// tells how many splits a request of `splits` really produces.
hipError_t launch_gemm_bf16_skinny(bool gateup, const uint16_t* A, int64_t A_src_rows,
                                   const int32_t* perm, int K, const uint16_t* B1,
                                   const uint16_t* B3, const int32_t* offsets, int n,
                                   int64_t A_rows, int Kdim, int N, void* C, int splits,
                                   int waves, int cus, hipStream_t s);
// Whether the skinny kernels can take these sizes (row table in LDS, 32-bit
// buffer offsets).
bool skinny_fits(int64_t A_src_rows, int64_t A_rows, int64_t Kdim, int64_t N, int splits);
int skinny_splits_used(int Kdim, int splits);

// y = sum_k gate * (sum over S splits of O) (+ x), rounded once.
hipError_t launch_combine(bool bf16, bool resid, const float* O, int64_t A, int S,
                          const int32_t* inv, const float* gate, int64_t T, int K, int d,
                          const void* x, void* y, hipStream_t s);

}  // namespace moe
