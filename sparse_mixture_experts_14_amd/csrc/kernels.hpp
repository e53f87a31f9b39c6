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
// Gate/up grouped GEMM that stores the pre-activations instead of H:
// AB[p] = [a | b] (bf16, 2 N columns), a = u_p W1_e^T, b = u_p W3_e^T.
hipError_t launch_gemm_bf16_gateup_ab(const uint16_t* A, int64_t A_src_rows, const int32_t* perm,
                                      int K, const uint16_t* B1, const uint16_t* B3,
                                      const int32_t* offsets, int n, int64_t A_rows, int Kdim,
                                      int N, uint16_t* AB, hipStream_t s);
// Per-expert weight gradients C_e[N1][N2] = A_e B_e^T over the expert's
// assignments: A [N1][Kp], B [N2][Kp] bf16, columns in expert order, each
// expert's run zero-padded to a multiple of 64; fp32 out, C_e = C + e N1 N2.
hipError_t launch_gemm_bf16_wgrad(const uint16_t* A, const uint16_t* B, const int32_t* offsets,
                                  int n, int Kp, int N1, int N2, float* C, hipStream_t s);
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

// ---- backward pass (backward.hip) ---------------------------------------------
// H = bf16(SiLU(a) b) from rows [a | b].
hipError_t launch_bwd_h(const uint16_t* AB, int64_t A, int dff, uint16_t* H, hipStream_t s);
// dg[a] = dy_t . O[p], DO[p] = bf16(gate[a] dy_t) for a = perm[p], t = a / K.
hipError_t launch_bwd_gates(const uint16_t* dy, const float* O, const int32_t* perm,
                            const float* gate, int64_t A, int K, int d, float* dg, uint16_t* DO,
                            hipStream_t s);
// [da | db] (bf16) from [a | b] and the fp32 gradient of h.
hipError_t launch_bwd_swiglu(const uint16_t* AB, const float* DH, int64_t A, int dff,
                             uint16_t* DADB, hipStream_t s);
// Router-logit gradient dl[T][n] and dx_t = W_g dl + sum_j DX[inv[t K + j]].
hipError_t launch_bwd_token(const uint16_t* wg, const int32_t* idx, const float* gate,
                            const float* dg, const float* DX, const int32_t* inv, int64_t T,
                            int K, int n, int d, float* dl, uint16_t* dx, hipStream_t s);
// dW_g = sum_t x_t dl_t^T via fixed-order partial sums (part: chunks x d x n).
int bwd_dwg_chunks(int64_t T);
hipError_t launch_bwd_dwg(const uint16_t* x, const float* dl, int64_t T, int d, int n,
                          float* part, float* dwg, hipStream_t s);
// Batched transpose: out[c][ooff + r] = in[r][icol0 + c].
hipError_t launch_transpose(const uint16_t* in, int64_t R, int C, int64_t istride, int icol0,
                            int64_t ibatch, uint16_t* out, int64_t ostride, int64_t ooff,
                            int64_t obatch, int batches, hipStream_t s);
// Expert-padded transpose of assignment rows (optionally gathered through
// perm / K) into out[C][Kp].
hipError_t launch_transpose_pad(const uint16_t* in, int C, int64_t istride, int icol0,
                                const int32_t* offsets, int n, const int32_t* perm, int K,
                                int64_t Kp, uint16_t* out, hipStream_t s);

}  // namespace moe
