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
                          int32_t* perm, int32_t* inv, int32_t* counts, hipStream_t s,
                          int32_t* scratch = nullptr);
// Many assignments run over several workgroups (blocks of permute_chunk(A)
// assignments) when launch_permute gets scratch for permute_blocks(A) * n
// per-block counts; fewer than kPermSplitMin stay in one workgroup.
constexpr int64_t kPermSplitMin = 4096;
constexpr int kPermMaxBlocks = 1024;
inline int64_t permute_chunk(int64_t A) {  // a multiple of 1024, at most kPermMaxBlocks blocks
    const int64_t c = (A + kPermMaxBlocks - 1) / kPermMaxBlocks;
    return c <= 1024 ? 1024 : (c + 1023) / 1024 * 1024;
}
int permute_blocks(int64_t A);

// fp32 grouped GEMMs (gate/up with SiLU*mul epilogue, or down).
hipError_t launch_gemm_f32(bool gateup, const float* A, const int32_t* perm, int K,
                           const float* B1, const float* B3, const int32_t* offsets, int n,
                           int64_t A_rows, int Kdim, int N, float* C, hipStream_t s);

// bf16 MFMA grouped GEMMs, LDS-tiled (many rows per expert).  A has
// A_src_rows rows of Kdim elements (x, u or H).
// The down projection (gateup false) splits the K range of its last round's
// tiles (the rows from R0 on) into Sr <= `splits` partial sums, written
// `A_rows * N` elements apart (buffer 0 holds every row's first or only
// sum); it writes (R0, Sr) to split_meta[0..1] for the combine.  `cus` is
// the CU count of the device.  Gate/up takes splits = 1 and no split_meta.
hipError_t launch_gemm_bf16_tiled(bool gateup, const uint16_t* A, int64_t A_src_rows,
                                  const int32_t* perm, int K, const uint16_t* B1,
                                  const uint16_t* B3, const int32_t* offsets, int n,
                                  int64_t A_rows, int Kdim, int N, void* C, int splits,
                                  int cus, int* split_meta, hipStream_t s);
// Gate/up grouped GEMM that stores the pre-activations instead of H:
// AB[p] = [a | b] (bf16, 2 N columns), a = u_p W1_e^T, b = u_p W3_e^T.
hipError_t launch_gemm_bf16_gateup_ab(const uint16_t* A, int64_t A_src_rows, const int32_t* perm,
                                      int K, const uint16_t* B1, const uint16_t* B3,
                                      const int32_t* offsets, int n, int64_t A_rows, int Kdim,
                                      int N, uint16_t* AB, hipStream_t s);
// Gate/up grouped GEMM that stores both H (as launch_gemm_bf16_tiled) and the
// pre-activation rows AB[p] = [a | b] (bf16, 2 N columns).
hipError_t launch_gemm_bf16_gateup_save(const uint16_t* A, int64_t A_src_rows,
                                        const int32_t* perm, int K, const uint16_t* B1,
                                        const uint16_t* B3, const int32_t* offsets, int n,
                                        int64_t A_rows, int Kdim, int N, uint16_t* H,
                                        uint16_t* AB, hipStream_t s);
// Per-expert weight gradients C_e[r][c] = sum over the expert's rows p of
// A[p][r] B[p][c] (A, B bf16 in expert order, row strides a_stride,
// b_stride); fp32 out, C_e = C + e N1 N2, zero for an expert without rows.
hipError_t launch_gemm_bf16_wgrad(const uint16_t* A, int64_t a_stride, const uint16_t* B,
                                  int64_t b_stride, const int32_t* offsets, int n,
                                  int64_t A_rows, int N1, int N2, float* C, int GM,
                                  hipStream_t s);
// C[s][p][c] (row stride N, split stride A_rows N) = sum over the K range
// of split s of A[p][k] W_e[k][c], over the rows p of each expert e, with
// K-row weights: W_e = B1 + e b_split N for k < b_split and B3 + e b_split N
// (row k - b_split) beyond (B3 NULL: Kdim = b_split).  C is fp32, or bf16
// (rounded once) when bf16_out, which allows one split only.  With
// split_meta (fp32 only), only the last round's tiles -- the rows from R0 on
// -- take Sr <= splits K splits, as in the tiled down projection, and
// (R0, Sr) go to split_meta; without it every tile takes `splits`.
hipError_t launch_gemm_bf16_krow(const uint16_t* A, int64_t A_rows, const uint16_t* B1,
                                 const uint16_t* B3, int b_split, const int32_t* offsets, int n,
                                 int Kdim, int N, void* C, bool bf16_out, int splits, int cus,
                                 int* split_meta, hipStream_t s);
// Weight-stream variant of launch_gemm_bf16_krow for few rows per expert:
// fp32 partial sums C[s][p][c] (split stride A_rows N) over `splits` K
// ranges (krow_stream_splits_used() tells how many a request produces),
// one persistent workgroup of `waves` (7 or 8) waves on each of `cus` CUs.
int krow_stream_splits_used(int Kdim, int splits);
hipError_t launch_gemm_bf16_krow_stream(const uint16_t* A, int64_t A_rows, const uint16_t* B1,
                                        const uint16_t* B3, int b_split,
                                        const int32_t* offsets, int n, int Kdim, int N,
                                        float* C, int splits, int waves, int cus,
                                        hipStream_t s);
// Whether the tiled kernels can take these sizes (32-bit buffer offsets).
bool tiled_fits(int64_t A_src_rows, int64_t Kdim, int64_t N);

// bf16 MFMA grouped GEMMs streaming weights (few rows per expert), one
// persistent workgroup of `waves` (7 or 8) waves per CU (`cus` of them).
// The down projection may split K into partial sums; skinny_splits_used()
// tells how many splits a request of `splits` really produces.  AB (gate/up
// only, may be NULL): also store the pre-activation rows [a | b] (bf16, 2 N
// columns); C may then be NULL to skip H.
hipError_t launch_gemm_bf16_skinny(bool gateup, const uint16_t* A, int64_t A_src_rows,
                                   const int32_t* perm, int K, const uint16_t* B1,
                                   const uint16_t* B3, const int32_t* offsets, int n,
                                   int64_t A_rows, int Kdim, int N, void* C, int splits,
                                   int waves, int cus, hipStream_t s, uint16_t* AB = nullptr);
// Whether the skinny kernels can take these sizes (row table in LDS, 32-bit
// buffer offsets).
bool skinny_fits(int64_t A_src_rows, int64_t A_rows, int64_t Kdim, int64_t N, int splits);
int skinny_splits_used(int Kdim, int splits);

// y = sum_k gate * (sum over S splits of O) (+ x), rounded once.  With
// split_meta (R0, Sr) from the tiled down projection, rows >= R0 hold Sr
// partial sums and the others one; without it every row holds S.
hipError_t launch_combine(bool bf16, bool resid, const float* O, int64_t A, int S,
                          const int32_t* inv, const float* gate, int64_t T, int K, int d,
                          const void* x, void* y, const int* split_meta, hipStream_t s);

// ---- backward pass (backward.hip) ---------------------------------------------
// Per assignment row p (a = perm[p]) from [a | b] = AB[p] and the bf16
// gradient DH[p] of h with respect to the ungated expert output (W2_e^T dy):
// dg[a] = h . DH[p] (h = bf16(SiLU(a) b)), DADB[p] = [da | db] of the gated
// gradient gate[a] DH[p], GH[p] = bf16(gate[a] h).
// DHP (instead of DH, may be NULL): r as S fp32 K-split partial sums
// [S][A][dff], added in split order.
hipError_t launch_bwd_swiglu(const uint16_t* AB, const uint16_t* DH, const float* DHP, int S,
                             const int32_t* perm, const float* gate, int64_t A, int dff,
                             float* dg, uint16_t* DADB, uint16_t* GH, hipStream_t s);
// Router-logit gradient dl[T][n] and dx_t = W_g dl + sum_j sum_s
// DX[s][inv[t K + j]] (K-split partials, split stride A d: S for every row,
// or with split_meta (R0, Sr) Sr for rows >= R0 and one below): bf16 dx, or
// fp32 dx32 when that is given.
hipError_t launch_bwd_token(const uint16_t* wg, const int32_t* idx, const float* gate,
                            const float* dg, const float* DX, int S, int64_t A,
                            const int32_t* inv, int64_t T, int K, int n, int d, float* dl,
                            uint16_t* dx, float* dx32, const int* split_meta, hipStream_t s);
// Stack layer: dx = dy + s (du - u (u . du) / d) per token (u = x s,
// s = 1 / sqrt(mean(x^2) + eps)); scale[t] = s.
hipError_t launch_bwd_rms(const uint16_t* x, const uint16_t* dy, const float* du, int64_t T,
                          int d, float eps, uint16_t* dx, float* scale, hipStream_t s);
// dW_g = sum_t (x_t scale_t) dl_t^T (scale nullable: 1) via fixed-order
// partial sums (part: chunks x d x n).
int bwd_dwg_chunks(int64_t T);
hipError_t launch_bwd_dwg(const uint16_t* x, const float* scale, const float* dl, int64_t T,
                          int d, int n, float* part, float* dwg, hipStream_t s);
// Zero `bytes` (a multiple of 16) at p with a kernel.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// counts[e] = offsets[e + 1] - offsets[e] (first) or counts[e] += that (n <= 64).
hipError_t launch_add_counts(const int32_t* offsets, int n, bool first, int32_t* counts,
                             hipStream_t s);
// XG[p] = x[perm[p] / K] and YG[p] = y[perm[p] / K] (bf16 rows of d
// elements), p < A.
hipError_t launch_gather_rows(const uint16_t* x, const uint16_t* y, const int32_t* perm, int K,
                              int64_t A, int d, uint16_t* XG, uint16_t* YG, hipStream_t s);

}  // namespace moe
