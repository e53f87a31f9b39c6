/*
 * moe.h -- C ABI of libmoe.so, a gfx950 (MI355X) implementation of the sparse
 * top-K mixture-of-experts feed-forward layer of "Mixtral of Experts"
 * (arXiv 2401.04088).
 *
 * What the layer computes (xyznot digest of the paper, section "Method (with
 * core equations)"; GeekNews summary, section "Cara Komputasi Layer MoE"):
 *
 *   l    = x . W_g                       router logits, one per expert (n of them)
 *   G(x) = Softmax(TopK(l))              TopK keeps the K largest logits and sets
 *                                        the others to -inf, so the softmax runs
 *                                        over the K kept logits only
 *   y    = sum_i G(x)_i * SwiGLU_i(x)    experts with a zero gate are not run
 *   SwiGLU_i(u) = W2_i (SiLU(W1_i u) (*) W3_i u),  SiLU(z) = z / (1 + e^-z)
 *
 * Readings this library fixes where the pages are silent:
 *   - exactly K experts are kept; among equal logits the lower index ranks
 *     first; slot 0 of a token's (idx, gate) pair holds the largest logit;
 *   - router logits are accumulated in fp32 and never rounded to bf16;
 *   - bf16 path: products accumulate in fp32; the SwiGLU hidden activation is
 *     rounded to bf16 before the down projection; expert outputs stay fp32
 *     until the gate-weighted sum, which is rounded once (RNE) into y.
 *
 * Layouts (all row-major, contiguous, device memory, 16-byte aligned):
 *   x    [T][d]           activations (dtype dt)
 *   W_g  [d][n]           router weight; column i belongs to expert i
 *   W1   [n][d_ff][d]     gate projection (SiLU branch), [out][in]
 *   W3   [n][d_ff][d]     up projection, [out][in]
 *   W2   [n][d][d_ff]     down projection, [out][in]
 *   y    [T][d]           output (dtype dt)
 *   idx  [T][K] int32, gate [T][K] float
 *
 * Ownership and side effects: every pointer is owned by the caller.  Inputs
 * are never written.  y is fully overwritten and must not overlap any input
 * or the workspace.  The library keeps no pointer after a call returns and
 * never allocates device memory; scratch space comes from the caller's
 * workspace, whose contents are undefined afterwards.
 *
 * Streams: all work is enqueued on `stream` (a hipStream_t; NULL = the null
 * stream).  No call synchronises the host with the device.
 *
 * Errors: arguments are validated before anything is enqueued, so a call that
 * returns an error other than MOE_ERR_HIP has had no effect.  MOE_ERR_HIP
 * reports a launch failure (hipGetLastError); a fault inside a kernel shows
 * up at the caller's next synchronisation instead.  No C++ exception crosses
 * this boundary.  moe_last_error() returns a thread-local description of the
 * most recent failure on the calling thread.
 *
 * Supported on the GPU: 1 <= n <= 64, 1 <= K <= min(n, 8), d and d_ff
 * multiples of 8, T * K < 2^31, dtype MOE_F32 or MOE_BF16.  T = 0 is a no-op
 * that returns MOE_OK.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1, /* null/misaligned pointer, bad size, aliasing */
    MOE_ERR_UNSUPPORTED = 2,      /* valid layer, but outside what the GPU path supports */
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_HIP = 4,              /* a HIP runtime call or launch failed */
    /* range markers, not statuses: every int32 value is a valid moe_status_t
     * (a C caller may pass any int to moe_status_string) */
    MOE_STATUS_MIN_ENUM_ = -0x7fffffff - 1,
    MOE_STATUS_MAX_ENUM_ = 0x7fffffff
} moe_status_t;

typedef enum moe_dtype {
    MOE_F32 = 0,  /* fp32 storage, fp32 arithmetic */
    MOE_BF16 = 1, /* bf16 storage, fp32 accumulation */
    /* range markers, not dtypes: any int32 a caller passes is a valid
     * moe_dtype_t value, which the calls then reject unless it is one of the
     * two above */
    MOE_DTYPE_MIN_ENUM_ = -0x7fffffff - 1,
    MOE_DTYPE_MAX_ENUM_ = 0x7fffffff
} moe_dtype_t;

/* Stages of moe_forward / moe_block_forward and of moe_backward, in launch
 * order. */
typedef enum moe_stage {
    MOE_STAGE_ROUTER = 0,   /* logits, TopK, softmax (and RMSNorm in the block layer) */
    MOE_STAGE_PERMUTE = 1,  /* per-expert grouping of the assignments */
    MOE_STAGE_GATE_UP = 2,  /* H = SiLU(u W1^T) * (u W3^T), grouped by expert */
    MOE_STAGE_DOWN = 3,     /* O = H W2^T, grouped by expert */
    MOE_STAGE_COMBINE = 4,  /* y = sum_k gate * O (+ x), back in token order */
    /* stages of moe_backward */
    MOE_STAGE_BWD_RECOMPUTE = 5, /* routing, [a | b] = u [W1 ; W3]^T, h, expert outputs */
    MOE_STAGE_BWD_DH = 6,   /* dg, g dy, dh = (g dy) W2, SwiGLU backward */
    MOE_STAGE_BWD_DX = 7,   /* dx, router gradient, dW_g, tokens gathered per expert */
    MOE_STAGE_BWD_WGRAD = 8 /* the three weight-gradient products dW2, dW1, dW3 */
} moe_stage_t;

/* Version of this ABI (MOE_ABI_VERSION of the library that was built). */
int32_t moe_abi_version(void);

/* Router only: the gating equation of the "Method" section.  Writes, for
 * every token t, idx[t][0..K) (experts in rank order: largest logit first,
 * ties to the lower index) and gate[t][0..K) (softmax over the K kept logits,
 * each >= 0, summing to 1).  Needs no workspace. */
moe_status_t moe_route(const void* x, const void* w_g, int64_t T, int64_t d,
                       int32_t n, int32_t K, moe_dtype_t dt, int32_t* idx,
                       float* gate, void* stream);

/* Token permutation.  Only the K experts a token keeps have a non-zero gate,
 * so only they need to run for it (GeekNews summary, section "Cara Komputasi
 * Layer MoE"); each expert therefore gets the contiguous list of the
 * assignments routed to it.
 * Input idx[T][K]; assignment a = t*K + k goes to expert idx[a].  Output:
 *   offsets[n+1]  offsets[e] = first position of expert e, offsets[n] = T*K
 *   perm[T*K]     perm[pos] = a, positions of one expert in increasing a
 *                 (a stable counting sort by expert)
 *   inv[T*K]      inv[a] = pos (the inverse of perm)
 * Every idx entry must lie in [0, n); the result is unspecified otherwise. */
moe_status_t moe_permute(const int32_t* idx, int64_t T, int32_t n, int32_t K,
                         int32_t* offsets, int32_t* perm, int32_t* inv,
                         void* stream);

/* Bytes of workspace that moe_forward and moe_block_forward need for these
 * sizes.  An upper bound that does not depend on how tokens get routed.  For
 * bf16 calls larger than one pass (see moe_forward) it is the workspace of one
 * chunk, so it stops growing with T.  Returns 0 if the sizes are invalid. */
size_t moe_workspace_bytes(int64_t T, int64_t d, int64_t d_ff, int32_t n,
                           int32_t K, moe_dtype_t dt);

/* The whole layer, y = sum_i G(x)_i SwiGLU_i(x) (output equation of the
 * "Method" section).  workspace: device memory of at least
 * moe_workspace_bytes(...) bytes, 256-byte aligned.  Optional outputs (NULL to
 * skip): idx_out[T][K], gate_out[T][K] -- the routing that was used -- and
 * counts_out[n], the number of assignments each expert received.  The
 * workspace must not overlap any other argument.
 *
 * The kernels index one pass's operands with 32-bit offsets: bf16 needs
 * T * d and T * K * d_ff below 2^30 elements (T <= 37449 at d = 4096,
 * d_ff = 14336, K = 2), fp32 needs T * K < 64 (65535 - n).  A call with more
 * tokens runs them in the fewest near-equal chunks that fit, one after the
 * other on `stream`, each chunk a whole layer pass over its own tokens (every
 * token is routed and computed on its own, so y, idx_out and gate_out equal
 * those of separate calls on the chunks; counts_out is their sum).  The
 * expert weights themselves must fit (bf16: d * d_ff < 2^30 per expert),
 * else MOE_ERR_UNSUPPORTED.  Stage events (moe_set_stage_events) then mark
 * the last chunk. */
moe_status_t moe_forward(const void* x, const void* w_g, const void* w1,
                         const void* w3, const void* w2, int64_t T, int64_t d,
                         int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt,
                         void* y, void* workspace, size_t workspace_bytes,
                         int32_t* idx_out, float* gate_out, int32_t* counts_out,
                         void* stream);

/* moe_forward without a workspace, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation).  The layer's scratch lives in a static device array of
 * the library, 64 MiB per device (held from the first call on a device until
 * the process ends): enough for T <= 256 tokens at d = 4096, d_ff = 14336,
 * n = 8, K = 2.  Larger sizes (moe_workspace_bytes(...) > 64 MiB) return
 * MOE_ERR_UNSUPPORTED before anything is enqueued.  No device memory is
 * allocated or freed.  All calls on one device share that device's array, so
 * calls that may overlap in time on one device (different streams, or
 * different host threads) race and give undefined results; serialise them,
 * e.g. on one stream.  Same arguments, outputs and rules as moe_forward
 * otherwise; y is bitwise equal to moe_forward's. */
moe_status_t moe_forward_noalloc(const void* x, const void* w_g, const void* w1,
                                 const void* w3, const void* w2, int64_t T, int64_t d,
                                 int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt,
                                 void* y, int32_t* idx_out, float* gate_out,
                                 int32_t* counts_out, void* stream);

/* One layer of a pre-normalised residual stack (the MoE replaces every
 * feed-forward sub-block, "Core ideas" of the xyznot digest; the
 * normalisation and residual are this workload's definition, not the
 * pages'):
 *   u = x / sqrt(mean(x^2) + eps)   (unit weight; routing uses u in fp32)
 *   y = x + MoE(u)                  (residual added in fp32, rounded once)
 * Same arguments and outputs as moe_forward plus eps (>= 0). */
moe_status_t moe_block_forward(const void* x, const void* w_g, const void* w1,
                               const void* w3, const void* w2, int64_t T,
                               int64_t d, int64_t d_ff, int32_t n, int32_t K,
                               moe_dtype_t dt, float eps, void* y, void* workspace,
                               size_t workspace_bytes, int32_t* idx_out,
                               float* gate_out, int32_t* counts_out,
                               void* stream);

/* Bytes of workspace that moe_backward needs for these sizes (an upper bound
 * that does not depend on the routing).  Returns 0 if the sizes are invalid
 * or dt is not MOE_BF16. */
size_t moe_backward_workspace_bytes(int64_t T, int64_t d, int64_t d_ff,
                                    int32_t n, int32_t K, moe_dtype_t dt);

/* Backward pass of the layer of moe_forward: the gradients of the scalar
 * L = sum_t dy_t . y_t with respect to every input, differentiating the gate
 * and output equations of the "Method" section.  TopK is piecewise constant,
 * so only the K kept logits of a token receive a gradient, through the
 * softmax over them:
 *   dg_j = dy . SwiGLU_{s_j}(x),  dl_{s_j} = g_j (dg_j - sum_k g_k dg_k).
 * The routing is recomputed from (x, W_g) exactly as moe_forward computes it.
 * Inputs x, W_g, W1, W3, W2 as in moe_forward and dy [T][d] (all MOE_BF16).
 * Outputs (overwritten, none may overlap an input, another output or the
 * workspace):
 *   dx   [T][d]         bf16, fp32 sums rounded once (RNE)
 *   dw_g [d][n]         float
 *   dw1, dw3 [n][d_ff][d], dw2 [n][d][d_ff]   float
 * Arithmetic: fp32 accumulation; the recomputed pre-activations, the hidden
 * activation, g dy and the SwiGLU input gradients are rounded to bf16 before
 * the products that consume them.  workspace: at least
 * moe_backward_workspace_bytes(...) bytes, 256-byte aligned.  dt = MOE_F32
 * returns MOE_ERR_UNSUPPORTED.  One pass only: T * d, T * K * 2 d_ff and the
 * expert weights must stay below 2^30 elements (T <= 18724 at d = 4096,
 * d_ff = 14336, K = 2), else MOE_ERR_UNSUPPORTED; larger batches are split by
 * the caller, who sums the weight gradients.  T = 0 zeroes the weight
 * gradients (x, dy and dx may then be NULL).  Weight gradients are cleared with kernels, never a
 * memset, so the call can be captured into a HIP graph. */
moe_status_t moe_backward(const void* x, const void* w_g, const void* w1,
                          const void* w3, const void* w2, const void* dy,
                          int64_t T, int64_t d, int64_t d_ff, int32_t n,
                          int32_t K, moe_dtype_t dt, void* dx, float* dw_g,
                          float* dw1, float* dw3, float* dw2, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Backward of the stack layer of moe_block_forward, y = x + MoE(u) with
 * u = x / sqrt(mean(x^2) + eps): the gradients of sum_t dy_t . y_t.  The MoE
 * part is differentiated as in moe_backward with u in place of x (the
 * routing from the fp32 u, the experts on bf16(u)), then through the
 * normalisation, plus the residual:
 *   dx = dy + s (du - u (u . du) / d),  s = 1 / sqrt(mean(x^2) + eps),
 * in fp32, rounded once.  dW_g sums the fp32 u.  Same arguments, layouts and
 * workspace (moe_backward_workspace_bytes) as moe_backward, plus eps (>= 0).
 * The normalisation and residual are this workload's definition, not the
 * pages'. */
moe_status_t moe_block_backward(const void* x, const void* w_g, const void* w1,
                                const void* w3, const void* w2, const void* dy,
                                int64_t T, int64_t d, int64_t d_ff, int32_t n,
                                int32_t K, moe_dtype_t dt, float eps, void* dx,
                                float* dw_g, float* dw1, float* dw3, float* dw2,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the saved state that moe_forward_train / moe_block_forward_train
 * write and moe_backward_saved / moe_block_backward_saved read, for these
 * sizes (bf16 only; 0 if invalid). */
size_t moe_saved_bytes(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K,
                       moe_dtype_t dt);

/* moe_forward for training: the same y (bit for bit), and the routing, the
 * per-expert permutation and the bf16 pre-activations [a | b] of every
 * assignment kept in `saved` (caller-owned device memory of at least
 * moe_saved_bytes(...) bytes, 256-byte aligned, opaque layout) for
 * moe_backward_saved, which then need not recompute them.  bf16 plain layer
 * only (MOE_ERR_UNSUPPORTED otherwise).  workspace as for moe_forward.  One
 * pass only: T beyond what one pass of moe_forward holds returns
 * MOE_ERR_UNSUPPORTED (the saved state covers all T tokens at once). */
moe_status_t moe_forward_train(const void* x, const void* w_g, const void* w1,
                               const void* w3, const void* w2, int64_t T, int64_t d,
                               int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt,
                               void* y, void* saved, size_t saved_bytes,
                               void* workspace, size_t workspace_bytes, void* stream);

/* moe_backward from a saved state: `saved` must hold what moe_forward_train
 * wrote for the same x, weights and sizes.  It is read, never written.  The
 * gradients then equal moe_backward's bit for bit.  Any other contents are
 * undefined behaviour: the kernels index rows with the saved permutation.
 * Workspace: moe_backward_workspace_bytes(...). */
moe_status_t moe_backward_saved(const void* x, const void* w_g, const void* w1,
                                const void* w3, const void* w2, const void* dy,
                                const void* saved, size_t saved_bytes, int64_t T,
                                int64_t d, int64_t d_ff, int32_t n, int32_t K,
                                moe_dtype_t dt, void* dx, float* dw_g, float* dw1,
                                float* dw3, float* dw2, void* workspace,
                                size_t workspace_bytes, void* stream);

/* The training pair for the stack layer of moe_block_forward /
 * moe_block_backward: the forward also keeps the routing, the permutation,
 * [a | b] and the normalised input bf16(u) in `saved`
 * (moe_saved_bytes(...) bytes, 256-byte aligned), and the backward uses them
 * instead of recomputing.  y and the gradients equal moe_block_forward's and
 * moe_block_backward's bit for bit.  The same rules for `saved` as for
 * moe_backward_saved. */
moe_status_t moe_block_forward_train(const void* x, const void* w_g, const void* w1,
                                     const void* w3, const void* w2, int64_t T,
                                     int64_t d, int64_t d_ff, int32_t n, int32_t K,
                                     moe_dtype_t dt, float eps, void* y, void* saved,
                                     size_t saved_bytes, void* workspace,
                                     size_t workspace_bytes, void* stream);
moe_status_t moe_block_backward_saved(const void* x, const void* w_g, const void* w1,
                                      const void* w3, const void* w2, const void* dy,
                                      const void* saved, size_t saved_bytes, int64_t T,
                                      int64_t d, int64_t d_ff, int32_t n, int32_t K,
                                      moe_dtype_t dt, float eps, void* dx, float* dw_g,
                                      float* dw1, float* dw3, float* dw2,
                                      void* workspace, size_t workspace_bytes,
                                      void* stream);

/* Timing hook (for profilers and benchmarks, not part of the layer): in later
 * moe_forward / moe_block_forward / moe_forward_train / moe_backward /
 * moe_backward_saved calls made by this thread, record
 * start_event on the call's stream right before `stage` is launched and
 * end_event right after it.  Both are caller-owned hipEvent_t handles that
 * must stay valid while set; NULL, NULL clears the hook.  Returns
 * MOE_ERR_INVALID_ARGUMENT for an unknown stage or a single NULL. */
moe_status_t moe_set_stage_events(int32_t stage, void* start_event, void* end_event);

/* bf16 GEMM kernel families (moe_set_gemm_path). */
typedef enum moe_gemm_path {
    MOE_GEMM_AUTO = 0,   /* chosen from the sizes: weight stream for few rows per expert */
    MOE_GEMM_TILED = 1,  /* MFMA tiles over many rows per expert */
    MOE_GEMM_STREAM = 2  /* weight stream (when its tables fit; tiled otherwise) */
} moe_gemm_path_t;

/* Testing and tuning hook (not part of the layer): later calls made by this
 * thread use the given bf16 GEMM kernel family instead of the one chosen from
 * the sizes.  Both families compute the same layer; the hook exists so that
 * tests can run each on the same input.  MOE_GEMM_AUTO restores the default.
 * The workspace bound (moe_workspace_bytes) covers every choice.  Returns
 * MOE_ERR_INVALID_ARGUMENT for an unknown value. */
moe_status_t moe_set_gemm_path(int32_t path);

/* Static description of a status code. */
const char* moe_status_string(moe_status_t status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
