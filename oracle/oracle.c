/*
 * Reference oracle for the sparse top-K mixture-of-experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct CPU
 * statement of what the layer computes.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark load it.  It shares no code, header,
 * table or helper with the GPU library, and the GPU library never calls it.
 *
 * Arithmetic: every product and sum is done in IEEE double.  Inputs arrive as
 * float arrays (a bf16 value widens to float exactly, and float widens to
 * double exactly), so no input is rounded.  Nothing intermediate is rounded.
 *
 * Sources (the pages on "Mixtral of Experts", arXiv 2401.04088):
 *   [G]  xyznot digest, section "Method (with core equations)": the gate
 *        G(x) := Softmax(TopK(x . W_g)), where TopK keeps the K largest entries
 *        of the logit vector l = x . W_g (n entries) and sets the rest to -inf.
 *   [Y]  same section: y = sum over i = 0..n-1 of G(x)_i * SwiGLU_i(x).
 *   [S]  same page, "Key terms": SwiGLU is a gated linear unit combining the
 *        Swish activation with an elementwise product; same section: each
 *        expert is a SwiGLU block with intermediate size 14336, n = 8, K = 2.
 *   [Z]  GeekNews summary, "Cara Komputasi Layer MoE": experts whose gate is
 *        zero need not be computed; the softmax is taken over the top-K logits
 *        of a linear layer.
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - SwiGLU_i(u) = W2_i (SiLU(W1_i u) (*) W3_i u), Swish with beta = 1 (SiLU),
 *     no biases.  The SiLU branch is W1.
 *   - Exactly K experts survive TopK; among equal logits the lower expert
 *     index ranks first.  Slot 0 holds the largest logit.
 *   - Storage: x[T][d], W_g[d][n] (column i belongs to expert i),
 *     W1,W3[n][d_ff][d], W2[n][d][d_ff], y[T][d], all row-major.
 *   - Block variant (a layer of a stack, not on the pages): u = x / sqrt(mean(x^2)
 *     + eps) with unit weight, y = x + MoE(u).
 *
 * Parallelism: OpenMP over tokens only.  Each token is computed by exactly the
 * per-token definition, so the result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Swish with beta = 1 ([S]): z * sigmoid(z). */
static double silu(double z) { return z / (1.0 + exp(-z)); }

/* Stack-layer pre-normalisation (not on the pages): u = x / sqrt(mean(x^2) + eps),
 * unit weight. */
static void rms_normalize(const float* x, int64_t d, double eps, double* u) {
    double ss = 0.0;
    for (int64_t k = 0; k < d; ++k) ss += (double)x[k] * (double)x[k];
    const double inv = 1.0 / sqrt(ss / (double)d + eps);
    for (int64_t k = 0; k < d; ++k) u[k] = (double)x[k] * inv;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* [G]: logits l_i = sum_k x_k W_g[k][i] for one token. */
static void token_logits(const float* x, const float* Wg, int64_t d, int32_t n,
                         double* l) {
    for (int32_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t k = 0; k < d; ++k) s += (double)x[k] * (double)Wg[k * n + i];
        l[i] = s;
    }
}

/* [G]: TopK.  Repeatedly take the largest logit not yet taken; a strictly
 * larger value is needed to displace an earlier (lower-index) candidate, so
 * ties go to the lower index.  Returns the K chosen experts in rank order. */
static void topk_select(const double* l, int32_t n, int32_t K, int32_t* sel) {
    unsigned char taken[4096];
    memset(taken, 0, (size_t)n);
    for (int32_t j = 0; j < K; ++j) {
        int32_t best = -1;
        for (int32_t i = 0; i < n; ++i) {
            if (taken[i]) continue;
            if (best < 0 || l[i] > l[best]) best = i;
        }
        sel[j] = best;
        taken[best] = 1;
    }
}

/* [G]: Softmax over the TopK-masked vector.  Masked entries are exp(-inf) = 0,
 * so only the K kept logits enter; m is subtracted for range only. */
static void masked_softmax(const double* l, const int32_t* sel, int32_t K,
                           double* g) {
    double m = l[sel[0]];
    for (int32_t j = 1; j < K; ++j)
        if (l[sel[j]] > m) m = l[sel[j]];
    double z = 0.0;
    for (int32_t j = 0; j < K; ++j) {
        g[j] = exp(l[sel[j]] - m);
        z += g[j];
    }
    for (int32_t j = 0; j < K; ++j) g[j] /= z;
}

/* [S]: one expert, o = W2 (SiLU(W1 u) (*) W3 u).  h has d_ff entries. */
static void swiglu_expert(const double* u, const float* W1, const float* W3,
                          const float* W2, int64_t d, int64_t d_ff, double* h,
                          double* o) {
    for (int64_t f = 0; f < d_ff; ++f) {
        double a = 0.0, b = 0.0;
        const float* w1 = W1 + f * d;
        const float* w3 = W3 + f * d;
        for (int64_t k = 0; k < d; ++k) {
            a += (double)w1[k] * u[k];
            b += (double)w3[k] * u[k];
        }
        h[f] = silu(a) * b;
    }
    for (int64_t c = 0; c < d; ++c) {
        double s = 0.0;
        const float* w2 = W2 + c * d_ff;
        for (int64_t f = 0; f < d_ff; ++f) s += (double)w2[f] * h[f];
        o[c] = s;
    }
}

/* One token of the layer: route, then [Y] y = sum_j g_j SwiGLU_{s_j}(u).
 * Experts off the selection have gate exactly 0 ([Z]) and are skipped.
 * If forced is non-null it replaces the TopK choice (used to evaluate the
 * other valid choice when two logits tie within a tolerance). */
static void token_forward(const double* u, const float* Wg,
                          const float* W1, const float* W3, const float* W2,
                          int64_t d, int64_t d_ff, int32_t n, int32_t K,
                          const int32_t* forced, double* y, int32_t* idx_out,
                          double* gate_out, double* logit_out, double* scratch) {
    double* l = scratch;            /* n */
    double* h = l + n;              /* d_ff */
    double* o = h + d_ff;           /* d */
    double g[64];
    int32_t sel[64] = {0};
    for (int32_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t k = 0; k < d; ++k) s += u[k] * (double)Wg[k * n + i];
        l[i] = s;
    }
    if (forced) {
        for (int32_t j = 0; j < K; ++j) sel[j] = forced[j];
    } else {
        topk_select(l, n, K, sel);
    }
    masked_softmax(l, sel, K, g);
    for (int64_t c = 0; c < d; ++c) y[c] = 0.0;
    for (int32_t j = 0; j < K; ++j) {
        const int64_t e = sel[j];
        swiglu_expert(u, W1 + e * d_ff * d, W3 + e * d_ff * d, W2 + e * d * d_ff,
                      d, d_ff, h, o);
        for (int64_t c = 0; c < d; ++c) y[c] += g[j] * o[c];
    }
    if (idx_out)
        for (int32_t j = 0; j < K; ++j) idx_out[j] = sel[j];
    if (gate_out)
        for (int32_t j = 0; j < K; ++j) gate_out[j] = g[j];
    if (logit_out)
        for (int32_t i = 0; i < n; ++i) logit_out[i] = l[i];
}

/* Router only ([G]): logits[T][n], idx[T][K], gate[T][K].  Any output may be
 * NULL.  Returns 0, or -1 on invalid sizes. */
int oracle_route(const float* x, const float* Wg, int64_t T, int64_t d, int32_t n,
                 int32_t K, double* logits, int32_t* idx, double* gate) {
    if (T < 0 || d <= 0 || n <= 0 || n > 4096 || K <= 0 || K > n || K > 64)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double lbuf[4096];
        double g[64];
        int32_t sel[64];
        token_logits(x + t * d, Wg, d, n, lbuf);
        topk_select(lbuf, n, K, sel);
        masked_softmax(lbuf, sel, K, g);
        if (logits)
            for (int32_t i = 0; i < n; ++i) logits[t * n + i] = lbuf[i];
        if (idx)
            for (int32_t j = 0; j < K; ++j) idx[t * K + j] = sel[j];
        if (gate)
            for (int32_t j = 0; j < K; ++j) gate[t * K + j] = g[j];
    }
    return 0;
}

/* Whole layer ([G], [Y], [S]) on the tokens listed in rows[0..R) (all T tokens
 * when rows is NULL, R = T).  Output row r of y/idx/gate/logits belongs to
 * token rows[r].  forced (nullable) is [R][K] expert ids replacing TopK.
 * Returns 0, -1 on invalid sizes, -2 on allocation failure. */
int oracle_forward(const float* x, const float* Wg, const float* W1, const float* W3,
                   const float* W2, int64_t T, int64_t d, int64_t d_ff, int32_t n,
                   int32_t K, const int64_t* rows, int64_t R, const int32_t* forced,
                   double* y, int32_t* idx, double* gate, double* logits) {
    if (T < 0 || d <= 0 || d_ff <= 0 || n <= 0 || n > 64 || K <= 0 || K > n)
        return -1;
    if (!rows) R = T;
    int err = 0;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * (size_t)(n + d_ff + 2 * d));
        if (!scratch) {
#pragma omp atomic write
            err = -2;
        } else {
            double* u = scratch + n + d_ff + d;
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < R; ++r) {
                const int64_t t = rows ? rows[r] : r;
                for (int64_t k = 0; k < d; ++k) u[k] = (double)x[t * d + k];
                token_forward(u, Wg, W1, W3, W2, d, d_ff, n, K,
                              forced ? forced + r * K : 0, y + r * d,
                              idx ? idx + r * K : 0, gate ? gate + r * K : 0,
                              logits ? logits + r * n : 0, scratch);
            }
            free(scratch);
        }
    }
    return err;
}

/* One layer of a stack (not on the pages; the stack workload's definition):
 * u = x / sqrt(mean(x^2) + eps) (unit weight), y = x + MoE(u).  Same row
 * selection and forced-routing conventions as oracle_forward; idx/gate/logits
 * describe the routing of u. */
int oracle_block_forward(const float* x, const float* Wg, const float* W1,
                         const float* W3, const float* W2, int64_t T, int64_t d,
                         int64_t d_ff, int32_t n, int32_t K, double eps,
                         const int64_t* rows, int64_t R, const int32_t* forced,
                         double* y, int32_t* idx, double* gate, double* logits) {
    if (T < 0 || d <= 0 || d_ff <= 0 || n <= 0 || n > 64 || K <= 0 || K > n ||
        !(eps >= 0.0))
        return -1;
    if (!rows) R = T;
    int err = 0;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * (size_t)(n + d_ff + 2 * d));
        if (!scratch) {
#pragma omp atomic write
            err = -2;
        } else {
            double* u = scratch + n + d_ff + d;
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < R; ++r) {
                const int64_t t = rows ? rows[r] : r;
                const float* xt = x + t * d;
                rms_normalize(xt, d, eps, u);
                double* yr = y + r * d;
                token_forward(u, Wg, W1, W3, W2, d, d_ff, n, K,
                              forced ? forced + r * K : 0, yr,
                              idx ? idx + r * K : 0, gate ? gate + r * K : 0,
                              logits ? logits + r * n : 0, scratch);
                for (int64_t k = 0; k < d; ++k) yr[k] += (double)xt[k];
            }
            free(scratch);
        }
    }
    return err;
}

/* Routing of a stack layer: TopK/Softmax of RMSNorm(x) . W_g on every token.
 * Same outputs as oracle_route. */
int oracle_block_route(const float* x, const float* Wg, int64_t T, int64_t d,
                       int32_t n, int32_t K, double eps, double* logits,
                       int32_t* idx, double* gate) {
    if (T < 0 || d <= 0 || n <= 0 || n > 64 || K <= 0 || K > n || !(eps >= 0.0))
        return -1;
    int err = 0;
#pragma omp parallel
    {
        double* u = (double*)malloc(sizeof(double) * (size_t)d);
        if (!u) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                double l[64], g[64];
                int32_t sel[64] = {0};
                rms_normalize(x + t * d, d, eps, u);
                for (int32_t i = 0; i < n; ++i) {
                    double s = 0.0;
                    for (int64_t k = 0; k < d; ++k) s += u[k] * (double)Wg[k * n + i];
                    l[i] = s;
                }
                topk_select(l, n, K, sel);
                masked_softmax(l, sel, K, g);
                if (logits)
                    for (int32_t i = 0; i < n; ++i) logits[t * n + i] = l[i];
                if (idx)
                    for (int32_t j = 0; j < K; ++j) idx[t * K + j] = sel[j];
                if (gate)
                    for (int32_t j = 0; j < K; ++j) gate[t * K + j] = g[j];
            }
            free(u);
        }
    }
    return err;
}

/* ------------------------------------------------------------------------
 * Backward of the layer: the gradients of L = sum_t dy_t . y_t by the chain
 * rule through the same definitions ([G], [Y], [S]).  For token t with kept
 * experts s_j, gates g_j and expert e = s_j:
 *   a = W1_e x, b = W3_e x, h = SiLU(a) (*) b, o = W2_e h
 *   dg_j = dy . o            do = g_j dy
 *   dh = W2_e^T do           db = dh (*) SiLU(a)
 *   da = dh (*) b (*) SiLU'(a),  SiLU'(a) = s + a s (1 - s), s = 1/(1 + e^-a)
 *   dW2_e += do h^T, dW1_e += da x^T, dW3_e += db x^T
 *   dx += W1_e^T da + W3_e^T db
 * The gates are the softmax of the kept logits, so for kept expert s_j
 *   dl_{s_j} = g_j (dg_j - sum_k g_k dg_k)
 * and every other logit gets 0 (TopK is constant under small changes away
 * from ties); then dW_g += x dl^T and dx += W_g dl.
 * ------------------------------------------------------------------------ */

/* Per-slot intermediates of one token, kept for the weight gradients. */
typedef struct {
    double* da;  /* [K][d_ff] */
    double* db;  /* [K][d_ff] */
    double* h;   /* [K][d_ff] */
    double* dO;  /* [K][d]    */
    double* dl;  /* [n]       */
    int32_t sel[64];
} slot_grads;

static void token_backward(const double* x, const float* Wg, const float* W1,
                           const float* W3, const float* W2, const float* dy,
                           int64_t d, int64_t d_ff, int32_t n, int32_t K,
                           const int32_t* forced, double* dx, slot_grads* sg,
                           double* scratch) {
    double* l = scratch;          /* n */
    double* a = l + n;            /* d_ff */
    double* b = a + d_ff;         /* d_ff */
    double* o = b + d_ff;         /* d */
    double* dh = o + d;           /* d_ff */
    double g[64], dg[64];
    int32_t* sel = sg->sel;
    for (int32_t i = 0; i < n; ++i) {
        double s = 0.0;
        for (int64_t k = 0; k < d; ++k) s += x[k] * (double)Wg[k * n + i];
        l[i] = s;
    }
    if (forced) {
        for (int32_t j = 0; j < K; ++j) sel[j] = forced[j];
    } else {
        topk_select(l, n, K, sel);
    }
    masked_softmax(l, sel, K, g);
    for (int64_t k = 0; k < d; ++k) dx[k] = 0.0;
    for (int32_t j = 0; j < K; ++j) {
        const int64_t e = sel[j];
        const float* w1 = W1 + e * d_ff * d;
        const float* w3 = W3 + e * d_ff * d;
        const float* w2 = W2 + e * d * d_ff;
        double* h = sg->h + j * d_ff;
        for (int64_t f = 0; f < d_ff; ++f) {
            double sa = 0.0, sb = 0.0;
            for (int64_t k = 0; k < d; ++k) {
                sa += (double)w1[f * d + k] * x[k];
                sb += (double)w3[f * d + k] * x[k];
            }
            a[f] = sa;
            b[f] = sb;
            h[f] = silu(sa) * sb;
        }
        double dgj = 0.0;
        for (int64_t c = 0; c < d; ++c) {
            double s = 0.0;
            for (int64_t f = 0; f < d_ff; ++f) s += (double)w2[c * d_ff + f] * h[f];
            o[c] = s;
            dgj += (double)dy[c] * s;
        }
        dg[j] = dgj;
        double* dO = sg->dO + j * d;
        for (int64_t c = 0; c < d; ++c) dO[c] = g[j] * (double)dy[c];
        for (int64_t f = 0; f < d_ff; ++f) dh[f] = 0.0;
        for (int64_t c = 0; c < d; ++c)
            for (int64_t f = 0; f < d_ff; ++f) dh[f] += (double)w2[c * d_ff + f] * dO[c];
        double* da = sg->da + j * d_ff;
        double* db = sg->db + j * d_ff;
        for (int64_t f = 0; f < d_ff; ++f) {
            const double s = 1.0 / (1.0 + exp(-a[f]));
            db[f] = dh[f] * a[f] * s;
            da[f] = dh[f] * b[f] * (s + a[f] * s * (1.0 - s));
        }
        for (int64_t f = 0; f < d_ff; ++f)
            for (int64_t k = 0; k < d; ++k)
                dx[k] += (double)w1[f * d + k] * da[f] + (double)w3[f * d + k] * db[f];
    }
    double gdg = 0.0;
    for (int32_t j = 0; j < K; ++j) gdg += g[j] * dg[j];
    for (int32_t i = 0; i < n; ++i) sg->dl[i] = 0.0;
    for (int32_t j = 0; j < K; ++j) sg->dl[sel[j]] = g[j] * (dg[j] - gdg);
    for (int64_t k = 0; k < d; ++k) {
        double s = 0.0;
        for (int32_t i = 0; i < n; ++i) s += (double)Wg[k * n + i] * sg->dl[i];
        dx[k] += s;
    }
}

/* The backward over input rows X[T][d] in fp64 (the layer's input, or its
 * normalised input for a stack layer): dx below is the gradient with respect
 * to X. */
static int backward_impl(const double* x, const float* Wg, const float* W1, const float* W3,
                         const float* W2, const float* dy, int64_t T, int64_t d, int64_t d_ff,
                         int32_t n, int32_t K, const int64_t* rows, int64_t R,
                         const int32_t* forced, double* dx, double* dWg, double* dW1,
                         double* dW3, double* dW2) {
    if (T < 0 || d <= 0 || d_ff <= 0 || n <= 0 || n > 64 || K <= 0 || K > n) return -1;
    const int weights = dWg || dW1 || dW3 || dW2;
    if (rows && weights) return -1;
    if (!rows) R = T;
    const size_t per_slot = (size_t)(3 * d_ff + d);
    /* per-token intermediates; only kept when weight gradients are wanted */
    double* keep = 0;
    int32_t* keep_sel = 0;
    if (weights) {
        keep = (double*)malloc(sizeof(double) * ((size_t)R * (K * per_slot + n)));
        keep_sel = (int32_t*)malloc(sizeof(int32_t) * (size_t)R * K);
        if (!keep || !keep_sel) {
            free(keep);
            free(keep_sel);
            return -2;
        }
    }
    int err = 0;
#pragma omp parallel
    {
        double* scratch = (double*)malloc(sizeof(double) * (size_t)(n + 3 * d_ff + 2 * d));
        double* tmp = (double*)malloc(sizeof(double) * (K * per_slot + n));
        double* dxt = (double*)malloc(sizeof(double) * (size_t)d);
        if (!scratch || !tmp || !dxt) {
#pragma omp atomic write
            err = -2;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < R; ++r) {
                const int64_t t = rows ? rows[r] : r;
                double* base = weights ? keep + (size_t)r * (K * per_slot + n) : tmp;
                slot_grads sg;
                sg.da = base;
                sg.db = sg.da + (size_t)K * d_ff;
                sg.h = sg.db + (size_t)K * d_ff;
                sg.dO = sg.h + (size_t)K * d_ff;
                sg.dl = sg.dO + (size_t)K * d;
                token_backward(x + t * d, Wg, W1, W3, W2, dy + t * d, d, d_ff, n, K,
                               forced ? forced + r * K : 0, dxt, &sg, scratch);
                if (dx)
                    for (int64_t k = 0; k < d; ++k) dx[r * d + k] = dxt[k];
                if (weights)
                    for (int32_t j = 0; j < K; ++j) keep_sel[r * K + j] = sg.sel[j];
            }
        }
        free(scratch);
        free(tmp);
        free(dxt);
    }
    if (err || !weights) {
        free(keep);
        free(keep_sel);
        return err;
    }
    /* Weight gradients: every output entry sums its tokens in token order. */
    const size_t stride = K * per_slot + n;
#define SLOT(t, j, off) (keep + (size_t)(t) * stride + (off))
    if (dWg) {
#pragma omp parallel for schedule(static)
        for (int64_t k = 0; k < d; ++k)
            for (int32_t i = 0; i < n; ++i) {
                double s = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    s += x[t * d + k] * SLOT(t, 0, K * per_slot)[i];
                dWg[k * n + i] = s;
            }
    }
    if (dW1 || dW3) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t ef = 0; ef < (int64_t)n * d_ff; ++ef) {
            const int64_t e = ef / d_ff, f = ef % d_ff;
            for (int64_t k = 0; k < d; ++k) {
                double s1 = 0.0, s3 = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int32_t j = 0; j < K; ++j)
                        if (keep_sel[t * K + j] == e) {
                            const double xv = x[t * d + k];
                            s1 += SLOT(t, 0, j * d_ff)[f] * xv;
                            s3 += SLOT(t, 0, (size_t)K * d_ff + j * d_ff)[f] * xv;
                        }
                if (dW1) dW1[(e * d_ff + f) * d + k] = s1;
                if (dW3) dW3[(e * d_ff + f) * d + k] = s3;
            }
        }
    }
    if (dW2) {
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t ec = 0; ec < (int64_t)n * d; ++ec) {
            const int64_t e = ec / d, c = ec % d;
            for (int64_t f = 0; f < d_ff; ++f) {
                double s = 0.0;
                for (int64_t t = 0; t < T; ++t)
                    for (int32_t j = 0; j < K; ++j)
                        if (keep_sel[t * K + j] == e)
                            s += SLOT(t, 0, 3 * (size_t)K * d_ff + j * d)[c] *
                                 SLOT(t, 0, 2 * (size_t)K * d_ff + j * d_ff)[f];
                dW2[(e * d + c) * d_ff + f] = s;
            }
        }
    }
#undef SLOT
    free(keep);
    free(keep_sel);
    return 0;
}

/* Gradients of L = sum_t dy_t . y_t.  dy[T][d] is the output gradient;
 * forced (nullable, [R][K]) replaces TopK as in oracle_forward.  Outputs
 * (each nullable): dx[R][d] for the tokens in rows[0..R) (all T when rows is
 * NULL), and -- only when rows is NULL -- dWg[d][n], dW1[n][d_ff][d],
 * dW3[n][d_ff][d], dW2[n][d][d_ff], each summed over tokens in token order.
 * Returns 0, -1 on invalid arguments, -2 on allocation failure. */
int oracle_backward(const float* x, const float* Wg, const float* W1, const float* W3,
                    const float* W2, const float* dy, int64_t T, int64_t d, int64_t d_ff,
                    int32_t n, int32_t K, const int64_t* rows, int64_t R,
                    const int32_t* forced, double* dx, double* dWg, double* dW1,
                    double* dW3, double* dW2) {
    if (T < 0 || d <= 0) return -1;
    double* X = (double*)malloc(sizeof(double) * ((size_t)T * d + 1));
    if (!X) return -2;
    for (int64_t q = 0; q < T * d; ++q) X[q] = (double)x[q];
    const int rc = backward_impl(X, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, rows, R, forced, dx,
                                 dWg, dW1, dW3, dW2);
    free(X);
    return rc;
}

/* Backward of a stack layer y = x + MoE(u), u = x / sqrt(mean(x^2) + eps)
 * (unit weight; the layer of oracle_block_forward).  The MoE part is
 * differentiated with respect to u (routing from u, as in the forward), then
 * through the normalisation: with s = 1 / sqrt(mean(x^2) + eps),
 *   du_k/dx_j = s (delta_kj - u_k u_j / d),
 * so dx = dy + s (du - u (u . du) / d).  Same arguments and outputs as
 * oracle_backward (weight gradients summed with u in place of x) plus eps. */
int oracle_block_backward(const float* x, const float* Wg, const float* W1, const float* W3,
                          const float* W2, const float* dy, int64_t T, int64_t d,
                          int64_t d_ff, int32_t n, int32_t K, double eps, const int64_t* rows,
                          int64_t R, const int32_t* forced, double* dx, double* dWg,
                          double* dW1, double* dW3, double* dW2) {
    if (T < 0 || d <= 0 || !(eps >= 0.0)) return -1;
    if (!rows) R = T;
    double* X = (double*)malloc(sizeof(double) * ((size_t)T * d + 1));
    double* du = (double*)malloc(sizeof(double) * ((size_t)R * d + 1));
    if (!X || !du) {
        free(X);
        free(du);
        return -2;
    }
    for (int64_t t = 0; t < T; ++t) rms_normalize(x + t * d, d, eps, X + t * d);
    int rc = backward_impl(X, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, rows, R, forced,
                           dx ? du : 0, dWg, dW1, dW3, dW2);
    if (rc == 0 && dx) {
        for (int64_t r = 0; r < R; ++r) {
            const int64_t t = rows ? rows[r] : r;
            const float* xt = x + t * d;
            const double* u = X + t * d;
            double ss = 0.0, c = 0.0;
            for (int64_t k = 0; k < d; ++k) ss += (double)xt[k] * (double)xt[k];
            const double sc = 1.0 / sqrt(ss / (double)d + eps);
            for (int64_t k = 0; k < d; ++k) c += u[k] * du[r * d + k];
            for (int64_t k = 0; k < d; ++k)
                dx[r * d + k] = (double)dy[t * d + k] + sc * (du[r * d + k] - u[k] * c / (double)d);
        }
    }
    free(X);
    free(du);
    return rc;
}

/* Selected entries of the expert weight gradients, for checks at sizes where
 * the full gradients are out of reach.  Each entry is summed over every token
 * routed to its expert, in token order, from the per-token definition above
 * restricted to the one hidden unit f the entry needs:
 *   a_f = W1_e[f] . x,  b_f = W3_e[f] . x,  h_f = SiLU(a_f) b_f,
 *   r_f = sum_c W2_e[c][f] dy[c]  (the f-th entry of W2_e^T dy),
 *   dh_f = g_j r_f,  da_f = dh_f b_f SiLU'(a_f),  db_f = dh_f SiLU(a_f);
 *   dW2_e[c][f] = sum g_j dy[c] h_f,  dW1_e[f][k] = sum da_f x[k],
 *   dW3_e[f][k] = sum db_f x[k].
 * Entry q: which[q] = 1 (dW1), 2 (dW2) or 3 (dW3), expert ex[q], row ri[q]
 * and column ci[q] of that matrix.  Routing: forced[T][K] if given, else
 * TopK.  out[Q] in fp64.  Returns 0, -1 on invalid arguments, -2 on
 * allocation failure. */
static int entries_impl(const double* x, const float* Wg, const float* W1, const float* W3,
                        const float* W2, const float* dy, int64_t T, int64_t d, int64_t d_ff,
                        int32_t n, int32_t K, const int32_t* forced, int64_t Q,
                        const int32_t* which, const int32_t* ex, const int64_t* ri,
                        const int64_t* ci, double* out) {
    if (T < 0 || d <= 0 || d_ff <= 0 || n <= 0 || n > 64 || K <= 0 || K > n || Q < 0)
        return -1;
    for (int64_t q = 0; q < Q; ++q) {
        if (which[q] < 1 || which[q] > 3 || ex[q] < 0 || ex[q] >= n) return -1;
        const int64_t rows = which[q] == 2 ? d : d_ff, cols = which[q] == 2 ? d_ff : d;
        if (ri[q] < 0 || ri[q] >= rows || ci[q] < 0 || ci[q] >= cols) return -1;
    }
    int32_t* sel = (int32_t*)malloc(sizeof(int32_t) * ((size_t)T * K + 1));
    double* gate = (double*)malloc(sizeof(double) * ((size_t)T * K + 1));
    if (!sel || !gate) {
        free(sel);
        free(gate);
        return -2;
    }
    /* routing and gates of every token */
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double l[64], g[64];
        int32_t s[64];
        for (int32_t i = 0; i < n; ++i) {
            double acc = 0.0;
            for (int64_t k = 0; k < d; ++k)
                acc += x[t * d + k] * (double)Wg[k * n + i];
            l[i] = acc;
        }
        if (forced) {
            for (int32_t j = 0; j < K; ++j) s[j] = forced[t * K + j];
        } else {
            topk_select(l, n, K, s);
        }
        masked_softmax(l, s, K, g);
        for (int32_t j = 0; j < K; ++j) {
            sel[t * K + j] = s[j];
            gate[t * K + j] = g[j];
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < Q; ++q) {
        const int64_t e = ex[q];
        const int64_t f = which[q] == 2 ? ci[q] : ri[q];  /* hidden unit */
        const float* w1 = W1 + (e * d_ff + f) * d;
        const float* w3 = W3 + (e * d_ff + f) * d;
        const float* w2 = W2 + e * d * d_ff;
        double s = 0.0;
        for (int64_t t = 0; t < T; ++t)
            for (int32_t j = 0; j < K; ++j) {
                if (sel[t * K + j] != e) continue;
                const double* xt = x + t * d;
                const float* dyt = dy + t * d;
                const double g = gate[t * K + j];
                double a = 0.0, b = 0.0;
                for (int64_t k = 0; k < d; ++k) {
                    a += (double)w1[k] * xt[k];
                    b += (double)w3[k] * xt[k];
                }
                if (which[q] == 2) {
                    s += g * (double)dyt[ri[q]] * (silu(a) * b);
                    continue;
                }
                double r = 0.0;
                for (int64_t c = 0; c < d; ++c) r += (double)w2[c * d_ff + f] * (double)dyt[c];
                const double dh = g * r;
                const double sg = 1.0 / (1.0 + exp(-a));
                const double unit = which[q] == 1 ? dh * b * (sg + a * sg * (1.0 - sg))
                                                  : dh * a * sg;
                s += unit * xt[ci[q]];
            }
        out[q] = s;
    }
    free(sel);
    free(gate);
    return 0;
}

int oracle_backward_entries(const float* x, const float* Wg, const float* W1,
                            const float* W3, const float* W2, const float* dy, int64_t T,
                            int64_t d, int64_t d_ff, int32_t n, int32_t K,
                            const int32_t* forced, int64_t Q, const int32_t* which,
                            const int32_t* ex, const int64_t* ri, const int64_t* ci,
                            double* out) {
    if (T < 0 || d <= 0) return -1;
    double* X = (double*)malloc(sizeof(double) * ((size_t)T * d + 1));
    if (!X) return -2;
    for (int64_t q = 0; q < T * d; ++q) X[q] = (double)x[q];
    const int rc = entries_impl(X, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, forced, Q, which, ex,
                                ri, ci, out);
    free(X);
    return rc;
}

/* The same entries for a stack layer: the experts' input is u = RMSNorm(x)
 * (eps, unit weight) and the routing comes from u. */
int oracle_block_backward_entries(const float* x, const float* Wg, const float* W1,
                                  const float* W3, const float* W2, const float* dy, int64_t T,
                                  int64_t d, int64_t d_ff, int32_t n, int32_t K, double eps,
                                  const int32_t* forced, int64_t Q, const int32_t* which,
                                  const int32_t* ex, const int64_t* ri, const int64_t* ci,
                                  double* out) {
    if (T < 0 || d <= 0 || !(eps >= 0.0)) return -1;
    double* X = (double*)malloc(sizeof(double) * ((size_t)T * d + 1));
    if (!X) return -2;
    for (int64_t t = 0; t < T; ++t) rms_normalize(x + t * d, d, eps, X + t * d);
    const int rc = entries_impl(X, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, forced, Q, which, ex,
                                ri, ci, out);
    free(X);
    return rc;
}
