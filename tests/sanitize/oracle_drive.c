/* Memory and undefined-behaviour check of the oracle (oracle/oracle.c), built
 * with AddressSanitizer and UndefinedBehaviorSanitizer by
 * tests/test_sanitizers.py.  Every entry point runs on small layers held in
 * buffers of exactly the documented sizes, so a read or write past any of
 * them, a use after free or a leak ends the run with a report.  Covered:
 * every routing width from K = 1 to K = n (n = 1 .. 64), T = 0, row subsets,
 * forced routing, weight-gradient entries of all three matrices, and the
 * argument checks.  Values are not checked here beyond plain invariants
 * (gates sum to one); the parity tests pin them. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_route(const float*, const float*, int64_t, int64_t, int32_t, int32_t, double*,
                 int32_t*, double*);
int oracle_block_route(const float*, const float*, int64_t, int64_t, int32_t, int32_t, double,
                       double*, int32_t*, double*);
int oracle_forward(const float*, const float*, const float*, const float*, const float*,
                   int64_t, int64_t, int64_t, int32_t, int32_t, const int64_t*, int64_t,
                   const int32_t*, double*, int32_t*, double*, double*);
int oracle_block_forward(const float*, const float*, const float*, const float*, const float*,
                         int64_t, int64_t, int64_t, int32_t, int32_t, double, const int64_t*,
                         int64_t, const int32_t*, double*, int32_t*, double*, double*);
int oracle_backward(const float*, const float*, const float*, const float*, const float*,
                    const float*, int64_t, int64_t, int64_t, int32_t, int32_t, const int64_t*,
                    int64_t, const int32_t*, double*, double*, double*, double*, double*);
int oracle_block_backward(const float*, const float*, const float*, const float*, const float*,
                          const float*, int64_t, int64_t, int64_t, int32_t, int32_t, double,
                          const int64_t*, int64_t, const int32_t*, double*, double*, double*,
                          double*, double*);
int oracle_backward_entries(const float*, const float*, const float*, const float*,
                            const float*, const float*, int64_t, int64_t, int64_t, int32_t,
                            int32_t, const int32_t*, int64_t, const int32_t*, const int32_t*,
                            const int64_t*, const int64_t*, double*);
int oracle_block_backward_entries(const float*, const float*, const float*, const float*,
                                  const float*, const float*, int64_t, int64_t, int64_t,
                                  int32_t, int32_t, double, const int32_t*, int64_t,
                                  const int32_t*, const int32_t*, const int64_t*,
                                  const int64_t*, double*);

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static double uniform(void) { /* xorshift64*, in [-1, 1) */
    rng ^= rng >> 12;
    rng ^= rng << 25;
    rng ^= rng >> 27;
    return (double)((rng * 0x2545F4914F6CDD1Dull) >> 11) / 4503599627370496.0 - 1.0;
}
static void* block(size_t bytes) { return malloc(bytes ? bytes : 1); }
static float* randf(size_t count, double scale) {
    float* p = (float*)block(count * sizeof(float));
    for (size_t i = 0; i < count; ++i) p[i] = (float)(scale * uniform());
    return p;
}

static int failures = 0;
#define CHECK(cond, ...)                          \
    do {                                          \
        if (!(cond)) {                            \
            fprintf(stderr, "FAIL: " __VA_ARGS__); \
            fprintf(stderr, "\n");                \
            ++failures;                           \
        }                                         \
    } while (0)

static void gates_sum_to_one(const double* gate, int64_t R, int32_t K, const char* what) {
    for (int64_t r = 0; r < R; ++r) {
        double s = 0.0;
        for (int32_t k = 0; k < K; ++k) s += gate[r * K + k];
        CHECK(fabs(s - 1.0) < 1e-12, "%s: gates of row %lld sum to %g", what, (long long)r, s);
    }
}

static void run_case(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K) {
    printf("case T=%lld d=%lld d_ff=%lld n=%d K=%d\n", (long long)T, (long long)d,
           (long long)d_ff, n, K);
    const size_t wsz = (size_t)n * (size_t)d_ff * (size_t)d;
    float* x = randf((size_t)T * d, 2.0);
    float* Wg = randf((size_t)d * n, 1.0 / sqrt((double)d));
    float* W1 = randf(wsz, 1.0 / sqrt((double)d));
    float* W3 = randf(wsz, 1.0 / sqrt((double)d));
    float* W2 = randf(wsz, 1.0 / sqrt((double)d_ff));
    float* dy = randf((size_t)T * d, 1.0);
    const double eps = 1e-5;

    double* logits = (double*)block(sizeof(double) * (size_t)T * n);
    int32_t* idx = (int32_t*)block(sizeof(int32_t) * (size_t)T * K);
    double* gate = (double*)block(sizeof(double) * (size_t)T * K);
    double* y = (double*)block(sizeof(double) * (size_t)T * d);
    CHECK(oracle_route(x, Wg, T, d, n, K, logits, idx, gate) == 0, "route");
    gates_sum_to_one(gate, T, K, "route");
    CHECK(oracle_block_route(x, Wg, T, d, n, K, eps, logits, idx, gate) == 0, "block_route");
    gates_sum_to_one(gate, T, K, "block_route");
    CHECK(oracle_forward(x, Wg, W1, W3, W2, T, d, d_ff, n, K, 0, 0, 0, y, idx, gate, logits) ==
              0, "forward");
    CHECK(oracle_block_forward(x, Wg, W1, W3, W2, T, d, d_ff, n, K, eps, 0, 0, 0, y, idx, gate,
                               logits) == 0, "block_forward");
    /* optional outputs left out */
    CHECK(oracle_forward(x, Wg, W1, W3, W2, T, d, d_ff, n, K, 0, 0, 0, y, 0, 0, 0) == 0,
          "forward without routing outputs");

    /* a row subset (last row first, repeats allowed) with forced experts:
     * row r takes experts (r + k) mod n, k = 0 .. K-1 (distinct) */
    const int64_t R = T < 3 ? T : 3;
    int64_t* rows = (int64_t*)block(sizeof(int64_t) * (size_t)R);
    int32_t* forced = (int32_t*)block(sizeof(int32_t) * (size_t)R * K);
    for (int64_t r = 0; r < R; ++r) {
        rows[r] = (T - 1 - 2 * r + 4 * T) % T;
        for (int32_t k = 0; k < K; ++k) forced[r * K + k] = (int32_t)((r + k) % n);
    }
    double* yr = (double*)block(sizeof(double) * (size_t)R * d);
    int32_t* ir = (int32_t*)block(sizeof(int32_t) * (size_t)R * K);
    double* gr = (double*)block(sizeof(double) * (size_t)R * K);
    double* lr = (double*)block(sizeof(double) * (size_t)R * n);
    CHECK(oracle_forward(x, Wg, W1, W3, W2, T, d, d_ff, n, K, rows, R, forced, yr, ir, gr, lr) ==
              0, "forward rows forced");
    for (int64_t q = 0; q < R * K; ++q) CHECK(ir[q] == forced[q], "forced expert %lld", (long long)q);
    gates_sum_to_one(gr, R, K, "forward rows forced");
    CHECK(oracle_block_forward(x, Wg, W1, W3, W2, T, d, d_ff, n, K, eps, rows, R, forced, yr, ir,
                               gr, lr) == 0, "block_forward rows forced");

    /* gradients: all tokens with weights, then a row subset without */
    double* dx = (double*)block(sizeof(double) * (size_t)T * d);
    double* dWg = (double*)block(sizeof(double) * (size_t)d * n);
    double* dW1 = (double*)block(sizeof(double) * wsz);
    double* dW3 = (double*)block(sizeof(double) * wsz);
    double* dW2 = (double*)block(sizeof(double) * wsz);
    CHECK(oracle_backward(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, 0, 0, 0, dx, dWg, dW1, dW3,
                          dW2) == 0, "backward");
    CHECK(oracle_block_backward(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, eps, 0, 0, 0, dx, dWg,
                                dW1, dW3, dW2) == 0, "block_backward");
    int32_t* fall = (int32_t*)block(sizeof(int32_t) * (size_t)T * K);
    for (int64_t t = 0; t < T; ++t)
        for (int32_t k = 0; k < K; ++k) fall[t * K + k] = (int32_t)((3 * t + k) % n);
    CHECK(oracle_backward(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, 0, 0, fall, dx, dWg, dW1,
                          dW3, dW2) == 0, "backward forced");
    double* dxr = (double*)block(sizeof(double) * (size_t)R * d);
    CHECK(oracle_backward(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, rows, R, forced, dxr, 0, 0, 0,
                          0) == 0, "backward rows");
    CHECK(oracle_block_backward(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, eps, rows, R, forced,
                                dxr, 0, 0, 0, 0) == 0, "block_backward rows");
    /* weight gradients with a row subset are refused */
    CHECK(oracle_backward(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, rows, R, 0, dxr, dWg, 0, 0,
                          0) == -1, "backward rows with weights");

    /* entries: corners of each matrix of the first and last expert */
    enum { Q = 12 };
    int32_t which[Q], ex[Q];
    int64_t ri[Q], ci[Q];
    for (int q = 0; q < Q; ++q) {
        which[q] = 1 + q % 3;
        ex[q] = (q / 3) % 2 ? n - 1 : 0;
        const int64_t rmax = which[q] == 2 ? d : d_ff, cmax = which[q] == 2 ? d_ff : d;
        ri[q] = (q / 6) ? rmax - 1 : 0;
        ci[q] = (q / 6) ? cmax - 1 : 0;
    }
    double* out = (double*)block(sizeof(double) * Q);
    CHECK(oracle_backward_entries(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, 0, Q, which, ex, ri,
                                  ci, out) == 0, "entries");
    CHECK(oracle_backward_entries(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, fall, Q, which, ex,
                                  ri, ci, out) == 0, "entries forced");
    CHECK(oracle_block_backward_entries(x, Wg, W1, W3, W2, dy, T, d, d_ff, n, K, eps, 0, Q,
                                        which, ex, ri, ci, out) == 0, "block entries");

    /* argument checks */
    CHECK(oracle_route(x, Wg, T, d, n, n + 1, logits, idx, gate) == -1, "K > n");
    CHECK(oracle_forward(x, Wg, W1, W3, W2, -1, d, d_ff, n, K, 0, 0, 0, y, 0, 0, 0) == -1,
          "T < 0");
    CHECK(oracle_block_route(x, Wg, T, d, n, K, -1.0, logits, idx, gate) == -1, "eps < 0");

    free(x); free(Wg); free(W1); free(W3); free(W2); free(dy);
    free(logits); free(idx); free(gate); free(y);
    free(rows); free(forced); free(yr); free(ir); free(gr); free(lr);
    free(dx); free(dWg); free(dW1); free(dW3); free(dW2); free(fall); free(dxr); free(out);
}

int main(void) {
    run_case(7, 16, 24, 8, 2);
    run_case(5, 8, 8, 1, 1);
    run_case(9, 24, 16, 4, 4);
    run_case(0, 8, 8, 4, 2);
    run_case(1, 8, 16, 8, 8);
    run_case(6, 40, 32, 64, 8);
    run_case(4, 16, 8, 13, 3);
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("oracle: all entry points clean\n");
    return 0;
}
