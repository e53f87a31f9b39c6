// Host-side argument handling of the C ABI (include/moe.h) under
// AddressSanitizer and UndefinedBehaviorSanitizer, built by
// tests/test_sanitizers.py with the library's host code instrumented.  Every
// call here is one the library must refuse (or finish, for T = 0) before
// touching a device, so the run needs no GPU; the pointers are never
// dereferenced.  The size queries sweep the whole supported range, up to
// T * K = 2^31 - 1 and d, d_ff = 2^24, where any signed overflow in the size
// arithmetic would be reported.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "moe.h"

namespace {

int failures = 0;

void* P(uint64_t k) { return reinterpret_cast<void*>(uintptr_t(0x10000) * k); }

void expect(moe_status_t got, moe_status_t want, const char* what, const char* msg = nullptr) {
    const char* err = moe_last_error();
    if (got != want || (msg && !std::strstr(err, msg))) {
        std::fprintf(stderr, "FAIL %s: got %s, want %s (%s)\n", what, moe_status_string(got),
                     moe_status_string(want), err);
        ++failures;
    }
}

void check(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAIL %s\n", what);
        ++failures;
    }
}

struct Fwd {
    void *x = P(1), *wg = P(2), *w1 = P(3), *w3 = P(4), *w2 = P(5), *y = P(64), *ws = P(128);
    int64_t T = 16, d = 64, d_ff = 64;
    int32_t n = 8, K = 2;
    moe_dtype_t dt = MOE_BF16;
    size_t ws_bytes = size_t(1) << 30;
    int32_t* idx = nullptr;
    float* gate = nullptr;
    int32_t* counts = nullptr;
    moe_status_t run() const {
        return moe_forward(x, wg, w1, w3, w2, T, d, d_ff, n, K, dt, y, ws, ws_bytes, idx, gate,
                           counts, nullptr);
    }
    moe_status_t run_block(float eps) const {
        return moe_block_forward(x, wg, w1, w3, w2, T, d, d_ff, n, K, dt, eps, y, ws, ws_bytes,
                                 idx, gate, counts, nullptr);
    }
    moe_status_t run_noalloc() const {
        return moe_forward_noalloc(x, wg, w1, w3, w2, T, d, d_ff, n, K, dt, y, idx, gate, counts,
                                   nullptr);
    }
};

void forward_validation() {
    struct Case {
        const char* name;
        void (*edit)(Fwd&);
        moe_status_t want;
        const char* msg;
    };
    const Case cases[] = {
        {"x NULL", [](Fwd& f) { f.x = nullptr; }, MOE_ERR_INVALID_ARGUMENT, "x is NULL"},
        {"w2 NULL", [](Fwd& f) { f.w2 = nullptr; }, MOE_ERR_INVALID_ARGUMENT, "w2 is NULL"},
        {"y NULL", [](Fwd& f) { f.y = nullptr; }, MOE_ERR_INVALID_ARGUMENT, "y is NULL"},
        {"x misaligned", [](Fwd& f) { f.x = (char*)P(1) + 8; }, MOE_ERR_INVALID_ARGUMENT,
         "aligned"},
        {"ws NULL", [](Fwd& f) { f.ws = nullptr; }, MOE_ERR_INVALID_ARGUMENT, "workspace"},
        {"ws misaligned", [](Fwd& f) { f.ws = (char*)P(128) + 16; }, MOE_ERR_INVALID_ARGUMENT,
         "256-byte"},
        {"ws small", [](Fwd& f) { f.ws_bytes = 100; }, MOE_ERR_WORKSPACE_TOO_SMALL, "needed"},
        {"T < 0", [](Fwd& f) { f.T = -1; }, MOE_ERR_INVALID_ARGUMENT, "T ="},
        {"T min", [](Fwd& f) { f.T = std::numeric_limits<int64_t>::min(); },
         MOE_ERR_INVALID_ARGUMENT, "T ="},
        {"T max", [](Fwd& f) { f.T = std::numeric_limits<int64_t>::max(); },
         MOE_ERR_UNSUPPORTED, "2^31"},
        {"T*K 2^31", [](Fwd& f) { f.T = int64_t(1) << 30; }, MOE_ERR_UNSUPPORTED, "2^31"},
        {"K 0", [](Fwd& f) { f.K = 0; }, MOE_ERR_INVALID_ARGUMENT, "K ="},
        {"K > n", [](Fwd& f) { f.K = 3, f.n = 2; }, MOE_ERR_INVALID_ARGUMENT, "K ="},
        {"K 9", [](Fwd& f) { f.K = 9, f.n = 16; }, MOE_ERR_UNSUPPORTED, "K = 9"},
        {"n 65", [](Fwd& f) { f.n = 65; }, MOE_ERR_UNSUPPORTED, "n = 65"},
        {"n min", [](Fwd& f) { f.n = std::numeric_limits<int32_t>::min(); },
         MOE_ERR_INVALID_ARGUMENT, "n ="},
        {"d 60", [](Fwd& f) { f.d = 60; }, MOE_ERR_UNSUPPORTED, "multiple of 8"},
        {"d huge", [](Fwd& f) { f.d = int64_t(1) << 40; }, MOE_ERR_UNSUPPORTED, "2^24"},
        {"d_ff 0", [](Fwd& f) { f.d_ff = 0; }, MOE_ERR_INVALID_ARGUMENT, "d_ff"},
        {"d_ff max", [](Fwd& f) { f.d_ff = std::numeric_limits<int64_t>::max(); },
         MOE_ERR_UNSUPPORTED, "d_ff"},
        {"dtype", [](Fwd& f) { f.dt = (moe_dtype_t)5; }, MOE_ERR_INVALID_ARGUMENT, "dtype"},
        {"y = x", [](Fwd& f) { f.y = P(1); }, MOE_ERR_INVALID_ARGUMENT, "overlaps"},
        {"y = ws", [](Fwd& f) { f.y = P(128); }, MOE_ERR_INVALID_ARGUMENT, "overlaps"},
        {"idx in y", [](Fwd& f) { f.idx = (int32_t*)((char*)P(64) + 4); },
         MOE_ERR_INVALID_ARGUMENT, "overlaps"},
        {"gate misaligned", [](Fwd& f) { f.gate = (float*)((char*)P(7) + 2); },
         MOE_ERR_INVALID_ARGUMENT, "aligned"},
        {"ws over w1", [](Fwd& f) { f.ws = P(3); }, MOE_ERR_INVALID_ARGUMENT,
         "workspace overlaps"},
        {"big weights", [](Fwd& f) { f.d = 16384, f.d_ff = 65536; }, MOE_ERR_UNSUPPORTED,
         "d * d_ff"},
    };
    for (const Case& c : cases) {
        Fwd f;
        c.edit(f);
        expect(f.run(), c.want, c.name, c.msg);
        expect(f.run_block(1e-5f), c.want, c.name, c.msg);
    }
    Fwd f;
    f.T = 0, f.x = nullptr, f.y = nullptr, f.ws = nullptr, f.ws_bytes = 0;
    expect(f.run(), MOE_OK, "T = 0");
    expect(f.run_noalloc(), MOE_OK, "noalloc T = 0");
    Fwd g;
    expect(g.run_block(-1.0f), MOE_ERR_INVALID_ARGUMENT, "eps < 0", "eps");
    expect(g.run_block(std::nanf("")), MOE_ERR_INVALID_ARGUMENT, "eps nan", "eps");
    expect(g.run_block(INFINITY), MOE_ERR_INVALID_ARGUMENT, "eps inf", "eps");
    // a chunked call is validated over all its tokens
    Fwd c;
    c.d = 128, c.d_ff = 32768, c.T = 50000;
    c.x = P(uint64_t(1) << 24), c.y = P(uint64_t(1) << 25), c.ws = P(uint64_t(1) << 26);
    c.ws_bytes = moe_workspace_bytes(c.T, c.d, c.d_ff, c.n, c.K, c.dt);
    c.idx = (int32_t*)((char*)c.ws - c.T * c.K * 4 + 256);
    expect(c.run(), MOE_ERR_INVALID_ARGUMENT, "chunked idx into ws", "workspace overlaps");
    c.idx = nullptr;
    c.ws_bytes -= 1;
    expect(c.run(), MOE_ERR_WORKSPACE_TOO_SMALL, "chunked ws small", "needed");
    // the static scratch: too large, and a chunk-sized batch
    Fwd a;
    a.d = 4096, a.d_ff = 14336, a.T = 4096;
    expect(a.run_noalloc(), MOE_ERR_UNSUPPORTED, "noalloc big", "static scratch");
    a.T = 40000;
    expect(a.run_noalloc(), MOE_ERR_UNSUPPORTED, "noalloc chunked", "split the tokens");
    a.T = 16, a.x = nullptr;
    expect(a.run_noalloc(), MOE_ERR_INVALID_ARGUMENT, "noalloc x NULL", "x is NULL");
}

void size_queries() {
    const int64_t Ts[] = {0, 1, 15, 16, 17, 128, 129, 256, 257, 4096, 16383, 16384, 37449, 37450,
                          1000003, (int64_t(1) << 30) - 1, int64_t(1) << 30,
                          std::numeric_limits<int64_t>::max(), -1};
    const int64_t ds[] = {8, 64, 4096, 8192, int64_t(1) << 24, (int64_t(1) << 24) + 8, 12};
    const int32_t ns[] = {1, 8, 64, 65, 0};
    const int32_t Ks[] = {1, 2, 8, 9};
    size_t checked = 0;
    for (int64_t T : Ts)
        for (int64_t d : ds)
            for (int64_t d_ff : ds)
                for (int32_t n : ns)
                    for (int32_t K : Ks)
                        for (int dt = 0; dt < 3; ++dt) {
                            const size_t w = moe_workspace_bytes(T, d, d_ff, n, K, (moe_dtype_t)dt);
                            const size_t b =
                                moe_backward_workspace_bytes(T, d, d_ff, n, K, (moe_dtype_t)dt);
                            const size_t s = moe_saved_bytes(T, d, d_ff, n, K, (moe_dtype_t)dt);
                            const bool valid = T >= 0 && n >= 1 && n <= 64 && K >= 1 && K <= n &&
                                               K <= 8 && d % 8 == 0 && d_ff % 8 == 0 &&
                                               d <= (int64_t(1) << 24) &&
                                               d_ff <= (int64_t(1) << 24) && dt < 2 &&
                                               T <= ((int64_t(1) << 31) - 1) / K;
                            check(valid == (w > 0), "workspace bytes of invalid sizes is 0");
                            check(!valid || dt != 1 || b > s, "backward workspace > saved state");
                            check(dt == 1 || (b == 0 && s == 0), "backward: bf16 only");
                            ++checked;
                        }
    std::printf("size queries: %zu combinations\n", checked);
}

void backward_validation() {
    const int64_t T = 16, d = 64, d_ff = 64;
    const int32_t n = 8, K = 2;
    const size_t sb = moe_saved_bytes(T, d, d_ff, n, K, MOE_BF16);
    const size_t bw = moe_backward_workspace_bytes(T, d, d_ff, n, K, MOE_BF16);
    void* ws = P(256);
    void* sv = P(1024);
    auto bwd = [&](void* dx, void* dwg, size_t wsb, moe_dtype_t dt) {
        return moe_backward(P(1), P(2), P(3), P(4), P(5), P(6), T, d, d_ff, n, K, dt, dx,
                            (float*)dwg, (float*)P(96), (float*)P(128), (float*)P(160), ws, wsb,
                            nullptr);
    };
    expect(bwd(P(64), P(80), bw, MOE_F32), MOE_ERR_UNSUPPORTED, "bwd fp32");
    expect(bwd(P(64), P(80), bw - 1, MOE_BF16), MOE_ERR_WORKSPACE_TOO_SMALL, "bwd ws");
    expect(bwd((char*)P(64) + 8, P(80), bw, MOE_BF16), MOE_ERR_INVALID_ARGUMENT, "bwd dx align");
    expect(bwd(P(1), P(80), bw, MOE_BF16), MOE_ERR_INVALID_ARGUMENT, "bwd dx over x");
    expect(bwd(P(64), P(64), bw, MOE_BF16), MOE_ERR_INVALID_ARGUMENT, "bwd outputs overlap");
    expect(moe_backward_saved(P(1), P(2), P(3), P(4), P(5), P(6), nullptr, sb, T, d, d_ff, n, K,
                              MOE_BF16, P(64), (float*)P(80), (float*)P(96), (float*)P(128),
                              (float*)P(160), ws, bw, nullptr),
           MOE_ERR_INVALID_ARGUMENT, "bwd saved NULL");
    expect(moe_backward_saved(P(1), P(2), P(3), P(4), P(5), P(6), sv, sb - 1, T, d, d_ff, n, K,
                              MOE_BF16, P(64), (float*)P(80), (float*)P(96), (float*)P(128),
                              (float*)P(160), ws, bw, nullptr),
           MOE_ERR_WORKSPACE_TOO_SMALL, "bwd saved small");
    for (float eps : {-1.0f, std::nanf(""), INFINITY}) {
        expect(moe_block_backward(P(1), P(2), P(3), P(4), P(5), P(6), T, d, d_ff, n, K, MOE_BF16,
                                  eps, P(64), (float*)P(80), (float*)P(96), (float*)P(128),
                                  (float*)P(160), ws, bw, nullptr),
               MOE_ERR_INVALID_ARGUMENT, "block bwd eps");
        expect(moe_block_forward_train(P(1), P(2), P(3), P(4), P(5), T, d, d_ff, n, K, MOE_BF16,
                                       eps, P(64), sv, sb, ws, size_t(1) << 30, nullptr),
               MOE_ERR_INVALID_ARGUMENT, "block fwd train eps");
    }
    expect(moe_forward_train(P(1), P(2), P(3), P(4), P(5), T, d, d_ff, n, K, MOE_BF16, P(64), sv,
                             sb - 1, ws, size_t(1) << 30, nullptr),
           MOE_ERR_WORKSPACE_TOO_SMALL, "fwd train saved small");
    expect(moe_forward_train(P(1), P(2), P(3), P(4), P(5), T, d, d_ff, n, K, MOE_BF16, P(64), ws,
                             sb, ws, size_t(1) << 30, nullptr),
           MOE_ERR_INVALID_ARGUMENT, "fwd train saved over ws");
    // T = 0 with fill kernels would need a device: stop at an invalid argument
    expect(moe_backward(nullptr, P(2), P(3), P(4), P(5), nullptr, 0, d, d_ff, n, K, MOE_BF16,
                        nullptr, nullptr, (float*)P(96), (float*)P(128), (float*)P(160), ws, bw,
                        nullptr),
           MOE_ERR_INVALID_ARGUMENT, "bwd T = 0 dw_g NULL", "dw_g is NULL");
    // the one-pass limit of the backward at Mixtral width
    const int64_t Tb = 18725;
    expect(moe_backward(P(1), P(2), P(3), P(4), P(5), P(6), Tb, 4096, 14336, n, K, MOE_BF16,
                        P(64), (float*)P(80), (float*)P(96), (float*)P(128), (float*)P(160), ws,
                        size_t(1) << 40, nullptr),
           MOE_ERR_UNSUPPORTED, "bwd one pass", "2 GiB");
}

void small_entry_points() {
    expect(moe_route(nullptr, P(1), 4, 64, 8, 2, MOE_BF16, (int32_t*)P(2), (float*)P(3),
                     nullptr),
           MOE_ERR_INVALID_ARGUMENT, "route x NULL");
    expect(moe_route(P(1), P(1), 4, 64, 8, 2, MOE_BF16, (int32_t*)P(2), (float*)P(2), nullptr),
           MOE_ERR_INVALID_ARGUMENT, "route idx = gate");
    expect(moe_route(P(1), P(1), 4, 12, 8, 2, MOE_BF16, (int32_t*)P(2), (float*)P(3), nullptr),
           MOE_ERR_UNSUPPORTED, "route d 12");
    expect(moe_route(P(1), P(1), 0, 64, 8, 2, MOE_BF16, (int32_t*)P(2), (float*)P(3), nullptr),
           MOE_OK, "route T = 0");
    expect(moe_permute(nullptr, 4, 8, 2, (int32_t*)P(1), (int32_t*)P(2), (int32_t*)P(3), nullptr),
           MOE_ERR_INVALID_ARGUMENT, "permute NULL");
    expect(moe_permute((int32_t*)P(1), 4, 80, 2, (int32_t*)P(1), (int32_t*)P(2), (int32_t*)P(3),
                       nullptr),
           MOE_ERR_UNSUPPORTED, "permute n 80");
    expect(moe_permute((int32_t*)P(1), 0, 8, 2, (int32_t*)P(1), (int32_t*)P(2), (int32_t*)P(3),
                       nullptr),
           MOE_OK, "permute T = 0");
    for (int32_t s : {-1, 9, std::numeric_limits<int32_t>::max()})
        expect(moe_set_stage_events(s, nullptr, nullptr), MOE_ERR_INVALID_ARGUMENT, "stage");
    expect(moe_set_stage_events(0, P(1), nullptr), MOE_ERR_INVALID_ARGUMENT, "one event");
    expect(moe_set_stage_events(0, nullptr, nullptr), MOE_OK, "clear events");
    for (int32_t p : {-1, 3, std::numeric_limits<int32_t>::min()})
        expect(moe_set_gemm_path(p), MOE_ERR_INVALID_ARGUMENT, "gemm path");
    for (int32_t p : {1, 2, 0}) expect(moe_set_gemm_path(p), MOE_OK, "gemm path ok");
    for (int s = -2; s < 8; ++s) check(moe_status_string((moe_status_t)s) != nullptr, "status");
    check(moe_abi_version() == MOE_ABI_VERSION, "abi version");
}

}  // namespace

int main() {
    forward_validation();
    backward_validation();
    small_entry_points();
    size_queries();
    if (failures) {
        std::fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    std::printf("abi: validation clean\n");
    return 0;
}
