// C ABI of libmoe.so: validation, workspace layout, launch sequence.
//
// Layer of "Mixtral of Experts" (xyznot digest, "Method (with core equations)"):
// G(x) = Softmax(TopK(x . W_g)),  y = sum_i G(x)_i SwiGLU_i(x).
// Launch sequence on the caller's stream, no host synchronisation:
//   router -> permute -> gate/up grouped GEMM -> down grouped GEMM -> combine
// Arguments are checked before anything is enqueued; see include/moe.h.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "kernels.hpp"
#include "moe.h"

namespace {

thread_local char g_last_error[512] = "";

// Per-thread timing hooks (moe_set_stage_events): events recorded on the
// call's stream right before and right after one stage's kernel launch.
constexpr int kStages = 9;
thread_local hipEvent_t g_ev_start[kStages] = {};
thread_local hipEvent_t g_ev_end[kStages] = {};

moe_status_t fail(moe_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
moe_status_t fail(moe_status_t st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return st;
}

moe_status_t hip_fail(hipError_t err, const char* where) {
    return fail(MOE_ERR_HIP, "%s: %s (%d)", where, hipGetErrorString(err), (int)err);
}

constexpr int64_t kMaxDim = int64_t(1) << 24;   // keeps in-kernel int index math exact
constexpr int64_t kMaxRows = (int64_t(1) << 31) - 1;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Which GEMM kernels run for these sizes, and how many K splits the down
// projection uses.  Depends on sizes only (so the workspace bound holds);
// moe_set_gemm_path (a per-thread testing and tuning hook) can force a bf16
// path.
thread_local int32_t g_gemm_path = MOE_GEMM_AUTO;
// Upper bound of the K splits of the down projection (partial sums in the
// workspace): up to 8 for the skinny kernel (few rows), 4 for the tiled one.
int requested_down_splits(int64_t T, int32_t K) { return T * K <= 256 ? 8 : 4; }

// Compute units of the current device (cached per device id; threads that
// race on the first query store the same value).
int device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int cus = cache[dev].load(std::memory_order_relaxed);
    if (cus == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                hipSuccess || cus <= 0)
            cus = 256;
        cache[dev].store(cus, std::memory_order_relaxed);
    }
    return cus;
}

// Waves per CU and K splits of a skinny GEMM: the pair whose item count
// (all n experts touched; `groups` 16-column items per split) spreads most
// evenly over the persistent waves; ties go to fewer splits, since longer
// runs along each weight row stream faster.
struct SkinnyShape {
    int waves, splits;
};
SkinnyShape choose_skinny(int32_t n, int64_t N, int64_t Kdim, int max_splits, int cus) {
    const int64_t groups = (N + 15) / 16;
    SkinnyShape best{7, 1};
    double best_eff = -1.0;
    for (int s = 1; s <= max_splits; ++s) {
        if (moe::skinny_splits_used((int)Kdim, s) != s) continue;
        for (int w = 7; w <= 8; ++w) {
            const int64_t items = (int64_t)n * groups * s;
            const int64_t nw = (int64_t)cus * w;
            const int64_t rounds = (items + nw - 1) / nw;
            const double eff = (double)items / (double)(rounds * nw);
            if (eff > best_eff + 1e-9) {
                best_eff = eff;
                best = {w, s};
            }
        }
    }
    return best;
}

struct Plan {
    bool skinny;
    int down_splits;  // partial sums of the down projection (skinny path)
};

Plan choose_plan(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt) {
    Plan p{false, 1};
    if (dt != MOE_BF16) return p;
    const int64_t A = T * K;
    // expected rows per expert; the skinny kernel re-streams weights per 16 rows
    p.skinny = A <= 16 * (int64_t)n;
    if (g_gemm_path == MOE_GEMM_TILED) p.skinny = false;
    if (g_gemm_path == MOE_GEMM_STREAM) p.skinny = true;
    if (!moe::skinny_fits(T, A, d, d_ff, 1) ||
        !moe::skinny_fits(A, A, d_ff, d, requested_down_splits(T, K)))
        p.skinny = false;
    // splits requested; the launcher may use fewer (never more) when d_ff is short
    if (p.skinny) p.down_splits = requested_down_splits(T, K);
    return p;
}

struct Layout {
    size_t idx, gate, offsets, perm, inv, meta, pcnt, u, H, O, total;
};

Layout layout(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt) {
    const size_t A = (size_t)T * (size_t)K;
    const size_t es = dt == MOE_BF16 ? 2 : 4;
    const int S = requested_down_splits(T, K);  // upper bound of the splits used
    Layout L{};
    size_t o = 0;
    L.idx = o;     o = align256(o + A * 4);
    L.gate = o;    o = align256(o + A * 4);
    L.offsets = o; o = align256(o + (size_t)(n + 1) * 4);
    L.perm = o;    o = align256(o + A * 4);
    L.inv = o;     o = align256(o + A * 4);
    L.meta = o;    o = align256(o + 2 * 4);  // (R0, Sr) of the tiled down projection
    L.pcnt = o;    o = align256(o + (size_t)moe::permute_blocks((int64_t)A) * (size_t)n * 4);
    L.u = o;       o = align256(o + (size_t)T * (size_t)d * es);
    L.H = o;       o = align256(o + A * (size_t)d_ff * es);
    L.O = o;       o = align256(o + (size_t)S * A * (size_t)d * 4);
    L.total = o;
    return L;
}

// Tokens per chunk of moe_forward / moe_block_forward: the most tokens whose
// operands the kernels index with 32-bit offsets (bf16: T * d and T * K * d_ff
// elements below 2^30; fp32: a grid bound of the grouped kernel).  A call with
// more tokens runs them in near-equal chunks of at most this many, one after
// the other on its stream, in a workspace sized for one chunk.  0: the weights
// themselves are too large for the kernels.
int64_t chunk_tokens(int64_t d, int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt) {
    if (dt != MOE_BF16) return ((int64_t)65535 - n) * 64 / K;
    if (!moe::tiled_fits(1, d, d_ff) || !moe::tiled_fits(K, d_ff, d)) return 0;
    const int64_t lim = (int64_t(1) << 31) - 1;
    const int64_t t1 = lim / (2 * d), t2 = lim / (2 * d_ff) / K;
    return t1 < t2 ? t1 : t2;
}

// The chunk length of a call over T tokens: T itself when it fits, else
// ceil(T / chunks) for the fewest chunks of at most chunk_tokens tokens.
int64_t chunk_len(int64_t T, int64_t cmax) {
    if (cmax <= 0 || T <= cmax) return T;
    const int64_t chunks = (T + cmax - 1) / cmax;
    return (T + chunks - 1) / chunks;
}

moe_status_t check_sizes(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K,
                         moe_dtype_t dt, bool need_ff) {
    if (dt != MOE_F32 && dt != MOE_BF16)
        return fail(MOE_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)dt);
    if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T = %lld < 0", (long long)T);
    if (d <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "d = %lld <= 0", (long long)d);
    if (need_ff && d_ff <= 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "d_ff = %lld <= 0", (long long)d_ff);
    if (n <= 0) return fail(MOE_ERR_INVALID_ARGUMENT, "n = %d <= 0", n);
    if (K <= 0 || K > n) return fail(MOE_ERR_INVALID_ARGUMENT, "K = %d outside [1, n=%d]", K, n);
    if (n > 64) return fail(MOE_ERR_UNSUPPORTED, "n = %d > 64", n);
    if (K > 8) return fail(MOE_ERR_UNSUPPORTED, "K = %d > 8", K);
    if (d % 8 != 0 || d > kMaxDim)
        return fail(MOE_ERR_UNSUPPORTED, "d = %lld must be a multiple of 8 and <= 2^24",
                    (long long)d);
    if (need_ff && (d_ff % 8 != 0 || d_ff > kMaxDim))
        return fail(MOE_ERR_UNSUPPORTED, "d_ff = %lld must be a multiple of 8 and <= 2^24",
                    (long long)d_ff);
    if (T > kMaxRows / K)
        return fail(MOE_ERR_UNSUPPORTED, "T * K = %lld * %d >= 2^31", (long long)T, K);
    return MOE_OK;
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
    if (!a || !b || an == 0 || bn == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + bn && y < x + an;
}

// ---- backward workspace and the saved training state ----------------------------
// Workspace of moe_backward (bf16): routing and the pre-activation rows
// [a | b] (recomputed), the stack layer's u, then the gradients in
// assignment (expert) order.  The saved state of moe_forward_train /
// moe_block_forward_train is exactly the first seven regions (idx .. U), at
// the same offsets.
struct BwdLayout {
    size_t idx, gate, offsets, perm, inv, AB, DX, dg, DYG, DH, DADB, GH, XG, dl, part, U, meta,
        pcnt, DU, SC, total;
};

constexpr int kBwdMaxSplits = 4;  // K splits of the tiled dx product

// K splits the weight-stream products may use for these sizes: partial sums
// of at most 64 MiB per product, at most 32 splits.
int stream_split_cap(int64_t A, int64_t d, int64_t d_ff) {
    const int64_t row = A * (d > d_ff ? d : d_ff) * 4;
    const int64_t cap = row > 0 ? (int64_t(64) << 20) / row : 32;
    return (int)(cap < 1 ? 1 : cap > 32 ? 32 : cap);
}

// Waves per CU and K splits of a weight-stream K-row product over Kdim rows
// and N columns: the pair whose items (all n experts touched, 512 columns
// each) spread most evenly over the persistent waves; ties go to fewer
// splits.
SkinnyShape choose_stream(int32_t n, int64_t N, int64_t Kdim, int max_splits, int cus) {
    const int64_t ncb = (N + 511) / 512;
    SkinnyShape best{7, 1};
    double best_eff = -1.0;
    for (int s = 1; s <= max_splits; ++s) {
        if (moe::krow_stream_splits_used((int)Kdim, s) != s) continue;
        for (int w = 7; w <= 8; ++w) {
            const int64_t items = (int64_t)n * ncb * s;
            const int64_t nw = (int64_t)cus * w;
            const int64_t rounds = (items + nw - 1) / nw;
            const double eff = (double)items / (double)(rounds * nw);
            if (eff > best_eff + 1e-9) {
                best_eff = eff;
                best = {w, s};
            }
        }
    }
    return best;
}

BwdLayout bwd_layout(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K) {
    const size_t A = (size_t)T * (size_t)K;
    const size_t dd = (size_t)d, ff = (size_t)d_ff;
    // partial sums: the tiled dx product's, or the weight stream's (r, dx)
    const size_t cap = (size_t)stream_split_cap((int64_t)A, d, d_ff);
    const size_t dx_parts = cap > (size_t)kBwdMaxSplits ? cap : (size_t)kBwdMaxSplits;
    const size_t dh_bytes = cap * A * ff * 4 > A * ff * 2 ? cap * A * ff * 4 : A * ff * 2;
    BwdLayout L{};
    size_t o = 0;
    L.idx = o;     o = align256(o + A * 4);
    L.gate = o;    o = align256(o + A * 4);
    L.offsets = o; o = align256(o + (size_t)(n + 1) * 4);
    L.perm = o;    o = align256(o + A * 4);
    L.inv = o;     o = align256(o + A * 4);
    L.AB = o;      o = align256(o + A * 2 * ff * 2);
    // stack layer: u = bf16(RMSNorm(x)) (also part of the saved state)
    L.U = o;       o = align256(o + (size_t)T * dd * 2);
    // (the saved state ends here)
    L.meta = o;    o = align256(o + 2 * 4);  // (R0, Sr) of the tiled dx product
    L.pcnt = o;    o = align256(o + (size_t)moe::permute_blocks((int64_t)A) * (size_t)n * 4);
    L.DX = o;      o = align256(o + dx_parts * A * dd * 4);
    L.dg = o;      o = align256(o + A * 4);
    L.DYG = o;     o = align256(o + A * dd * 2);
    L.DH = o;      o = align256(o + dh_bytes);
    L.DADB = o;    o = align256(o + A * 2 * ff * 2);
    L.GH = o;      o = align256(o + A * ff * 2);
    L.XG = o;      o = align256(o + A * dd * 2);
    L.dl = o;      o = align256(o + (size_t)T * (size_t)n * 4);
    L.part = o;    o = align256(o + (size_t)moe::bwd_dwg_chunks(T) * dd * (size_t)n * 4);
    // stack layer: the gradient with respect to u, the per-token scales
    L.DU = o;      o = align256(o + (size_t)T * dd * 4);
    L.SC = o;      o = align256(o + (size_t)T * 4);
    L.total = o;
    return L;
}

size_t saved_bytes_for(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K) {
    const BwdLayout L = bwd_layout(T, d, d_ff, n, K);
    return L.U + align256((size_t)T * (size_t)d * 2);
}

// ---- the static scratch of moe_forward_noalloc -----------------------------
// For callers that cannot allocate device memory: a file-scope device array
// stands in for the workspace.  Each device that the library runs on holds
// its own copy until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the symbol): the
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.  Every call on one device shares its array; no kernel of
// the forward needs the workspace cleared, so nothing is zeroed.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

moe_status_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "moe_forward_noalloc: device %d >= %d", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "moe_forward_noalloc: hipGetSymbolAddress");
        if (!p) return fail(MOE_ERR_HIP, "moe_forward_noalloc: scratch has no device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MOE_OK;
}

// One pass of the layer over T tokens (at most chunk_tokens): router,
// permutation, the two grouped GEMMs and the combine, launched on `stream`.
// counts_mode: 0 = the permutation writes counts_out; 1 / 2 = the first /
// a later chunk of a chunked call (counts_out set / summed from the offsets).
moe_status_t forward_pass(bool block, const void* x, const void* w_g, const void* w1,
                          const void* w3, const void* w2, int64_t T, int64_t d, int64_t d_ff,
                          int32_t n, int32_t K, moe_dtype_t dt, float eps, void* y,
                          void* workspace, int32_t* idx_out, float* gate_out,
                          int32_t* counts_out, int counts_mode, void* stream, void* saved) {
    const Layout L = layout(T, d, d_ff, n, K, dt);
    const size_t A = (size_t)T * (size_t)K;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(workspace);
    int32_t* idx = idx_out ? idx_out : reinterpret_cast<int32_t*>(ws + L.idx);
    float* gate = gate_out ? gate_out : reinterpret_cast<float*>(ws + L.gate);
    int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
    void* u = ws + L.u;
    uint16_t* save_ab = nullptr;
    if (saved) {  // the routing, the permutation and [a | b] go to the saved state
        const BwdLayout SL = bwd_layout(T, d, d_ff, n, K);
        char* sv = static_cast<char*>(saved);
        idx = reinterpret_cast<int32_t*>(sv + SL.idx);
        gate = reinterpret_cast<float*>(sv + SL.gate);
        offsets = reinterpret_cast<int32_t*>(sv + SL.offsets);
        perm = reinterpret_cast<int32_t*>(sv + SL.perm);
        inv = reinterpret_cast<int32_t*>(sv + SL.inv);
        save_ab = reinterpret_cast<uint16_t*>(sv + SL.AB);
        if (block) u = sv + SL.U;  // the normalised input is saved too
    }
    void* H = ws + L.H;
    float* O = reinterpret_cast<float*>(ws + L.O);
    const bool bf16 = dt == MOE_BF16;
    const Plan plan = choose_plan(T, d, d_ff, n, K, dt);

    hipError_t err = hipSuccess;
    auto mark = [&](hipEvent_t ev) {
        if (ev && err == hipSuccess) err = hipEventRecord(ev, s);
    };
    mark(g_ev_start[MOE_STAGE_ROUTER]);
    if (err == hipSuccess)
        err = moe::launch_router(bf16, block, x, w_g, T, (int)d, n, K, eps, idx, gate, u, s);
    mark(g_ev_end[MOE_STAGE_ROUTER]);
    if (err != hipSuccess) return hip_fail(err, "router launch");
    mark(g_ev_start[MOE_STAGE_PERMUTE]);
    if (err == hipSuccess)
        err = moe::launch_permute(idx, (int64_t)A, n, offsets, perm, inv,
                                  counts_mode == 0 ? counts_out : nullptr, s,
                                  reinterpret_cast<int32_t*>(ws + L.pcnt));
    if (err == hipSuccess && counts_mode != 0 && counts_out)
        err = moe::launch_add_counts(offsets, n, counts_mode == 1, counts_out, s);
    mark(g_ev_end[MOE_STAGE_PERMUTE]);
    if (err != hipSuccess) return hip_fail(err, "permute launch");
    const void* act = block ? u : x;
    int splits = 1;
    int* split_meta = nullptr;  // the tiled down projection's (R0, Sr), for the combine
    const int cus = device_cus();
    SkinnyShape sk_gu{7, 1}, sk_dn{7, 1};
    if (bf16 && plan.skinny) {
        sk_gu = choose_skinny(n, d_ff, d, 1, cus);
        sk_dn = choose_skinny(n, d, d_ff, plan.down_splits, cus);
        splits = sk_dn.splits;
    } else if (bf16) {
        splits = requested_down_splits(T, K);  // at most; the kernel picks Sr from the tiles
        split_meta = reinterpret_cast<int*>(ws + L.meta);
    }
    for (int stage = MOE_STAGE_GATE_UP; stage <= MOE_STAGE_DOWN; ++stage) {
        const bool gu = stage == MOE_STAGE_GATE_UP;
        const void* a_in = gu ? act : H;
        const void* b1 = gu ? w1 : w2;
        const void* b3 = gu ? w3 : nullptr;
        void* c_out = gu ? H : static_cast<void*>(O);
        const int kdim = (int)(gu ? d : d_ff), ndim = (int)(gu ? d_ff : d);
        const int32_t* pm = gu ? perm : nullptr;
        mark(g_ev_start[stage]);
        if (err == hipSuccess) {
            if (!bf16)
                err = moe::launch_gemm_f32(gu, static_cast<const float*>(a_in), pm, K,
                                           static_cast<const float*>(b1),
                                           static_cast<const float*>(b3), offsets, n,
                                           (int64_t)A, kdim, ndim, static_cast<float*>(c_out), s);
            else if (plan.skinny)
                err = moe::launch_gemm_bf16_skinny(gu, static_cast<const uint16_t*>(a_in),
                                                   gu ? T : (int64_t)A, pm, K,
                                                   static_cast<const uint16_t*>(b1),
                                                   static_cast<const uint16_t*>(b3), offsets, n,
                                                   (int64_t)A, kdim, ndim, c_out,
                                                   gu ? 1 : splits,
                                                   gu ? sk_gu.waves : sk_dn.waves, cus, s,
                                                   gu ? save_ab : nullptr);
            else if (gu && save_ab)
                err = moe::launch_gemm_bf16_gateup_save(
                    static_cast<const uint16_t*>(a_in), T, pm, K,
                    static_cast<const uint16_t*>(b1), static_cast<const uint16_t*>(b3), offsets,
                    n, (int64_t)A, kdim, ndim, static_cast<uint16_t*>(c_out), save_ab, s);
            else
                err = moe::launch_gemm_bf16_tiled(gu, static_cast<const uint16_t*>(a_in),
                                                  gu ? T : (int64_t)A, pm, K,
                                                  static_cast<const uint16_t*>(b1),
                                                  static_cast<const uint16_t*>(b3), offsets, n,
                                                  (int64_t)A, kdim, ndim, c_out,
                                                  gu ? 1 : splits, cus, split_meta, s);
        }
        mark(g_ev_end[stage]);
        if (err != hipSuccess) return hip_fail(err, gu ? "gate/up GEMM launch" : "down GEMM launch");
    }
    mark(g_ev_start[MOE_STAGE_COMBINE]);
    if (err == hipSuccess)
        err = moe::launch_combine(bf16, block, O, (int64_t)A, splits, inv, gate, T, K, (int)d, x,
                                  y, split_meta, s);
    mark(g_ev_end[MOE_STAGE_COMBINE]);
    if (err != hipSuccess) return hip_fail(err, "combine launch");
    return MOE_OK;
}


moe_status_t layer_forward(bool block, const void* x, const void* w_g, const void* w1,
                           const void* w3, const void* w2, int64_t T, int64_t d,
                           int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt, float eps,
                           void* y, void* workspace, size_t ws_bytes, int32_t* idx_out,
                           float* gate_out, int32_t* counts_out, void* stream,
                           void* saved = nullptr, size_t saved_bytes = 0,
                           bool static_scratch = false) {
    const char* fn = static_scratch ? "moe_forward_noalloc"
                     : saved ? (block ? "moe_block_forward_train" : "moe_forward_train")
                             : block ? "moe_block_forward" : "moe_forward";
    moe_status_t st = check_sizes(T, d, d_ff, n, K, dt, true);
    if (st != MOE_OK) return st;
    if (saved) {
        if (dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
        if (!aligned(saved, 256))
            return fail(MOE_ERR_INVALID_ARGUMENT, "%s: saved is not 256-byte aligned", fn);
        if (saved_bytes < saved_bytes_for(T, d, d_ff, n, K))
            return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: saved %zu bytes < %zu needed", fn,
                        saved_bytes, saved_bytes_for(T, d, d_ff, n, K));
    }
    if (block && !(eps >= 0.0f && eps < 1e30f))
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);
    const void* ptrs[] = {x, w_g, w1, w3, w2, y};
    const char* names[] = {"x", "w_g", "w1", "w3", "w2", "y"};
    for (int i = 0; i < 6; ++i) {
        // x and y hold T rows: with T = 0 they may be NULL
        if (!ptrs[i] && T == 0 && (i == 0 || i == 5)) continue;
        if (!ptrs[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, names[i]);
        if (!aligned(ptrs[i], 16))
            return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s is not 16-byte aligned", fn, names[i]);
    }
    if ((idx_out && !aligned(idx_out, 4)) || (gate_out && !aligned(gate_out, 4)) ||
        (counts_out && !aligned(counts_out, 4)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: optional outputs must be 4-byte aligned", fn);
    const int64_t cmax = chunk_tokens(d, d_ff, n, K, dt);
    if (cmax <= 0)
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: bf16 expert weights must stay below 2 GiB (d * d_ff < 2^30)", fn);
    // the saved training state and the static scratch hold one pass over all T tokens
    if ((saved || static_scratch) && T > cmax)
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: %lld tokens exceed the %lld one pass can index (%s); split the tokens "
                    "into several calls",
                    fn, (long long)T, (long long)cmax,
                    dt == MOE_BF16 ? "bf16 operands below 2 GiB" : "the fp32 grid bound");
    const int64_t Tc = chunk_len(T, cmax);  // tokens per chunk (T when one pass fits)
    const Layout L = layout(Tc, d, d_ff, n, K, dt);
    if (static_scratch && L.total > kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED,
                    "%s: these sizes need %zu bytes of scratch, the library's static scratch "
                    "holds %zu (enough for 256 tokens at d = 4096, d_ff = 14336, n = 8, K = 2); "
                    "call moe_forward with a workspace instead",
                    fn, L.total, kScratchBytes);
    if (T > 0 && !static_scratch) {
        if (!workspace) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace is NULL", fn);
        if (!aligned(workspace, 256))
            return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace is not 256-byte aligned", fn);
        if (ws_bytes < L.total)
            return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < %zu needed", fn,
                        ws_bytes, L.total);
    }
    const size_t es = dt == MOE_BF16 ? 2 : 4;
    const size_t A = (size_t)T * (size_t)K;
    const size_t ybytes = (size_t)T * (size_t)d * es;
    const size_t wbytes = (size_t)n * (size_t)d_ff * (size_t)d * es;
    if (overlaps(y, ybytes, x, ybytes) || overlaps(y, ybytes, w_g, (size_t)d * n * es) ||
        overlaps(y, ybytes, w1, wbytes) || overlaps(y, ybytes, w3, wbytes) ||
        overlaps(y, ybytes, w2, wbytes) || overlaps(y, ybytes, workspace, L.total) ||
        overlaps(y, ybytes, idx_out, A * 4) || overlaps(y, ybytes, gate_out, A * 4) ||
        overlaps(y, ybytes, counts_out, (size_t)n * 4) || overlaps(y, ybytes, saved, saved_bytes))
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: y overlaps another argument", fn);
    if (saved) {
        const void* others[] = {x, w_g, w1, w3, w2, workspace};
        const size_t osz[] = {ybytes, (size_t)d * n * es, wbytes, wbytes, wbytes, L.total};
        for (int i = 0; i < 6; ++i)
            if (overlaps(saved, saved_bytes, others[i], osz[i]))
                return fail(MOE_ERR_INVALID_ARGUMENT, "%s: saved overlaps another argument", fn);
    }
    if (!static_scratch) {  // the kernels write the workspace while reading the inputs
        const void* others[] = {x, w_g, w1, w3, w2, idx_out, gate_out, counts_out, saved};
        const size_t osz[] = {ybytes, (size_t)d * n * es, wbytes, wbytes, wbytes, A * 4, A * 4,
                              (size_t)n * 4, saved_bytes};
        for (int i = 0; i < 9; ++i)
            if (overlaps(workspace, L.total, others[i], osz[i]))
                return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace overlaps another argument",
                            fn);
    }
    if (T == 0) return MOE_OK;
    if (static_scratch) {
        st = scratch_address(&workspace);
        if (st != MOE_OK) return st;
    }
    (void)hipGetLastError();  // clear a stale error so launch checks report our own
    for (int64_t c0 = 0; c0 < T; c0 += Tc) {
        const int64_t t = T - c0 < Tc ? T - c0 : Tc;
        const size_t xo = (size_t)c0 * (size_t)d * es, ao = (size_t)c0 * (size_t)K;
        st = forward_pass(block, static_cast<const char*>(x) + xo, w_g, w1, w3, w2, t, d, d_ff, n,
                          K, dt, eps, static_cast<char*>(y) + xo, workspace,
                          idx_out ? idx_out + ao : nullptr, gate_out ? gate_out + ao : nullptr,
                          counts_out, Tc < T ? (c0 == 0 ? 1 : 2) : 0, stream, saved);
        if (st != MOE_OK) return st;
    }
    g_last_error[0] = '\0';
    return MOE_OK;
}

moe_status_t layer_backward(const void* x, const void* w_g, const void* w1, const void* w3,
                            const void* w2, const void* dy, int64_t T, int64_t d, int64_t d_ff,
                            int32_t n, int32_t K, moe_dtype_t dt, void* dx, float* dw_g,
                            float* dw1, float* dw3, float* dw2, void* workspace,
                            size_t ws_bytes, void* stream, const void* saved = nullptr,
                            size_t saved_bytes = 0, bool block = false, float eps = 0.0f) {
    const char* fn = saved ? (block ? "moe_block_backward_saved" : "moe_backward_saved")
                           : block ? "moe_block_backward" : "moe_backward";
    moe_status_t st = check_sizes(T, d, d_ff, n, K, dt, true);
    if (st != MOE_OK) return st;
    if (dt != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "%s: bf16 only", fn);
    if (block && !(eps >= 0.0f && eps < 1e30f))
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: eps must be finite and >= 0", fn);

    if (saved) {
        if (!aligned(saved, 256))
            return fail(MOE_ERR_INVALID_ARGUMENT, "%s: saved is not 256-byte aligned", fn);
        if (saved_bytes < saved_bytes_for(T, d, d_ff, n, K))
            return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: saved %zu bytes < %zu needed", fn,
                        saved_bytes, saved_bytes_for(T, d, d_ff, n, K));
    }
    const void* ptrs[] = {x, w_g, w1, w3, w2, dy, dx, dw_g, dw1, dw3, dw2};
    const char* names[] = {"x", "w_g", "w1", "w3", "w2", "dy", "dx", "dw_g", "dw1", "dw3", "dw2"};
    for (int i = 0; i < 11; ++i) {
        const bool rows = i == 0 || i == 5 || i == 6;  // x, dy, dx hold T rows
        if (!ptrs[i] && T == 0 && rows) continue;
        if (!ptrs[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s is NULL", fn, names[i]);
        if (!aligned(ptrs[i], 16))
            return fail(MOE_ERR_INVALID_ARGUMENT, "%s: %s is not 16-byte aligned", fn, names[i]);
    }
    const int64_t A = T * K;
    if (!moe::tiled_fits(T, d, d_ff) || !moe::tiled_fits(A, d_ff, d) ||
        !moe::tiled_fits(A, 2 * d_ff, d) || !moe::tiled_fits(A, d, d_ff))
        return fail(MOE_ERR_UNSUPPORTED, "%s: operands must stay below 2 GiB; split the tokens",
                    fn);
    const BwdLayout L = bwd_layout(T, d, d_ff, n, K);
    if (!workspace) return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace is NULL", fn);
    if (!aligned(workspace, 256))
        return fail(MOE_ERR_INVALID_ARGUMENT, "%s: workspace is not 256-byte aligned", fn);
    if (ws_bytes < L.total)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "%s: workspace %zu bytes < %zu needed", fn,
                    ws_bytes, L.total);
    const size_t xbytes = (size_t)T * (size_t)d * 2;
    const size_t wbytes = (size_t)n * (size_t)d_ff * (size_t)d;
    const void* outs[] = {dx, dw_g, dw1, dw3, dw2, workspace};
    const size_t osz[] = {xbytes, (size_t)d * n * 4, wbytes * 4, wbytes * 4, wbytes * 4, L.total};
    const void* ins[] = {x, w_g, w1, w3, w2, dy};
    const size_t isz[] = {xbytes, (size_t)d * n * 2, wbytes * 2, wbytes * 2, wbytes * 2, xbytes};
    for (int i = 0; i < 6; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], osz[i], ins[j], isz[j]))
                return fail(MOE_ERR_INVALID_ARGUMENT, "%s: an output overlaps an input", fn);
        for (int j = i + 1; j < 6; ++j)
            if (overlaps(outs[i], osz[i], outs[j], osz[j]))
                return fail(MOE_ERR_INVALID_ARGUMENT, "%s: two outputs overlap", fn);
        if (overlaps(outs[i], osz[i], saved, saved_bytes))
            return fail(MOE_ERR_INVALID_ARGUMENT, "%s: an output overlaps the saved state", fn);
    }
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipError_t err = hipSuccess;
    if (T == 0) {  // no tokens: every weight gradient is zero (fill kernels, no memset)
        err = moe::launch_fill_zero(dw_g, (size_t)d * n * 4, s);
        if (err == hipSuccess) err = moe::launch_fill_zero(dw1, wbytes * 4, s);
        if (err == hipSuccess) err = moe::launch_fill_zero(dw3, wbytes * 4, s);
        if (err == hipSuccess) err = moe::launch_fill_zero(dw2, wbytes * 4, s);
        if (err != hipSuccess) return hip_fail(err, "zero gradients");
        g_last_error[0] = '\0';
        return MOE_OK;
    }
    char* ws = static_cast<char*>(workspace);
    // routing, permutation and [a | b]: from the saved state, else recomputed
    // into the same regions of the workspace
    char* rs = saved ? static_cast<char*>(const_cast<void*>(saved)) : ws;
    auto at = [&](size_t off) { return static_cast<void*>(ws + off); };
    int32_t* idx = reinterpret_cast<int32_t*>(rs + L.idx);
    float* gate = reinterpret_cast<float*>(rs + L.gate);
    int32_t* offsets = reinterpret_cast<int32_t*>(rs + L.offsets);
    int32_t* perm = reinterpret_cast<int32_t*>(rs + L.perm);
    int32_t* inv = reinterpret_cast<int32_t*>(rs + L.inv);
    uint16_t* AB = reinterpret_cast<uint16_t*>(rs + L.AB);
    float* DX = static_cast<float*>(at(L.DX));
    float* dg = static_cast<float*>(at(L.dg));
    uint16_t* DYG = static_cast<uint16_t*>(at(L.DYG));
    uint16_t* DH = static_cast<uint16_t*>(at(L.DH));
    uint16_t* DADB = static_cast<uint16_t*>(at(L.DADB));
    uint16_t* GH = static_cast<uint16_t*>(at(L.GH));
    uint16_t* XG = static_cast<uint16_t*>(at(L.XG));
    float* dl = static_cast<float*>(at(L.dl));
    float* part = static_cast<float*>(at(L.part));
    uint16_t* U = reinterpret_cast<uint16_t*>(rs + L.U);  // saved state or workspace
    float* DU = static_cast<float*>(at(L.DU));
    float* SC = static_cast<float*>(at(L.SC));
    const uint16_t* x_in = static_cast<const uint16_t*>(x);
    // the experts' input: x, or for the stack layer u = bf16(RMSNorm(x))
    // (written by the router, which routes on the fp32 u)
    const uint16_t* xb = block ? U : x_in;
    const uint16_t* w1b = static_cast<const uint16_t*>(w1);
    const uint16_t* w3b = static_cast<const uint16_t*>(w3);
    const uint16_t* w2b = static_cast<const uint16_t*>(w2);
    const int D = (int)d, F = (int)d_ff;
#define STEP(call, what)                                  \
    do {                                                  \
        if (err == hipSuccess) {                          \
            err = (call);                                 \
            if (err != hipSuccess) return hip_fail(err, what); \
        }                                                 \
    } while (0)
    auto mark = [&](hipEvent_t ev) {
        if (ev && err == hipSuccess) err = hipEventRecord(ev, s);
        if (err != hipSuccess) return false;
        return true;
    };
    const int cus = device_cus();
    // the forward's GEMM family: MFMA tiles, or weight streams for few rows
    // per expert
    const Plan plan = choose_plan(T, d, d_ff, n, K, dt);
    // the tiled dx product splits K for its last round's tiles only (at most
    // kBwdMaxSplits), recording (R0, Sr) for the token kernel
    int dx_splits = kBwdMaxSplits;
    int* dx_meta = reinterpret_cast<int*>(ws + L.meta);
    SkinnyShape st_r{7, 1}, st_x{7, 1};
    if (plan.skinny) {
        dx_meta = nullptr;
        const int cap = stream_split_cap(A, d, d_ff);
        st_r = choose_stream(n, d_ff, d, cap, cus);
        st_x = choose_stream(n, d, 2 * d_ff, cap, cus);
        dx_splits = st_x.splits;
    }
    // routing and the pre-activations [a | b] recomputed, on the same kernels
    // as the forward's (so a saved state from moe_forward_train is identical)
    if (!mark(g_ev_start[MOE_STAGE_BWD_RECOMPUTE])) return hip_fail(err, "event record");
    if (!saved) {
        STEP(moe::launch_router(true, block, x, w_g, T, D, n, K, eps, idx, gate,
                                block ? U : nullptr, s),
             "router");
        STEP(moe::launch_permute(idx, A, n, offsets, perm, inv, nullptr, s,
                                 reinterpret_cast<int32_t*>(ws + L.pcnt)),
             "permute");
        if (plan.skinny) {
            const SkinnyShape sk = choose_skinny(n, d_ff, d, 1, cus);
            STEP(moe::launch_gemm_bf16_skinny(true, xb, T, perm, K, w1b, w3b, offsets, n, A, D,
                                              F, nullptr, 1, sk.waves, cus, s, AB),
                 "gate/up recompute");
        } else {
            STEP(moe::launch_gemm_bf16_gateup_ab(xb, T, perm, K, w1b, w3b, offsets, n, A, D, F,
                                                 AB, s),
                 "gate/up recompute");
        }
    }
    if (!mark(g_ev_end[MOE_STAGE_BWD_RECOMPUTE])) return hip_fail(err, "event record");
    if (!mark(g_ev_start[MOE_STAGE_BWD_DH])) return hip_fail(err, "event record");
    // tokens and output gradients of every assignment in expert order
    STEP(moe::launch_gather_rows(xb, static_cast<const uint16_t*>(dy), perm, K, A, D, XG, DYG, s),
         "row gather");
    // r = dy W2_e (W2_e [d][d_ff] read as K rows), then per row: dg = h . r,
    // [da | db] of g r, g h
    if (plan.skinny) {
        float* DHP = reinterpret_cast<float*>(DH);
        STEP(moe::launch_gemm_bf16_krow_stream(DYG, A, w2b, nullptr, D, offsets, n, D, F, DHP,
                                               st_r.splits, st_r.waves, cus, s),
             "dh product");
        STEP(moe::launch_bwd_swiglu(AB, nullptr, DHP, st_r.splits, perm, gate, A, F, dg, DADB,
                                    GH, s),
             "SwiGLU backward");
    } else {
        STEP(moe::launch_gemm_bf16_krow(DYG, A, w2b, nullptr, D, offsets, n, D, F, DH, true, 1,
                                        cus, nullptr, s),
             "dh product");
        STEP(moe::launch_bwd_swiglu(AB, DH, nullptr, 1, perm, gate, A, F, dg, DADB, GH, s),
             "SwiGLU backward");
    }
    if (!mark(g_ev_end[MOE_STAGE_BWD_DH])) return hip_fail(err, "event record");
    if (!mark(g_ev_start[MOE_STAGE_BWD_DX])) return hip_fail(err, "event record");
    // dx per assignment = da W1_e + db W3_e: K rows 0..d_ff-1 from W1_e, the
    // next d_ff from W3_e, against the rows [da | db]; K-split partials
    if (plan.skinny)
        STEP(moe::launch_gemm_bf16_krow_stream(DADB, A, w1b, w3b, F, offsets, n, 2 * F, D, DX,
                                               st_x.splits, st_x.waves, cus, s),
             "dx product");
    else
        STEP(moe::launch_gemm_bf16_krow(DADB, A, w1b, w3b, F, offsets, n, 2 * F, D, DX, false,
                                        dx_splits, cus, dx_meta, s),
             "dx product");
    // router gradient, dx back in token order, dW_g
    STEP(moe::launch_bwd_token(static_cast<const uint16_t*>(w_g), idx, gate, dg, DX, dx_splits,
                               A, inv, T, K, n, D, dl,
                               block ? nullptr : static_cast<uint16_t*>(dx), block ? DU : nullptr,
                               dx_meta, s),
         "token gradients");
    if (block)  // through the normalisation, plus the residual
        STEP(moe::launch_bwd_rms(x_in, static_cast<const uint16_t*>(dy), DU, T, D, eps,
                                 static_cast<uint16_t*>(dx), SC, s),
             "normalisation backward");
    // dW_g = sum u dl^T with the router's own input: x, or the fp32 u = x s
    STEP(moe::launch_bwd_dwg(x_in, block ? SC : nullptr, dl, T, D, n, part, dw_g, s),
         "router weight gradient");
    if (!mark(g_ev_end[MOE_STAGE_BWD_DX])) return hip_fail(err, "event record");
    if (!mark(g_ev_start[MOE_STAGE_BWD_WGRAD])) return hip_fail(err, "event record");
    // weight gradients over each expert's rows: dW2_e = dy^T (g h),
    // dW1_e = da^T u, dW3_e = db^T u
    // row groups of 4 tiles (measured: 7% faster than one group per expert)
    const int wg_gm = 4;
    STEP(moe::launch_gemm_bf16_wgrad(DYG, D, GH, F, offsets, n, A, D, F, dw2, wg_gm, s), "dW2");
    STEP(moe::launch_gemm_bf16_wgrad(DADB, 2 * (int64_t)F, XG, D, offsets, n, A, F, D, dw1,
                                     wg_gm, s),
         "dW1");
    STEP(moe::launch_gemm_bf16_wgrad(DADB + F, 2 * (int64_t)F, XG, D, offsets, n, A, F, D, dw3,
                                     wg_gm, s),
         "dW3");
    if (!mark(g_ev_end[MOE_STAGE_BWD_WGRAD])) return hip_fail(err, "event record");
#undef STEP
    g_last_error[0] = '\0';
    return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(moe_status_t st) {
    switch (st) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
        default: return "MOE_ERR_UNKNOWN";
    }
}

const char* moe_last_error(void) { return g_last_error; }

size_t moe_workspace_bytes(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K,
                           moe_dtype_t dt) {
    if (check_sizes(T, d, d_ff, n, K, dt, true) != MOE_OK) return 0;
    return layout(chunk_len(T, chunk_tokens(d, d_ff, n, K, dt)), d, d_ff, n, K, dt).total;
}

moe_status_t moe_route(const void* x, const void* w_g, int64_t T, int64_t d, int32_t n,
                       int32_t K, moe_dtype_t dt, int32_t* idx, float* gate, void* stream) {
    moe_status_t st = check_sizes(T, d, 8, n, K, dt, false);
    if (st != MOE_OK) return st;
    if (!x || !w_g || !idx || !gate)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_route: NULL pointer argument");
    if (!aligned(x, 16) || !aligned(w_g, 16) || !aligned(idx, 4) || !aligned(gate, 4))
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_route: misaligned pointer argument");
    const size_t A = (size_t)T * (size_t)K;
    if (overlaps(idx, A * 4, gate, A * 4))
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_route: idx and gate overlap");
    if (T == 0) return MOE_OK;
    (void)hipGetLastError();
    hipError_t err = moe::launch_router(dt == MOE_BF16, false, x, w_g, T, (int)d, n, K, 0.0f,
                                        idx, gate, nullptr, reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "router launch");
    g_last_error[0] = '\0';
    return MOE_OK;
}

moe_status_t moe_permute(const int32_t* idx, int64_t T, int32_t n, int32_t K, int32_t* offsets,
                         int32_t* perm, int32_t* inv, void* stream) {
    moe_status_t st = check_sizes(T, 8, 8, n, K, MOE_F32, false);
    if (st != MOE_OK) return st;
    if (!idx || !offsets || !perm || !inv)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_permute: NULL pointer argument");
    if (!aligned(idx, 4) || !aligned(offsets, 4) || !aligned(perm, 4) || !aligned(inv, 4))
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_permute: misaligned pointer argument");
    if (T == 0) return MOE_OK;
    (void)hipGetLastError();
    hipError_t err = moe::launch_permute(idx, T * K, n, offsets, perm, inv, nullptr,
                                         reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) return hip_fail(err, "permute launch");
    g_last_error[0] = '\0';
    return MOE_OK;
}

moe_status_t moe_set_stage_events(int32_t stage, void* start_event, void* end_event) {
    if (stage < 0 || stage >= kStages)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_set_stage_events: stage %d", stage);
    if ((start_event == nullptr) != (end_event == nullptr))
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_set_stage_events: give both events or none");
    g_ev_start[stage] = static_cast<hipEvent_t>(start_event);
    g_ev_end[stage] = static_cast<hipEvent_t>(end_event);
    return MOE_OK;
}

moe_status_t moe_forward_noalloc(const void* x, const void* w_g, const void* w1,
                                 const void* w3, const void* w2, int64_t T, int64_t d,
                                 int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt, void* y,
                                 int32_t* idx_out, float* gate_out, int32_t* counts_out,
                                 void* stream) {
    return layer_forward(false, x, w_g, w1, w3, w2, T, d, d_ff, n, K, dt, 0.0f, y, nullptr, 0,
                         idx_out, gate_out, counts_out, stream, nullptr, 0, true);
}

moe_status_t moe_set_gemm_path(int32_t path) {
    if (path < MOE_GEMM_AUTO || path > MOE_GEMM_STREAM)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_set_gemm_path: path %d", path);
    g_gemm_path = path;
    return MOE_OK;
}

moe_status_t moe_forward(const void* x, const void* w_g, const void* w1, const void* w3,
                         const void* w2, int64_t T, int64_t d, int64_t d_ff, int32_t n,
                         int32_t K, moe_dtype_t dt, void* y, void* workspace,
                         size_t workspace_bytes, int32_t* idx_out, float* gate_out,
                         int32_t* counts_out, void* stream) {
    return layer_forward(false, x, w_g, w1, w3, w2, T, d, d_ff, n, K, dt, 0.0f, y, workspace,
                         workspace_bytes, idx_out, gate_out, counts_out, stream);
}

moe_status_t moe_block_forward(const void* x, const void* w_g, const void* w1, const void* w3,
                               const void* w2, int64_t T, int64_t d, int64_t d_ff, int32_t n,
                               int32_t K, moe_dtype_t dt, float eps, void* y, void* workspace,
                               size_t workspace_bytes, int32_t* idx_out, float* gate_out,
                               int32_t* counts_out, void* stream) {
    return layer_forward(true, x, w_g, w1, w3, w2, T, d, d_ff, n, K, dt, eps, y, workspace,
                         workspace_bytes, idx_out, gate_out, counts_out, stream);
}

size_t moe_backward_workspace_bytes(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K,
                                    moe_dtype_t dt) {
    if (check_sizes(T, d, d_ff, n, K, dt, true) != MOE_OK || dt != MOE_BF16) return 0;
    return bwd_layout(T, d, d_ff, n, K).total;
}

size_t moe_saved_bytes(int64_t T, int64_t d, int64_t d_ff, int32_t n, int32_t K,
                       moe_dtype_t dt) {
    if (check_sizes(T, d, d_ff, n, K, dt, true) != MOE_OK || dt != MOE_BF16) return 0;
    return saved_bytes_for(T, d, d_ff, n, K);
}

moe_status_t moe_forward_train(const void* x, const void* w_g, const void* w1, const void* w3,
                               const void* w2, int64_t T, int64_t d, int64_t d_ff, int32_t n,
                               int32_t K, moe_dtype_t dt, void* y, void* saved,
                               size_t saved_bytes, void* workspace, size_t workspace_bytes,
                               void* stream) {
    if (!saved) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_forward_train: saved is NULL");
    return layer_forward(false, x, w_g, w1, w3, w2, T, d, d_ff, n, K, dt, 0.0f, y, workspace,
                         workspace_bytes, nullptr, nullptr, nullptr, stream, saved, saved_bytes);
}

moe_status_t moe_backward_saved(const void* x, const void* w_g, const void* w1, const void* w3,
                                const void* w2, const void* dy, const void* saved,
                                size_t saved_bytes, int64_t T, int64_t d, int64_t d_ff,
                                int32_t n, int32_t K, moe_dtype_t dt, void* dx, float* dw_g,
                                float* dw1, float* dw3, float* dw2, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (!saved) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_backward_saved: saved is NULL");
    return layer_backward(x, w_g, w1, w3, w2, dy, T, d, d_ff, n, K, dt, dx, dw_g, dw1, dw3, dw2,
                          workspace, workspace_bytes, stream, saved, saved_bytes);
}

moe_status_t moe_block_forward_train(const void* x, const void* w_g, const void* w1,
                                     const void* w3, const void* w2, int64_t T, int64_t d,
                                     int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt,
                                     float eps, void* y, void* saved, size_t saved_bytes,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    if (!saved) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_block_forward_train: saved is NULL");
    return layer_forward(true, x, w_g, w1, w3, w2, T, d, d_ff, n, K, dt, eps, y, workspace,
                         workspace_bytes, nullptr, nullptr, nullptr, stream, saved, saved_bytes);
}

moe_status_t moe_block_backward_saved(const void* x, const void* w_g, const void* w1,
                                      const void* w3, const void* w2, const void* dy,
                                      const void* saved, size_t saved_bytes, int64_t T,
                                      int64_t d, int64_t d_ff, int32_t n, int32_t K,
                                      moe_dtype_t dt, float eps, void* dx, float* dw_g,
                                      float* dw1, float* dw3, float* dw2, void* workspace,
                                      size_t workspace_bytes, void* stream) {
    if (!saved)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_block_backward_saved: saved is NULL");
    return layer_backward(x, w_g, w1, w3, w2, dy, T, d, d_ff, n, K, dt, dx, dw_g, dw1, dw3, dw2,
                          workspace, workspace_bytes, stream, saved, saved_bytes, true, eps);
}

moe_status_t moe_block_backward(const void* x, const void* w_g, const void* w1,
                                const void* w3, const void* w2, const void* dy, int64_t T,
                                int64_t d, int64_t d_ff, int32_t n, int32_t K, moe_dtype_t dt,
                                float eps, void* dx, float* dw_g, float* dw1, float* dw3,
                                float* dw2, void* workspace, size_t workspace_bytes,
                                void* stream) {
    return layer_backward(x, w_g, w1, w3, w2, dy, T, d, d_ff, n, K, dt, dx, dw_g, dw1, dw3, dw2,
                          workspace, workspace_bytes, stream, nullptr, 0, true, eps);
}

moe_status_t moe_backward(const void* x, const void* w_g, const void* w1, const void* w3,
                          const void* w2, const void* dy, int64_t T, int64_t d, int64_t d_ff,
                          int32_t n, int32_t K, moe_dtype_t dt, void* dx, float* dw_g,
                          float* dw1, float* dw3, float* dw2, void* workspace,
                          size_t workspace_bytes, void* stream) {
    return layer_backward(x, w_g, w1, w3, w2, dy, T, d, d_ff, n, K, dt, dx, dw_g, dw1, dw3, dw2,
                          workspace, workspace_bytes, stream);
}

}  // extern "C"
