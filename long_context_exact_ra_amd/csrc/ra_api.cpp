// ra_api.cpp -- the C ABI of the ring-attention share library (include/ra.h):
// argument validation, the ring schedule, the grouped-query head map, and
// dispatch to the gfx950 kernels.  Validation happens before any HIP call, so a
// rejected call neither touches the device nor enqueues work.
#include "../../include/ra.h"

#include <atomic>
#include <cstdint>
#include <cmath>
#include <cstdlib>
#include <cstring>

#include "ra_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return RA_EHIP;
}

bool debug_sync() {
    static const bool on = [] {
        const char *v = std::getenv("RA_DEBUG");
        return v && v[0] && std::strcmp(v, "0") != 0;
    }();
    return on;
}

// After a launch: report a launch error, and in RA_DEBUG mode wait for the
// stream so that a fault is attributed to the call that caused it.
int after_launch(hipError_t e, hipStream_t st) {
    if (e != hipSuccess) return hip_fail(e);
    if (debug_sync()) {
        e = hipStreamSynchronize(st);
        if (e != hipSuccess) return hip_fail(e);
    }
    return RA_OK;
}

// 0 unknown, 1 gfx950, 2 other architecture; indexed by device ordinal.
std::atomic<int> g_device_kind[64];

int check_device() {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev >= 0 && dev < 64) {
        const int k = g_device_kind[dev].load(std::memory_order_relaxed);
        if (k == 1) return RA_OK;
        if (k == 2) return RA_ENOTSUP;
    }
    hipDeviceProp_t p;
    e = hipGetDeviceProperties(&p, dev);
    if (e != hipSuccess) return hip_fail(e);
    const bool ok = std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
    if (dev >= 0 && dev < 64) g_device_kind[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? RA_OK : RA_ENOTSUP;
}

// Size arithmetic of the checks below, over non-negative operands.  A product that does
// not fit int64 saturates at INT64_MAX, so an absurd size is rejected instead of wrapping
// round (signed overflow), and a rounded-up quotient never forms a + b - 1.
int64_t sat_mul(int64_t a, int64_t b) {
    if (a == 0 || b == 0) return 0;
    return a > INT64_MAX / b ? INT64_MAX : a * b;
}

template <class... R>
int64_t sat_mul(int64_t a, int64_t b, int64_t c, R... r) {
    return sat_mul(sat_mul(a, b), c, (int64_t)r...);
}

int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// True if a tensor of these extents, at up to 8 bytes an element, has a byte size (and so
// every element and byte offset the kernels form) that fits int64.
template <class... E>
bool extent_ok(E... e) {
    return sat_mul(8, (int64_t)e...) < INT64_MAX;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool ptr_ok(const void *p) { return p != nullptr && aligned16(p); }

bool opt_ptr_ok(const void *p) { return p == nullptr || aligned16(p); }

bool heads_ok(int32_t B, int32_t H, int32_t H_kv, int32_t d, int32_t dtype) {
    return B >= 1 && H >= 1 && H_kv >= 1 && H % H_kv == 0 && (d == 64 || d == 128) &&
           (dtype == RA_F32 || dtype == RA_BF16);
}

bool scale_ok(float scale) { return std::isfinite(scale) && scale > 0.f; }

// The bf16 kernel reads one K/V head through a buffer resource with a 32-bit range.
bool head_range_ok(int32_t dtype, int64_t rows, int32_t d) {
    return dtype != RA_BF16 || rows <= (int64_t)INT32_MAX / (2 * d);
}

// Work-group count of the forward kernels; false if it does not fit a 1-D grid.
bool grid_size(int32_t B, int32_t H, int64_t l_q, int32_t dtype, int32_t *n_qtiles,
               int32_t *n_wg) {
    const int64_t tile = dtype == RA_BF16 ? ra::bf16_query_tile() : ra::kF32QueryTile;
    const int64_t qt = ceil_div(l_q, tile);
    const int64_t total = sat_mul(qt, B, H);
    if (qt > INT32_MAX || total > INT32_MAX) return false;
    *n_qtiles = (int32_t)qt;
    *n_wg = (int32_t)total;
    return true;
}

int launch_fwd(const ra::FwdArgs &a, int32_t B, int32_t d, int32_t dtype, int mode,
               hipStream_t st) {
    const hipError_t e = dtype == RA_BF16 ? ra::launch_fwd_bf16(a, B, d, mode, st)
                                          : ra::launch_fwd_f32(a, B, d, mode, st);
    return after_launch(e, st);
}

int share_launch(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv, int32_t d,
                 int32_t B, int32_t dtype, int32_t layout, const void *Q_i, const void *K,
                 const void *V, float scale, float *O, float *m_out, float *l_out,
                 void *O_cast, int32_t *sched_trace, void *stream) {
    if (N < 1 || rank < 0 || rank >= N || L < 0 || L % N != 0 ||
        !heads_ok(B, H, H_kv, d, dtype) || !scale_ok(scale))
        return RA_EINVAL;
    if (L == 0) return RA_OK;
    if (!ptr_ok(Q_i) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(O) || !opt_ptr_ok(m_out) ||
        !opt_ptr_ok(l_out) || !opt_ptr_ok(O_cast) ||
        (sched_trace != nullptr && ((uintptr_t)sched_trace & 3u) != 0))
        return RA_EINVAL;
    if (!head_range_ok(dtype, L, d) || !extent_ok(B, H_kv, L, d)) return RA_ENOTSUP;
    const int64_t l = L / N;
    ra::FwdArgs a{};
    if (!grid_size(B, H, l, dtype, &a.n_qtiles, &a.n_wg)) return RA_ENOTSUP;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    a.Q = Q_i;
    a.K = K;
    a.V = V;
    a.O = O;
    a.m = m_out;
    a.l = l_out;
    a.O_cast = O_cast;
    a.trace = sched_trace;
    a.l_q = l;
    a.blk_rows = l;
    a.kv_head_stride = L * d;
    a.kv_batch_stride = (int64_t)H_kv * L * d;
    a.n_blocks = N;
    a.rank = rank;
    a.H = H;
    a.H_kv = H_kv;
    a.group = H / H_kv;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.layout = layout;
    return launch_fwd(a, B, d, dtype, ra::MODE_SHARE, (hipStream_t)stream);
}

// Shared by ra_share_backward (layout kNoCausal) and ra_causal_share_backward.
// With validate_only, it returns after the argument checks (no HIP call at all).
int backward_launch(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv, int32_t d,
                    int32_t B, int32_t dtype, int32_t layout, const void *Q_i, const void *K,
                    const void *V, const float *O, const void *dO, const float *m,
                    const float *l, float scale, float *dQ, float *dK, float *dV,
                    void *workspace, void *stream, bool validate_only = false) {
    if (N < 1 || rank < 0 || rank >= N || L < 0 || L % N != 0 ||
        !heads_ok(B, H, H_kv, d, dtype) || !scale_ok(scale))
        return RA_EINVAL;
    if (L == 0) return RA_OK;
    if (!ptr_ok(Q_i) || !ptr_ok(K) || !ptr_ok(V) || !ptr_ok(O) || !ptr_ok(dO) || !ptr_ok(m) ||
        !ptr_ok(l) || !ptr_ok(dQ) || !ptr_ok(dK) || !ptr_ok(dV) || !ptr_ok(workspace))
        return RA_EINVAL;
    if (dtype != RA_BF16) return RA_ENOTSUP;  // the backward kernels take bf16 inputs
    const int64_t lq = L / N;
    if (!head_range_ok(dtype, L, d) || !head_range_ok(dtype, lq, d) ||
        lq > (int64_t)INT32_MAX / 8)  // one head's statistics through a 32-bit buffer range
        return RA_ENOTSUP;
    const bool causal = layout != ra::kNoCausal;
    const int64_t kblk = causal ? lq : L;
    const int64_t nkb = causal ? N : 1;
    const int64_t qt = ceil_div(lq, ra::bwd_query_tile());
    const int64_t kpb = ceil_div(kblk, ra::bwd_key_tile());
    const int64_t kt = kpb * nkb;
    if (sat_mul(qt, B, H) > INT32_MAX || sat_mul(kt, B, H_kv) > INT32_MAX) return RA_ENOTSUP;
    if (validate_only) return RA_OK;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    ra::BwdArgs a{};
    a.Q = Q_i;
    a.K = K;
    a.V = V;
    a.dO = dO;
    a.ws = (float *)workspace;
    a.dQ = dQ;
    a.dK = dK;
    a.dV = dV;
    a.l_q = lq;
    a.L = L;
    a.kv_head_stride = L * d;
    a.kv_batch_stride = (int64_t)H_kv * L * d;
    a.H = H;
    a.H_kv = H_kv;
    a.group = H / H_kv;
    a.n_qtiles = (int32_t)qt;
    a.n_wg = (int32_t)(qt * B * H);
    a.n_ktiles = (int32_t)kt;
    a.n_kv_wg = (int32_t)(kt * B * H_kv);
    a.n_kblocks = (int32_t)nkb;
    a.kblk_rows = kblk;
    a.n_ktiles_blk = (int32_t)kpb;
    a.layout = layout;
    a.rank = rank;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    hipStream_t st = (hipStream_t)stream;
    return after_launch(
        ra::launch_bwd_bf16(a, O, dO, m, l, (int64_t)B * H * lq, d, st), st);
}

// Shared by ra_share_forward_fp8 (layout kNoCausal) and ra_causal_share_forward_fp8.
int fp8_share_launch(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv, int32_t d,
                     int32_t B, int32_t layout, const void *Q8, const float *q_descale,
                     const void *K8, const float *k_descale, const void *V8t,
                     const float *v_descale, float scale, float *O, float *m_out, float *l_out,
                     void *O_cast, void *stream) {
    if (N < 1 || rank < 0 || rank >= N || L < 0 || L % N != 0 ||
        !heads_ok(B, H, H_kv, d, RA_BF16) || !scale_ok(scale))
        return RA_EINVAL;
    if (L == 0) return RA_OK;
    if (!ptr_ok(Q8) || !ptr_ok(q_descale) || !ptr_ok(K8) || !ptr_ok(k_descale) ||
        !ptr_ok(V8t) || !ptr_ok(v_descale) || !ptr_ok(O) || !opt_ptr_ok(m_out) ||
        !opt_ptr_ok(l_out) || !opt_ptr_ok(O_cast))
        return RA_EINVAL;
    const int64_t l = L / N;
    const int64_t T = ceil_div(l, 64);
    // one K head and one V head are each addressed through a 32-bit byte range
    if (sat_mul(L, d) > INT32_MAX || sat_mul(N, T, 64, d) > INT32_MAX ||
        sat_mul(N, T, 4) > INT32_MAX)
        return RA_ENOTSUP;
    const int64_t qt = ceil_div(l, ra::fp8_query_tile());
    if (sat_mul(qt, B, H) > INT32_MAX) return RA_ENOTSUP;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    ra::Fp8Args a{};
    a.Q8 = (const uint8_t *)Q8;
    a.qs = q_descale;
    a.K8 = (const uint8_t *)K8;
    a.ks = k_descale;
    a.V8 = (const uint8_t *)V8t;
    a.vs = v_descale;
    a.O = O;
    a.m = m_out;
    a.l = l_out;
    a.O_cast = O_cast;
    a.l_q = l;
    a.n_blocks = N;
    a.rank = rank;
    a.H = H;
    a.H_kv = H_kv;
    a.group = H / H_kv;
    a.n_tiles_blk = (int32_t)T;
    a.n_qtiles = (int32_t)qt;
    a.n_wg = (int32_t)(qt * B * H);
    a.scale = scale;
    a.layout = layout;
    hipStream_t st = (hipStream_t)stream;
    return after_launch(ra::launch_fwd_fp8(a, d, st), st);
}

}  // namespace

extern "C" {

int32_t ra_ring_block(int32_t rank, int32_t N, int32_t t) {
    if (N < 1 || rank < 0 || rank >= N || t < 0 || t >= N) return -RA_EINVAL;
    // (rank - t) mod N with the non-negative remainder; both are in [0, N).
    const int32_t j = rank - t;
    return j < 0 ? j + N : j;
}

int ra_ring_schedule(int32_t rank, int32_t N, int32_t *out) {
    if (N < 1 || rank < 0 || rank >= N || out == nullptr) return RA_EINVAL;
    for (int32_t t = 0; t < N; ++t) out[t] = ra_ring_block(rank, N, t);
    return RA_OK;
}

int32_t ra_kv_head(int32_t h, int32_t H, int32_t H_kv) {
    if (H < 1 || H_kv < 1 || H % H_kv != 0 || h < 0 || h >= H) return -RA_EINVAL;
    return h / (H / H_kv);
}

int ra_state_init(float *O_acc, float *m, float *l, const ra_shape *s, void *stream) {
    if (s == nullptr || !heads_ok(s->B, s->H, s->H_kv, s->d, s->dtype) || s->l_q < 0)
        return RA_EINVAL;
    if (!extent_ok(s->B, s->H, s->l_q, s->d)) return RA_ENOTSUP;
    const int64_t rows = (int64_t)s->B * s->H * s->l_q;
    if (rows == 0) return RA_OK;
    if (!ptr_ok(O_acc) || !ptr_ok(m) || !ptr_ok(l)) return RA_EINVAL;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    return after_launch(ra::launch_state_init(O_acc, m, l, rows, s->d, st), st);
}

int ra_step(const void *Q_i, const void *K_blk, const void *V_blk, float *O_acc, float *m,
            float *l, float scale, const ra_shape *s, void *stream) {
    if (s == nullptr || !heads_ok(s->B, s->H, s->H_kv, s->d, s->dtype) || s->l_q < 0 ||
        s->l_kv < 0 || !scale_ok(scale) || s->kv_head_stride < 0 || s->kv_batch_stride < 0)
        return RA_EINVAL;
    if (!extent_ok(s->l_kv, s->d)) return RA_ENOTSUP;
    const int64_t blk = s->l_kv * s->d;
    const int64_t hs = s->kv_head_stride ? s->kv_head_stride : blk;
    if (hs < blk || hs % 8 != 0) return RA_EINVAL;
    // H_kv heads at stride hs, then B batch entries at stride bs, must stay addressable
    if (!extent_ok(s->H_kv, hs)) return RA_ENOTSUP;
    const int64_t bs = s->kv_batch_stride ? s->kv_batch_stride : (int64_t)s->H_kv * hs;
    if (bs % 8 != 0 || bs < (int64_t)(s->H_kv - 1) * hs + blk) return RA_EINVAL;
    if (!extent_ok(s->B, bs) || !extent_ok(s->B, s->H, s->l_q, s->d)) return RA_ENOTSUP;
    if (s->l_q == 0 || s->l_kv == 0) return RA_OK;
    if (!ptr_ok(Q_i) || !ptr_ok(K_blk) || !ptr_ok(V_blk) || !ptr_ok(O_acc) || !ptr_ok(m) ||
        !ptr_ok(l))
        return RA_EINVAL;
    if (!head_range_ok(s->dtype, s->l_kv, s->d)) return RA_ENOTSUP;
    ra::FwdArgs a{};
    if (!grid_size(s->B, s->H, s->l_q, s->dtype, &a.n_qtiles, &a.n_wg)) return RA_ENOTSUP;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    a.Q = Q_i;
    a.K = K_blk;
    a.V = V_blk;
    a.O = O_acc;
    a.m = m;
    a.l = l;
    a.l_q = s->l_q;
    a.blk_rows = s->l_kv;
    a.kv_head_stride = hs;
    a.kv_batch_stride = bs;
    a.n_blocks = 1;
    a.rank = 0;
    a.layout = ra::kNoCausal;
    a.H = s->H;
    a.H_kv = s->H_kv;
    a.group = s->H / s->H_kv;
    a.scale = scale;
    a.scale_log2 = scale * 1.4426950408889634f;
    return launch_fwd(a, s->B, s->d, s->dtype, ra::MODE_STEP, (hipStream_t)stream);
}

int ra_finalize(float *O_acc, const float *l, const ra_shape *s, void *O_out, void *stream) {
    if (s == nullptr || !heads_ok(s->B, s->H, s->H_kv, s->d, s->dtype) || s->l_q < 0)
        return RA_EINVAL;
    if (!extent_ok(s->B, s->H, s->l_q, s->d)) return RA_ENOTSUP;
    const int64_t rows = (int64_t)s->B * s->H * s->l_q;
    if (rows == 0) return RA_OK;
    if (!ptr_ok(O_acc) || !ptr_ok(l) || !opt_ptr_ok(O_out)) return RA_EINVAL;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    return after_launch(ra::launch_finalize(O_acc, l, rows, s->d, s->dtype, O_out, st), st);
}

int ra_share_forward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                     int32_t d, int32_t B, int32_t dtype, const void *Q_i, const void *K,
                     const void *V, float scale, float *O, float *m_out, float *l_out,
                     void *O_cast, int32_t *sched_trace, void *stream) {
    return share_launch(rank, N, L, H, H_kv, d, B, dtype, ra::kNoCausal, Q_i, K, V, scale, O,
                        m_out, l_out, O_cast, sched_trace, stream);
}

int ra_causal_share_forward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                            int32_t d, int32_t B, int32_t dtype, int32_t layout,
                            const void *Q_i, const void *K, const void *V, float scale,
                            float *O, float *m_out, float *l_out, void *O_cast, void *stream) {
    if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED &&
        layout != RA_LAYOUT_ZIGZAG)
        return RA_EINVAL;
    // Zigzag: each half-block must be whole 64-key tiles, so no key tile straddles the
    // two chunks a member holds.
    if (layout == RA_LAYOUT_ZIGZAG && N >= 1 && L >= 0 && L % N == 0 && (L / N) % 128 != 0)
        return RA_EINVAL;
    return share_launch(rank, N, L, H, H_kv, d, B, dtype, layout, Q_i, K, V, scale, O, m_out,
                        l_out, O_cast, nullptr, stream);
}

int64_t ra_causal_pairs(int32_t rank, int32_t N, int64_t L, int32_t layout) {
    if (N < 1 || rank < 0 || rank >= N || L < 0 || L % N != 0) return -RA_EINVAL;
    // 128-bit arithmetic: every term below is at most L * l < 2^126, so none overflows.
    const __int128 l = L / N, r = rank, n = N;
    __int128 pairs;
    switch (layout) {
    case RA_LAYOUT_CONTIGUOUS:  // queries r*l + x see r*l + x + 1 keys
        pairs = l * r * l + l * (l + 1) / 2;
        break;
    case RA_LAYOUT_STRIPED:  // queries x*N + r see x*N + r + 1 keys
        pairs = n * (l * (l - 1) / 2) + l * (r + 1);
        break;
    case RA_LAYOUT_ZIGZAG: {  // chunk r then chunk 2N-1-r, h tokens each
        if (l % 2) return -RA_EINVAL;
        const __int128 h = l / 2;
        pairs = h * (r * h) + h * (h + 1) / 2 + h * ((2 * n - 1 - r) * h) + h * (h + 1) / 2;
        break;
    }
    default: return -RA_EINVAL;
    }
    return pairs > INT64_MAX ? -RA_ENOTSUP : (int64_t)pairs;
}

int64_t ra_share_backward_workspace(int32_t B, int32_t H, int64_t l_q) {
    if (B < 0 || H < 0 || l_q < 0) return -RA_EINVAL;
    const int64_t bytes = sat_mul(8, B, H, l_q);  // a multiple of 8 unless saturated
    return bytes == INT64_MAX ? -RA_ENOTSUP : bytes;
}

int ra_share_backward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv, int32_t d,
                      int32_t B, int32_t dtype, const void *Q_i, const void *K, const void *V,
                      const float *O, const void *dO, const float *m, const float *l,
                      float scale, float *dQ, float *dK, float *dV, void *workspace,
                      void *stream) {
    return backward_launch(rank, N, L, H, H_kv, d, B, dtype, ra::kNoCausal, Q_i, K, V, O, dO,
                           m, l, scale, dQ, dK, dV, workspace, stream);
}

int ra_causal_share_backward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                             int32_t d, int32_t B, int32_t dtype, int32_t layout,
                             const void *Q_i, const void *K, const void *V, const float *O,
                             const void *dO, const float *m, const float *l, float scale,
                             float *dQ, float *dK, float *dV, void *workspace, void *stream) {
    if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED &&
        layout != RA_LAYOUT_ZIGZAG)
        return RA_EINVAL;
    // Zigzag: each half-block must be whole 64-row tiles (as in the forward pass).
    if (layout == RA_LAYOUT_ZIGZAG && N >= 1 && L >= 0 && L % N == 0 && (L / N) % 128 != 0)
        return RA_EINVAL;
    return backward_launch(rank, N, L, H, H_kv, d, B, dtype, layout, Q_i, K, V, O, dO, m, l,
                           scale, dQ, dK, dV, workspace, stream);
}

int ra_share_backward_noalloc(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                              int32_t d, int32_t B, int32_t dtype, const void *Q_i,
                              const void *K, const void *V, const float *O, const void *dO,
                              const float *m, const float *l, float scale, float *dQ,
                              float *dK, float *dV, void *stream) {
    // Every argument check first, with a stand-in (aligned, never used) workspace address.
    void *const stand_in = (void *)(uintptr_t)256;
    int rc = backward_launch(rank, N, L, H, H_kv, d, B, dtype, ra::kNoCausal, Q_i, K, V, O,
                             dO, m, l, scale, dQ, dK, dV, stand_in, stream, true);
    if (rc != RA_OK || L == 0) return rc;
    if (ra_share_backward_workspace(B, H, L / N) > (int64_t)RA_NOALLOC_SCRATCH_BYTES)
        return RA_ESCRATCH;
    rc = check_device();
    if (rc != RA_OK) return rc;
    void *scratch = nullptr;
    const hipError_t e = ra::noalloc_scratch(&scratch);
    if (e != hipSuccess) return hip_fail(e);
    return backward_launch(rank, N, L, H, H_kv, d, B, dtype, ra::kNoCausal, Q_i, K, V, O, dO,
                           m, l, scale, dQ, dK, dV, scratch, stream);
}

int64_t ra_fp8_tiles(int64_t seg) {
    if (seg < 0) return -RA_EINVAL;
    return ceil_div(seg, 64);
}

int ra_quantize_fp8(int32_t kind, int32_t B, int32_t Hx, int32_t n_seg, int64_t seg, int32_t d,
                    const void *x, void *codes, float *descale, void *stream) {
    if ((kind != RA_FP8_ROWS && kind != RA_FP8_VT) || B < 1 || Hx < 1 || n_seg < 1 ||
        seg < 0 || (d != 64 && d != 128))
        return RA_EINVAL;
    if (seg == 0) return RA_OK;
    if (!ptr_ok(x) || !ptr_ok(codes) || !ptr_ok(descale)) return RA_EINVAL;
    const int64_t heads = (int64_t)B * Hx;
    const int64_t T = ceil_div(seg, 64);
    const int64_t rows = sat_mul(n_seg, seg);
    if (sat_mul(heads, n_seg, T) > INT32_MAX || sat_mul(heads, ceil_div(rows, 256)) > INT32_MAX ||
        sat_mul(heads, d) > INT32_MAX)
        return RA_ENOTSUP;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e =
        kind == RA_FP8_ROWS
            ? ra::launch_quant_rows(x, (uint8_t *)codes, descale, heads, n_seg, seg, d, st)
            : ra::launch_quant_vt(x, (uint8_t *)codes, descale, heads, n_seg, seg, d, st);
    return after_launch(e, st);
}

int ra_quantize_fp8_hadamard(int32_t B, int32_t Hx, int32_t n_seg, int64_t seg, int32_t d,
                             const void *x, const float *signs, int32_t query_side,
                             void *codes, float *descale, void *stream) {
    if (B < 1 || Hx < 1 || n_seg < 1 || seg < 0 || (d != 64 && d != 128)) return RA_EINVAL;
    if (seg == 0) return RA_OK;
    if (!ptr_ok(x) || !ptr_ok(signs) || !ptr_ok(codes) || !ptr_ok(descale)) return RA_EINVAL;
    const int64_t heads = (int64_t)B * Hx;
    const int64_t T = ceil_div(seg, 64);
    if (sat_mul(heads, n_seg, T) > INT32_MAX) return RA_ENOTSUP;
    int rc = check_device();
    if (rc != RA_OK) return rc;
    hipStream_t st = (hipStream_t)stream;
    return after_launch(ra::launch_quant_rows_hadamard(x, signs, query_side != 0,
                                                       (uint8_t *)codes, descale, heads, n_seg,
                                                       seg, d, st),
                        st);
}

int ra_share_forward_fp8(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                         int32_t d, int32_t B, const void *Q8, const float *q_descale,
                         const void *K8, const float *k_descale, const void *V8t,
                         const float *v_descale, float scale, float *O, float *m_out,
                         float *l_out, void *O_cast, void *stream) {
    return fp8_share_launch(rank, N, L, H, H_kv, d, B, ra::kNoCausal, Q8, q_descale, K8,
                            k_descale, V8t, v_descale, scale, O, m_out, l_out, O_cast, stream);
}

int ra_causal_share_forward_fp8(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                                int32_t d, int32_t B, int32_t layout, const void *Q8,
                                const float *q_descale, const void *K8, const float *k_descale,
                                const void *V8t, const float *v_descale, float scale, float *O,
                                float *m_out, float *l_out, void *O_cast, void *stream) {
    if (layout != RA_LAYOUT_CONTIGUOUS && layout != RA_LAYOUT_STRIPED &&
        layout != RA_LAYOUT_ZIGZAG)
        return RA_EINVAL;
    if (layout == RA_LAYOUT_ZIGZAG && N >= 1 && L >= 0 && L % N == 0 && (L / N) % 128 != 0)
        return RA_EINVAL;
    return fp8_share_launch(rank, N, L, H, H_kv, d, B, layout, Q8, q_descale, K8, k_descale,
                            V8t, v_descale, scale, O, m_out, l_out, O_cast, stream);
}

const char *ra_strerror(int status) {
    switch (status) {
    case RA_OK: return "success";
    case RA_EINVAL: return "invalid argument";
    case RA_ENOTSUP: return "unsupported device or size (needs gfx950)";
    case RA_EHIP: return "HIP runtime error (see ra_last_hip_error)";
    case RA_ESCRATCH:
        return "problem too large for the allocation-free entry point's scratch "
               "(RA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int ra_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
