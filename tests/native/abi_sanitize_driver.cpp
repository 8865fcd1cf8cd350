// Drives every entry point of include/ra.h, built with host AddressSanitizer and
// UndefinedBehaviorSanitizer against stand-ins for the HIP runtime and the kernel
// launchers (abi_stubs.cpp): host-only functions over ranges of arguments, each
// device entry point once with valid arguments (it must reach its launch) and with
// every class of invalid argument (it must return RA_EINVAL without launching).
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "ra.h"

extern int g_launches;
static int failures = 0;
#define CHECK(cond, what)                                                     \
    do {                                                                      \
        if (!(cond)) {                                                        \
            std::fprintf(stderr, "FAIL: %s (line %d)\n", what, __LINE__);     \
            failures++;                                                       \
        }                                                                     \
    } while (0)

// A valid call must launch; an invalid one must return RA_EINVAL and launch nothing.
#define EXPECT_OK(call, what)                                                 \
    do {                                                                      \
        const int before = g_launches;                                        \
        const int rc = (call);                                                \
        CHECK(rc == RA_OK && g_launches > before, what);                      \
    } while (0)
#define EXPECT_INVAL(call, what)                                              \
    do {                                                                      \
        const int before = g_launches;                                        \
        const int rc = (call);                                                \
        CHECK(rc == RA_EINVAL && g_launches == before, what);                 \
    } while (0)
// Sizes beyond what the kernels address: RA_ENOTSUP, nothing launched.
#define EXPECT_NOTSUP(call, what)                                             \
    do {                                                                      \
        const int before = g_launches;                                        \
        const int rc = (call);                                                \
        CHECK(rc == RA_ENOTSUP && g_launches == before, what);                \
    } while (0)

static void host_functions() {
    for (int N = 1; N <= 70; ++N)
        for (int rank = 0; rank < N; ++rank) {
            int seen[70] = {0};
            for (int t = 0; t < N; ++t) {
                const int j = ra_ring_block(rank, N, t);
                CHECK(j >= 0 && j < N && !seen[j], "schedule is a permutation");
                if (j >= 0 && j < N) seen[j] = 1;
            }
            int out[70];
            CHECK(ra_ring_schedule(rank, N, out) == RA_OK && out[0] == rank, "schedule");
        }
    CHECK(ra_ring_block(0, 0, 0) < 0 && ra_ring_block(4, 4, 0) < 0 && ra_ring_block(0, 4, 4) < 0 &&
              ra_ring_block(-1, 4, 0) < 0 && ra_ring_block(0, 4, -1) < 0,
          "ring block rejects");
    int out[4];
    CHECK(ra_ring_schedule(0, 4, nullptr) != RA_OK && ra_ring_schedule(4, 4, out) != RA_OK,
          "schedule rejects");
    CHECK(ra_kv_head(27, 28, 4) == 3 && ra_kv_head(0, 28, 4) == 0, "kv head");
    CHECK(ra_kv_head(28, 28, 4) < 0 && ra_kv_head(0, 28, 5) < 0 && ra_kv_head(0, 0, 1) < 0,
          "kv head rejects");
    for (int layout = 0; layout < 3; ++layout)
        for (int N : {1, 2, 3, 4, 8, 64})
            for (long L : {2L * N, 8L * N, 1024L * N})
                for (int rank = 0; rank < N; rank += (N > 8 ? 7 : 1)) {
                    const long long p = ra_causal_pairs(rank, N, L, layout);
                    const long long l = L / N;
                    CHECK(p >= l * (l + 1) / 2 && p <= l * L, "causal pairs in range");
                }
    CHECK(ra_causal_pairs(0, 4, 10, 0) < 0 && ra_causal_pairs(0, 4, 12, 2) < 0 &&
              ra_causal_pairs(0, 4, 16, 3) < 0 && ra_causal_pairs(5, 4, 16, 0) < 0,
          "causal pairs rejects");
    CHECK(ra_fp8_tiles(1) == 1 && ra_fp8_tiles(64) == 1 && ra_fp8_tiles(65) == 2, "fp8 tiles");
    CHECK(ra_fp8_tiles(0) == 0 && ra_fp8_tiles(-3) < 0, "fp8 tiles: empty, negative");
    CHECK(ra_share_backward_workspace(1, 32, 16384) > 0, "workspace");
    CHECK(ra_share_backward_workspace(0, 32, 16384) == 0 &&
              ra_share_backward_workspace(-1, 32, 16384) < 0,
          "workspace: empty, negative");
    for (int s = -2; s < 8; ++s) CHECK(ra_strerror(s) != nullptr, "strerror");
    (void)ra_last_hip_error();
}

static void device_entry_points(char *p) {
    // p: one 4 KiB aligned host block standing in for every device buffer (the ABI layer
    // never dereferences device pointers).
    const float nan = std::numeric_limits<float>::quiet_NaN();
    float *f = (float *)p;
    int32_t *trace = (int32_t *)p;
    void *st = nullptr;

    ra_shape s = {1, 4, 2, 128, 256, 512, 512L * 128, 2L * 512 * 128, RA_BF16};
    EXPECT_OK(ra_state_init(f, f, f, &s, st), "state init");
    EXPECT_OK(ra_step(p, p, p, f, f, f, 0.088f, &s, st), "step");
    EXPECT_OK(ra_finalize(f, f, &s, p, st), "finalize");
    ra_shape bad = s;
    bad.H = 3;
    EXPECT_INVAL(ra_step(p, p, p, f, f, f, 0.088f, &bad, st), "step H % H_kv");
    bad = s;
    bad.d = 96;
    EXPECT_INVAL(ra_step(p, p, p, f, f, f, 0.088f, &bad, st), "step head dim");
    bad = s;
    bad.dtype = 7;
    EXPECT_INVAL(ra_state_init(f, f, f, &bad, st), "state init dtype");
    EXPECT_INVAL(ra_step(p, p, p, f, f, f, nan, &s, st), "step scale NaN");
    EXPECT_INVAL(ra_step(p, p, p, f, f, f, -1.f, &s, st), "step scale < 0");
    EXPECT_INVAL(ra_step(p + 4, p, p, f, f, f, 0.088f, &s, st), "step misaligned Q");
    EXPECT_INVAL(ra_step(nullptr, p, p, f, f, f, 0.088f, &s, st), "step null Q");
    EXPECT_INVAL(ra_step(p, p, p, f, f, f, 0.088f, nullptr, st), "step null shape");

    for (int dtype : {RA_F32, RA_BF16})
        for (int d : {64, 128})
            EXPECT_OK(ra_share_forward(3, 8, 8 * 256, 4, 2, d, 2, dtype, p, p, p, 0.1f, f, f, f,
                                       p, trace, st),
                      "share forward");
    EXPECT_INVAL(ra_share_forward(8, 8, 2048, 4, 2, 128, 1, RA_BF16, p, p, p, 0.1f, f, f, f, p,
                                  trace, st), "share rank");
    EXPECT_INVAL(ra_share_forward(0, 8, 2047, 4, 2, 128, 1, RA_BF16, p, p, p, 0.1f, f, f, f, p,
                                  trace, st), "share L % N");
    EXPECT_INVAL(ra_share_forward(0, 8, 2048, 4, 3, 128, 1, RA_BF16, p, p, p, 0.1f, f, f, f, p,
                                  trace, st), "share H % H_kv");
    EXPECT_INVAL(ra_share_forward(0, 8, 2048, 4, 2, 128, 0, RA_BF16, p, p, p, 0.1f, f, f, f, p,
                                  trace, st), "share B");
    EXPECT_INVAL(ra_share_forward(0, 8, 2048, 4, 2, 128, 1, RA_BF16, p, p, p, INFINITY, f, f, f,
                                  p, trace, st), "share scale inf");
    EXPECT_INVAL(ra_share_forward(0, 8, 2048, 4, 2, 128, 1, RA_BF16, p, p + 2, p, 0.1f, f, f, f,
                                  p, trace, st), "share misaligned K");

    for (int layout = 0; layout < 3; ++layout) {
        EXPECT_OK(ra_causal_share_forward(3, 8, 8 * 256, 4, 2, 128, 1, RA_BF16, layout, p, p, p,
                                          0.1f, f, f, f, p, st), "causal forward");
        EXPECT_OK(ra_share_backward(3, 8, 8 * 256, 4, 2, 128, 1, RA_BF16, p, p, p, f, p, f, f,
                                    0.1f, f, f, f, p, st), "backward");
        EXPECT_OK(ra_causal_share_backward(3, 8, 8 * 256, 4, 2, 128, 1, RA_BF16, layout, p, p,
                                           p, f, p, f, f, 0.1f, f, f, f, p, st),
                  "causal backward");
        EXPECT_OK(ra_causal_share_forward_fp8(3, 8, 8 * 256, 4, 2, 128, 1, layout, p, f, p, f,
                                              p, f, 0.1f, f, f, f, p, st),
                  "causal fp8");
    }
    EXPECT_INVAL(ra_causal_share_forward(0, 8, 2048, 4, 2, 128, 1, RA_BF16, 3, p, p, p, 0.1f, f,
                                         f, f, p, st), "causal layout");
    EXPECT_INVAL(ra_causal_share_forward(0, 8, 8 * 130, 4, 2, 128, 1, RA_BF16, RA_LAYOUT_ZIGZAG,
                                         p, p, p, 0.1f, f, f, f, p, st), "zigzag odd chunks");
    EXPECT_INVAL(ra_share_backward(0, 8, 2048, 4, 2, 128, 1, RA_BF16, p, p, p, f, p, f, f, 0.1f,
                                   f, f, f, nullptr, st), "backward null workspace");
    EXPECT_OK(ra_share_backward_noalloc(3, 8, 8 * 256, 4, 2, 128, 1, RA_BF16, p, p, p, f, p, f,
                                        f, 0.1f, f, f, f, st), "backward noalloc");
    CHECK(ra_share_backward_noalloc(0, 1, 65537, 16, 16, 128, 1, RA_BF16, p, p, p, f, p, f, f,
                                    0.1f, f, f, f, st) == RA_ESCRATCH, "noalloc too large");
    EXPECT_INVAL(ra_share_backward_noalloc(0, 8, 2048, 4, 2, 128, 1, RA_BF16, p, p, p, nullptr,
                                           p, f, f, 0.1f, f, f, f, st), "noalloc null O");
    EXPECT_INVAL(ra_share_backward(0, 8, 2048, 4, 2, 128, 1, RA_BF16, p, p, p, nullptr, p, f, f,
                                   0.1f, f, f, f, p, st), "backward null O");

    for (int kind : {RA_FP8_ROWS, RA_FP8_VT})
        EXPECT_OK(ra_quantize_fp8(kind, 1, 4, 8, 256, 128, p, p, f, st), "quantize");
    EXPECT_INVAL(ra_quantize_fp8(2, 1, 4, 8, 256, 128, p, p, f, st), "quantize kind");
    EXPECT_OK(ra_quantize_fp8_hadamard(1, 4, 8, 256, 128, p, f, 1, p, f, st), "hadamard");
    EXPECT_INVAL(ra_quantize_fp8_hadamard(1, 4, 8, 256, 128, p, nullptr, 0, p, f, st),
                 "hadamard null signs");
    EXPECT_INVAL(ra_quantize_fp8_hadamard(1, 4, 8, 256, 96, p, f, 0, p, f, st), "hadamard d");
    EXPECT_INVAL(ra_quantize_fp8(RA_FP8_ROWS, 1, 4, 0, 256, 128, p, p, f, st), "quantize n_seg");
    EXPECT_INVAL(ra_quantize_fp8(RA_FP8_ROWS, 1, 4, 8, 256, 96, p, p, f, st), "quantize d");
    EXPECT_OK(ra_share_forward_fp8(3, 8, 8 * 256, 4, 2, 128, 1, p, f, p, f, p, f, 0.1f, f, f, f,
                                   p, st), "fp8 share");
    EXPECT_INVAL(ra_share_forward_fp8(3, 8, 8 * 256, 4, 2, 128, 1, p, nullptr, p, f, p, f, 0.1f,
                                      f, f, f, p, st), "fp8 null descale");
    EXPECT_INVAL(ra_share_forward_fp8(3, 8, 8 * 256, 4, 3, 128, 1, p, f, p, f, p, f, 0.1f, f, f,
                                      f, p, st), "fp8 H % H_kv");
}

// Sizes whose products overflow 64 bits (the checks must saturate, not wrap): every call
// returns RA_ENOTSUP without launching, and UBSan sees no signed overflow on the way.
static void huge_sizes(char *p) {
    float *f = (float *)p;
    void *st = nullptr;
    const int32_t big = std::numeric_limits<int32_t>::max();
    const int64_t top = std::numeric_limits<int64_t>::max();
    const int64_t top8 = top - top % 8;  // a multiple of N = 8

    for (int dtype : {RA_F32, RA_BF16}) {
        EXPECT_NOTSUP(ra_share_forward(0, 1, 1024, big, big, 128, big, dtype, p, p, p, 0.1f, f,
                                       f, f, p, nullptr, st), "share: huge B, H");
        EXPECT_NOTSUP(ra_causal_share_forward(0, 1, 1024, big, big, 64, big, dtype, 0, p, p, p,
                                              0.1f, f, f, f, p, st), "causal: huge B, H");
    }
    EXPECT_NOTSUP(ra_share_forward(0, 1, top, 1, 1, 128, 1, RA_F32, p, p, p, 0.1f, f, f, f, p,
                                   nullptr, st), "share f32: huge L");
    EXPECT_NOTSUP(ra_share_forward(7, 8, top8, 1, 1, 128, 1, RA_F32, p, p, p, 0.1f, f, f, f, p,
                                   nullptr, st), "share f32: huge L, N = 8");
    EXPECT_NOTSUP(ra_share_forward(0, 1, (int64_t)1 << 40, 64, 64, 128, 1 << 20, RA_F32, p, p,
                                   p, 0.1f, f, f, f, p, nullptr, st), "share f32: huge K/V");
    EXPECT_NOTSUP(ra_share_backward(0, 1, 1024, big, big, 128, big, RA_BF16, p, p, p, f, p, f,
                                    f, 0.1f, f, f, f, p, st), "backward: huge B, H");
    EXPECT_NOTSUP(ra_causal_share_backward(0, 1, 1024, big, big, 128, big, RA_BF16, 1, p, p,
                                           p, f, p, f, f, 0.1f, f, f, f, p, st),
                  "causal backward: huge B, H");
    EXPECT_NOTSUP(ra_share_backward_noalloc(0, 1, 1024, big, big, 128, big, RA_BF16, p, p, p,
                                            f, p, f, f, 0.1f, f, f, f, st),
                  "noalloc: huge B, H");
    EXPECT_NOTSUP(ra_share_forward_fp8(0, 1, 1024, big, big, 128, big, p, f, p, f, p, f, 0.1f,
                                       f, f, f, p, st), "fp8: huge B, H");
    EXPECT_NOTSUP(ra_share_forward_fp8(0, 1, top, 1, 1, 128, 1, p, f, p, f, p, f, 0.1f, f, f,
                                       f, p, st), "fp8: huge L");
    EXPECT_NOTSUP(ra_share_forward_fp8(7, 8, top8, 1, 1, 128, 1, p, f, p, f, p, f, 0.1f, f, f,
                                       f, p, st), "fp8: huge L, N = 8");
    EXPECT_NOTSUP(ra_causal_share_forward_fp8(0, big - 1, (int64_t)(big - 1) * 64, 1, 1, 128,
                                              1, 0, p, f, p, f, p, f, 0.1f, f, f, f, p, st),
                  "causal fp8: huge N");

    ra_shape s = {big, big, big, 128, top, top, 0, 0, RA_F32};
    EXPECT_NOTSUP(ra_state_init(f, f, f, &s, st), "state init: huge rows");
    EXPECT_NOTSUP(ra_finalize(f, f, &s, p, st), "finalize: huge rows");
    EXPECT_NOTSUP(ra_step(p, p, p, f, f, f, 0.1f, &s, st), "step: huge sizes");
    s = {1, 1, 1, 128, 64, top / 64, 0, 0, RA_F32};
    EXPECT_NOTSUP(ra_step(p, p, p, f, f, f, 0.1f, &s, st), "step: huge key rows");
    s = {1, 2, 2, 128, 64, 64, top - top % 8, 0, RA_F32};
    EXPECT_NOTSUP(ra_step(p, p, p, f, f, f, 0.1f, &s, st), "step: huge head stride");
    s = {big, 1, 1, 128, 64, 64, 64 * 128, top - top % 8, RA_F32};
    EXPECT_NOTSUP(ra_step(p, p, p, f, f, f, 0.1f, &s, st), "step: huge batch stride");

    for (int kind : {RA_FP8_ROWS, RA_FP8_VT}) {
        EXPECT_NOTSUP(ra_quantize_fp8(kind, big, big, big, 256, 128, p, p, f, st),
                      "quantize: huge B, Hx, n_seg");
        EXPECT_NOTSUP(ra_quantize_fp8(kind, 1, 1, big, top, 128, p, p, f, st),
                      "quantize: huge seg");
    }
    EXPECT_NOTSUP(ra_quantize_fp8_hadamard(big, big, big, 256, 128, p, f, 0, p, f, st),
                  "hadamard: huge B, Hx, n_seg");
    EXPECT_NOTSUP(ra_quantize_fp8_hadamard(1, 1, big, top, 64, p, f, 1, p, f, st),
                  "hadamard: huge seg");

    CHECK(ra_share_backward_workspace(big, big, top) == -RA_ENOTSUP, "workspace: overflow");
    CHECK(ra_fp8_tiles(top) == top / 64 + 1, "fp8 tiles: largest seg");
    for (int layout = 0; layout < 3; ++layout) {
        CHECK(ra_causal_pairs(0, 2, top - top % 4, layout) == -RA_ENOTSUP,
              "causal pairs: overflow");
        CHECK(ra_causal_pairs(big - 1, big, (int64_t)big * 2, layout) > 0,
              "causal pairs: many members");
    }
}

int main() {
    host_functions();
    char *p = (char *)std::aligned_alloc(256, 4096);
    device_entry_points(p);
    huge_sizes(p);
    std::free(p);
    if (failures) {
        std::fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    std::printf("abi sanitize driver: ok (%d stub launches)\n", g_launches);
    return 0;
}
