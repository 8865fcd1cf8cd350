// Host-only stand-ins for the HIP runtime calls and the kernel launchers that the C ABI
// layer (ra_api.cpp) uses, so its host logic (validation, schedules, causal pair counts,
// grid sizing) can be built with host sanitizers and driven without a GPU.  The stand-in
// device reports gfx950; every launch records its work description, checks that the grid
// matches it, and returns success without running anything.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "ra_internal.h"

int g_launches = 0;

static void require(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "stub launch: inconsistent %s\n", what);
        std::abort();
    }
}

extern "C" {
hipError_t hipGetDevice(int *d) {
    *d = 0;
    return hipSuccess;
}
hipError_t hipGetDevicePropertiesR0600(hipDeviceProp_tR0600 *p, int) {
    std::memset(p, 0, sizeof *p);
    std::strcpy(p->gcnArchName, "gfx950:sramecc+:xnack-");
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

namespace ra {
int bf16_query_tile() { return 256; }
int bwd_query_tile() { return 256; }
int bwd_key_tile() { return 128; }
int fp8_query_tile() { return 256; }

hipError_t launch_fwd_bf16(const FwdArgs &a, int B, int d, int mode, hipStream_t) {
    require(a.n_wg == a.n_qtiles * B * a.H && a.n_wg > 0, "bf16 grid");
    require(d == 64 || d == 128, "head dim");
    require(mode == MODE_SHARE || mode == MODE_STEP, "mode");
    require(a.H % a.H_kv == 0 && a.group == a.H / a.H_kv, "head groups");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_fwd_f32(const FwdArgs &a, int B, int d, int mode, hipStream_t) {
    require(a.n_wg == a.n_qtiles * B * a.H && a.n_wg > 0, "f32 grid");
    require(d == 64 || d == 128, "head dim");
    require(mode == MODE_SHARE || mode == MODE_STEP, "mode");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_bwd_bf16(const BwdArgs &a, const float *, const void *, const float *,
                           const float *, int64_t rows, int d, hipStream_t) {
    require(rows > 0 && a.n_wg > 0 && a.n_kv_wg > 0, "backward grid");
    require(d == 64 || d == 128, "head dim");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_fwd_fp8(const Fp8Args &a, int d, hipStream_t) {
    require(a.n_wg > 0 && a.n_qtiles > 0, "fp8 grid");
    require(d == 64 || d == 128, "head dim");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_quant_rows(const void *, uint8_t *, float *, int64_t heads, int32_t n_seg,
                             int64_t seg, int d, hipStream_t) {
    require(heads > 0 && n_seg > 0 && seg > 0 && (d == 64 || d == 128), "quant rows");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_quant_vt(const void *, uint8_t *, float *, int64_t heads, int32_t n_seg,
                           int64_t seg, int d, hipStream_t) {
    require(heads > 0 && n_seg > 0 && seg > 0 && (d == 64 || d == 128), "quant vt");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_state_init(float *, float *, float *, int64_t rows, int d, hipStream_t) {
    require(rows >= 0 && d > 0, "state init");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_finalize(float *, const float *, int64_t rows, int d, int, void *,
                           hipStream_t) {
    require(rows >= 0 && d > 0, "finalize");
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_quant_rows_hadamard(const void *, const float *, bool, uint8_t *, float *,
                                      int64_t heads, int32_t n_seg, int64_t seg, int d,
                                      hipStream_t) {
    require(heads > 0 && n_seg > 0 && seg > 0 && (d == 64 || d == 128), "quant hadamard");
    ++g_launches;
    return hipSuccess;
}
// Stand-in for the static scratch lookup: a host buffer that the stub launches never read.
alignas(256) static unsigned char g_scratch_stub[256];
hipError_t noalloc_scratch(void **ptr) {
    *ptr = g_scratch_stub;
    return hipSuccess;
}
}  // namespace ra
