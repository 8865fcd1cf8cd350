// fp8_quant.hip -- block quantization of bf16 tensors to OCP FP8 E4M3 for the FP8 share.
//
// FlashAttention-3 feeds its forward products from FP8 inputs with block quantization
// (aliyun FlashAttention explainer, section 2, FlashAttention-3).  Here a block's scale
// is descale = max(amax / 448, 2^-126) (fp32, 448 = the largest E4M3 value), a value x
// is stored as the E4M3 code of fp32(x * fp32(1 / descale)), rounded to nearest even by
// v_cvt_pk_fp8_f32, and stands for descale * value(code).
//  * rows mode (Q and K): one scale per 64-row block of each segment of `seg` rows (a
//    ring member's block); codes keep the input layout [heads, n_seg * seg, d].
//  * vt mode (V): one scale per channel over all rows of a head, so the share kernel
//    applies it once to its output; codes are stored per 64-row tile transposed,
//    [heads, n_seg, T, d, 64], columns past a segment's end zero.  The per-channel
//    maxima go through the descale array itself (as the bit patterns of non-negative
//    floats, which order like unsigned integers) before it is finalised in place.
// Memory-bound, one pass over the input (two for vt mode).
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int QT = 64;  // rows per scale block / per stored V tile
constexpr float kE4m3Max = 448.0f;
constexpr float kFltMin = 1.17549435e-38f;  // 2^-126

__device__ __forceinline__ float descale_of(float amax) {
    return fmaxf(amax / kE4m3Max, kFltMin);
}

// Four values -> four E4M3 bytes (little-endian order) of one dword.
__device__ __forceinline__ unsigned pack4(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (unsigned)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

__device__ __forceinline__ float block_max(float v, float *red) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    v = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    return v;
}

// One 64-row block per work-group (256 threads, 16-byte chunks of 8 values).
template <int D>
__global__ __launch_bounds__(256) void quant_rows_kernel(const bf16 *x, uint8_t *codes,
                                                         float *descale, int32_t n_seg,
                                                         int64_t seg, int32_t T) {
    constexpr int CPR = D / 8;               // chunks per row
    constexpr int PER = QT * CPR / 256;      // chunks per thread
    __shared__ float red[4];
    const int64_t wg = blockIdx.x;
    const int u = (int)(wg % T);
    const int64_t hs = wg / T;  // head * n_seg + segment
    const int s = (int)(hs % n_seg);
    const int64_t hd = hs / n_seg;
    const int64_t row0 = (int64_t)s * seg + (int64_t)u * QT;
    const int64_t left = seg - (int64_t)u * QT;
    const int nrows = left < QT ? (int)left : QT;
    const int64_t base = (hd * n_seg * seg + row0) * D;  // element offset of the block

    bf16x8 v[PER];
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = threadIdx.x + 256 * i;
        const int r = q / CPR;
        if (r < nrows) {
            v[i] = *(const bf16x8 *)(x + base + (int64_t)q * 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)v[i][e]));
        }
    }
    const float ds = descale_of(block_max(amax, red));
    const float inv = 1.0f / ds;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = threadIdx.x + 256 * i;
        if (q / CPR < nrows) {
            float f[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = (float)v[i][e] * inv;
            *(u32x2 *)(codes + base + (int64_t)q * 8) =
                u32x2{pack4(f[0], f[1], f[2], f[3]), pack4(f[4], f[5], f[6], f[7])};
        }
    }
    if (threadIdx.x == 0) descale[hs * T + u] = ds;
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0.f;
}

// Per-channel maxima over 256-row chunks of each head, merged with atomic max on the
// float bits (all non-negative).
template <int D>
__global__ __launch_bounds__(256) void vt_amax_kernel(const bf16 *x, float *amax, int64_t rows,
                                                      int32_t n_chunks) {
    constexpr int CPR = D / 8;
    constexpr int RPP = 256 / CPR;  // rows per pass
    __shared__ float red[RPP][D + 1];
    const int64_t hd = blockIdx.x / n_chunks;
    const int64_t r0 = (int64_t)(blockIdx.x % n_chunks) * 256;
    const int c8 = threadIdx.x % CPR, rp = threadIdx.x / CPR;
    float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int r = rp; r < 256; r += RPP) {
        const int64_t row = r0 + r;
        if (row >= rows) break;
        const bf16x8 v = *(const bf16x8 *)(x + (hd * rows + row) * D + 8 * c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = fmaxf(m[e], fabsf((float)v[e]));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rp][8 * c8 + e] = m[e];
    __syncthreads();
    if (threadIdx.x < D) {
        float t = 0.f;
#pragma unroll 8
        for (int r = 0; r < RPP; ++r) t = fmaxf(t, red[r][threadIdx.x]);
        atomicMax((unsigned *)(amax + hd * D + threadIdx.x), __float_as_uint(t));
    }
}

__global__ void vt_finalize_kernel(float *descale, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) descale[i] = descale_of(descale[i]);
}

// One stored tile per work-group: thread (channel c, row group rg) quantizes rows
// 64u + RG*rg ... of channel c and writes them as RG consecutive bytes of row c of the
// transposed tile.
template <int D>
__global__ __launch_bounds__(256) void vt_quant_kernel(const bf16 *x, uint8_t *codes,
                                                       const float *descale, int32_t n_seg,
                                                       int64_t seg, int32_t T) {
    constexpr int NG = 256 / D;  // row groups
    constexpr int RG = QT / NG;  // rows per thread: 32 (d = 128) or 16 (d = 64)
    const int64_t wg = blockIdx.x;
    const int u = (int)(wg % T);
    const int64_t hs = wg / T;
    const int s = (int)(hs % n_seg);
    const int64_t hd = hs / n_seg;
    const int c = threadIdx.x % D, rg = threadIdx.x / D;
    const int64_t left = seg - (int64_t)u * QT;
    const int nrows = left < QT ? (int)left : QT;
    const float inv = 1.0f / descale[hd * D + c];
    const bf16 *xp = x + ((hd * n_seg + s) * seg + (int64_t)u * QT) * D + c;
    unsigned w[RG / 4];
#pragma unroll
    for (int k = 0; k < RG / 4; ++k) {
        float f[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = RG * rg + 4 * k + e;
            f[e] = r < nrows ? (float)xp[(int64_t)r * D] * inv : 0.f;
        }
        w[k] = pack4(f[0], f[1], f[2], f[3]);
    }
    uint8_t *op = codes + (hs * T + u) * (int64_t)(D * QT) + c * QT + RG * rg;
#pragma unroll
    for (int k = 0; k < RG / 16; ++k)
        *(u32x4 *)(op + 16 * k) = u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]};
}

template <int D>
hipError_t rows_impl(const void *x, uint8_t *codes, float *descale, int64_t heads,
                     int32_t n_seg, int64_t seg, hipStream_t st) {
    const int32_t T = (int32_t)((seg + QT - 1) / QT);
    const int64_t n = heads * n_seg * T;
    hipLaunchKernelGGL((quant_rows_kernel<D>), dim3((unsigned)n), dim3(256), 0, st,
                       (const bf16 *)x, codes, descale, n_seg, seg, T);
    return hipGetLastError();
}

template <int D>
hipError_t vt_impl(const void *x, uint8_t *codes, float *descale, int64_t heads,
                   int32_t n_seg, int64_t seg, hipStream_t st) {
    const int32_t T = (int32_t)((seg + QT - 1) / QT);
    const int64_t rows = (int64_t)n_seg * seg;
    const int64_t nd = heads * D;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0, st,
                       descale, nd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int32_t n_chunks = (int32_t)((rows + 255) / 256);
    hipLaunchKernelGGL((vt_amax_kernel<D>), dim3((unsigned)(heads * n_chunks)), dim3(256), 0,
                       st, (const bf16 *)x, descale, rows, n_chunks);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(vt_finalize_kernel, dim3((unsigned)((nd + 255) / 256)), dim3(256), 0,
                       st, descale, nd);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL((vt_quant_kernel<D>), dim3((unsigned)(heads * n_seg * T)), dim3(256), 0,
                       st, (const bf16 *)x, codes, descale, n_seg, seg, T);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quant_rows(const void *x, uint8_t *codes, float *descale, int64_t heads,
                             int32_t n_seg, int64_t seg, int d, hipStream_t st) {
    if (d == 128) return rows_impl<128>(x, codes, descale, heads, n_seg, seg, st);
    if (d == 64) return rows_impl<64>(x, codes, descale, heads, n_seg, seg, st);
    return hipErrorInvalidValue;
}

hipError_t launch_quant_vt(const void *x, uint8_t *codes, float *descale, int64_t heads,
                           int32_t n_seg, int64_t seg, int d, hipStream_t st) {
    if (d == 128) return vt_impl<128>(x, codes, descale, heads, n_seg, seg, st);
    if (d == 64) return vt_impl<64>(x, codes, descale, heads, n_seg, seg, st);
    return hipErrorInvalidValue;
}

}  // namespace ra
