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
    static_assert(256 % CPR == 0, "a thread's chunks share their position in the row");
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

    // Loads without branches (chunks of rows past the block's end read the last row's chunk,
    // then count as zeros), so a thread's loads are in flight together.
    bf16x8 v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = threadIdx.x + 256 * i;
        const int qq = q / CPR < nrows ? q : (nrows - 1) * CPR + q % CPR;
        v[i] = *(const bf16x8 *)(x + base + (int64_t)qq * 8);
    }
    float f[PER][8];
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            f[i][e] = (threadIdx.x + 256 * i) / CPR < nrows ? (float)v[i][e] : 0.f;
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < PER; ++i)
        if ((threadIdx.x + 256 * i) / CPR < nrows)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(f[i][e]));
    const float ds = descale_of(block_max(amax, red));
    const float inv = 1.0f / ds;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int q = threadIdx.x + 256 * i;
        if (q / CPR < nrows) {
            float g[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) g[e] = f[i][e] * inv;
            *(u32x2 *)(codes + base + (int64_t)q * 8) =
                u32x2{pack4(g[0], g[1], g[2], g[3]), pack4(g[4], g[5], g[6], g[7])};
        }
    }
    if (threadIdx.x == 0) descale[hs * T + u] = ds;
}

// Butterfly stage across the lanes of a DPP quad: lanes L and L ^ K hold entries i and
// i + K * D / 4 of one row; the lower lane becomes a + b, the upper a - b, each computed as
// partner + (+-own), one fp32 rounding either way as in a + b and a - b.  The partner's
// value comes by a DPP quad permute ([1, 0, 3, 2] for K = 1, [2, 3, 0, 1] for K = 2).
template <int K, int N>
__device__ __forceinline__ void quad_stage(float (&f)[N], int qd) {
    static_assert(K == 1 || K == 2, "lanes of one quad");
    const unsigned flip = (qd & K) ? 0x80000000u : 0u;
#pragma unroll
    for (int e = 0; e < N; ++e) {
        const int mine = __builtin_bit_cast(int, f[e]);
        const int other = __builtin_amdgcn_mov_dpp(mine, K == 1 ? 0xB1 : 0x4E, 0xF, 0xF, true);
        f[e] = __builtin_bit_cast(float, other) + __builtin_bit_cast(float, (unsigned)mine ^ flip);
    }
}

// Rows mode with incoherent processing: each row is first multiplied by diag(signs) H_D,
// H_D the Sylvester Hadamard matrix (entries +-1), in fp32 by the fast transform: for
// h = 1, 2, 4, ..., D/2 every pair of entries (i, i + h) with i & h == 0 becomes
// (a + b, a - b).  One 64-row block per work-group; a row's D values sit in the four lanes
// of a DPP quad, D/4 consecutive values per lane, so the stages h < D/4 run inside the lane
// and the last two pair lane L with L ^ 1, then L ^ 2.  Every entry goes through the same
// fp32 operations in the same order whichever lane computes it.  The block is then
// quantized as in rows mode, and its descale multiplied by `post` (1, or 1/D for the query
// side: a power of two, exact).
template <int D>
__global__ __launch_bounds__(256) void quant_rows_rot_kernel(const bf16 *x, const float *signs,
                                                             float post, uint8_t *codes,
                                                             float *descale, int32_t n_seg,
                                                             int64_t seg, int32_t T) {
    constexpr int VPL = D / 4;  // values per lane: 32 (d = 128) or 16 (d = 64)
    __shared__ float red[4];
    const int64_t wg = blockIdx.x;
    const int u = (int)(wg % T);
    const int64_t hs = wg / T;  // head * n_seg + segment
    const int s = (int)(hs % n_seg);
    const int64_t hd = hs / n_seg;
    const int64_t row0 = (int64_t)s * seg + (int64_t)u * QT;
    const int64_t left = seg - (int64_t)u * QT;
    const int nrows = left < QT ? (int)left : QT;
    const int r = threadIdx.x >> 2, qd = threadIdx.x & 3;  // row of the block, quarter of it
    const int64_t off = (hd * n_seg * seg + row0 + r) * D + qd * VPL;  // this lane's values
    float f[VPL];
    if (r < nrows) {
#pragma unroll
        for (int k = 0; k < VPL / 8; ++k) {
            const bf16x8 v = *(const bf16x8 *)(x + off + 8 * k);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[8 * k + e] = (float)v[e] * signs[qd * VPL + 8 * k + e];
        }
    } else {
#pragma unroll
        for (int e = 0; e < VPL; ++e) f[e] = 0.f;
    }
#pragma unroll
    for (int h = 1; h < VPL; h *= 2)
#pragma unroll
        for (int e = 0; e < VPL; ++e)
            if (!(e & h)) {
                const float a = f[e], b = f[e + h];
                f[e] = a + b;
                f[e + h] = a - b;
            }
    quad_stage<1>(f, qd);
    quad_stage<2>(f, qd);
    float amax = 0.f;  // rows past the block's end hold zeros
#pragma unroll
    for (int e = 0; e < VPL; ++e) amax = fmaxf(amax, fabsf(f[e]));
    const float ds = descale_of(block_max(amax, red));
    const float inv = 1.0f / ds;
    if (r < nrows) {
#pragma unroll
        for (int k = 0; k < VPL / 16; ++k) {
            const float *g = f + 16 * k;
            *(u32x4 *)(codes + off + 16 * k) =
                u32x4{pack4(g[0] * inv, g[1] * inv, g[2] * inv, g[3] * inv),
                      pack4(g[4] * inv, g[5] * inv, g[6] * inv, g[7] * inv),
                      pack4(g[8] * inv, g[9] * inv, g[10] * inv, g[11] * inv),
                      pack4(g[12] * inv, g[13] * inv, g[14] * inv, g[15] * inv)};
        }
    }
    if (threadIdx.x == 0) descale[hs * T + u] = ds * post;
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
    // A fixed trip count without branches, so all of a thread's loads can be in flight at
    // once: rows past the head's end read its last row again, which leaves a maximum as is.
#pragma unroll
    for (int k = 0; k < 256 / RPP; ++k) {
        const int64_t want = r0 + rp + k * RPP;
        const int64_t row = want < rows ? want : rows - 1;
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

// One stored tile per work-group, transposed through LDS.  Load phase: each thread reads
// RPT consecutive rows of 8 channels (16-byte loads; each row of the tile is read whole by
// CPR neighbouring lanes), quantizes every value as in rows mode with its channel's scale
// (rows past the segment's end are zero) and writes each channel's RPT codes as one word
// of that channel's row in LDS (channel-major, row stride VS; VS / 4 odd spreads the rows
// over the banks).  Store phase: thread (channel c, row group rg) copies the RG codes
// RG*rg ... of channel row c to the stored tile.
template <int D>
__global__ __launch_bounds__(256) void vt_quant_kernel(const bf16 *x, uint8_t *codes,
                                                       const float *descale, int32_t n_seg,
                                                       int64_t seg, int32_t T) {
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int RPT = QT * CPR / 256;    // rows per thread in the load phase: 4 or 2
    constexpr int NG = 256 / D;            // row groups of the store phase
    constexpr int RG = QT / NG;            // codes per thread: 32 (d = 128) or 16 (d = 64)
    constexpr int VS = QT + 4;             // LDS bytes per channel row
    static_assert(RPT == 4 || RPT == 2, "load phase packs 2 or 4 rows per channel");
    __shared__ __attribute__((aligned(16))) uint8_t tile[D * VS];
    const int64_t wg = blockIdx.x;
    const int u = (int)(wg % T);
    const int64_t hs = wg / T;
    const int s = (int)(hs % n_seg);
    const int64_t hd = hs / n_seg;
    const int64_t left = seg - (int64_t)u * QT;
    const int nrows = left < QT ? (int)left : QT;
    const bf16 *xt = x + ((hd * n_seg + s) * seg + (int64_t)u * QT) * D;
    const int c8 = threadIdx.x % CPR, r0 = RPT * (threadIdx.x / CPR);
    float inv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) inv[e] = 1.0f / descale[hd * D + 8 * c8 + e];
    // Loads without branches (rows past the segment's end read its last row, then count as
    // zeros), so a thread's loads are in flight together.
    bf16x8 v[RPT];
#pragma unroll
    for (int k = 0; k < RPT; ++k) {
        const int r = r0 + k < nrows ? r0 + k : nrows - 1;
        v[k] = *(const bf16x8 *)(xt + (int64_t)r * D + 8 * c8);
    }
    float f[RPT][8];
#pragma unroll
    for (int k = 0; k < RPT; ++k)
#pragma unroll
        for (int e = 0; e < 8; ++e) f[k][e] = r0 + k < nrows ? (float)v[k][e] * inv[e] : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint8_t *tp = tile + (8 * c8 + e) * VS + r0;
        if constexpr (RPT == 4)
            *(unsigned *)tp = pack4(f[0][e], f[1][e], f[2][e], f[3][e]);
        else
            *(uint16_t *)tp =
                (uint16_t)__builtin_amdgcn_cvt_pk_fp8_f32(f[0][e], f[1][e], 0, false);
    }
    __syncthreads();
    const int c = threadIdx.x % D, rg = threadIdx.x / D;
    const uint8_t *src = tile + c * VS + RG * rg;
    uint8_t *op = codes + (hs * T + u) * (int64_t)(D * QT) + c * QT + RG * rg;
#pragma unroll
    for (int k = 0; k < RG / 16; ++k) {
        const unsigned *sp = (const unsigned *)(src + 16 * k);
        *(u32x4 *)(op + 16 * k) = u32x4{sp[0], sp[1], sp[2], sp[3]};
    }
}

template <int D, bool ROT>
hipError_t rows_impl(const void *x, const float *signs, float post, uint8_t *codes,
                     float *descale, int64_t heads, int32_t n_seg, int64_t seg,
                     hipStream_t st) {
    const int32_t T = (int32_t)((seg + QT - 1) / QT);
    const int64_t n = heads * n_seg * T;
    if constexpr (ROT)
        hipLaunchKernelGGL((quant_rows_rot_kernel<D>), dim3((unsigned)n), dim3(256), 0, st,
                           (const bf16 *)x, signs, post, codes, descale, n_seg, seg, T);
    else
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
    if (d == 128)
        return rows_impl<128, false>(x, nullptr, 1.f, codes, descale, heads, n_seg, seg, st);
    if (d == 64)
        return rows_impl<64, false>(x, nullptr, 1.f, codes, descale, heads, n_seg, seg, st);
    return hipErrorInvalidValue;
}

hipError_t launch_quant_rows_hadamard(const void *x, const float *signs, bool query_side,
                                      uint8_t *codes, float *descale, int64_t heads,
                                      int32_t n_seg, int64_t seg, int d, hipStream_t st) {
    const float post = query_side ? 1.0f / (float)d : 1.0f;
    if (d == 128)
        return rows_impl<128, true>(x, signs, post, codes, descale, heads, n_seg, seg, st);
    if (d == 64)
        return rows_impl<64, true>(x, signs, post, codes, descale, heads, n_seg, seg, st);
    return hipErrorInvalidValue;
}

hipError_t launch_quant_vt(const void *x, uint8_t *codes, float *descale, int64_t heads,
                           int32_t n_seg, int64_t seg, int d, hipStream_t st) {
    if (d == 128) return vt_impl<128>(x, codes, descale, heads, n_seg, seg, st);
    if (d == 64) return vt_impl<64>(x, codes, descale, heads, n_seg, seg, st);
    return hipErrorInvalidValue;
}

}  // namespace ra
