// fwd_f32.hip -- blockwise exact attention for fp32 inputs, fp32 arithmetic.
//
// Same computation as the bf16 path (slowleelab "Ring Attention" page, 4.2 and
// 4.3: ring-ordered K/V blocks merged with online softmax; final division by l),
// for inputs whose products must stay in fp32.  This path serves correctness at
// small sizes, so it uses the vector ALUs: a work-group holds 64 query rows, four
// lanes per row, each lane owning every fourth element of the head dimension;
// K/V tiles of 32 keys are staged in LDS and read as broadcasts.
#include "ra_internal.h"

namespace ra {
namespace {

constexpr int BR = kF32QueryTile;  // query rows per work-group
constexpr int BC = 32;             // keys per tile
constexpr int NT = 256;            // 4 lanes per query row
constexpr float kLog2e = 1.4426950408889634f;

// Global sequence position of local token x of ring member `member` under a causal
// share's token layout: contiguous r*l + x, striped x*N + r, zigzag (h = l/2) r*h + x
// for x < h and (2N-1-r)*h + (x-h) after (slowleelab "Ring Attention" page, 4.5 and
// 4.8).  A key is admissible for a query when its position is not later.
__device__ __forceinline__ int64_t token_position(int32_t layout, int64_t member, int64_t N,
                                                  int64_t l, int64_t x) {
    if (layout == 0) return member * l + x;
    if (layout == 1) return x * N + member;
    const int64_t h = l / 2;
    return x < h ? member * h + x : (2 * N - 1 - member) * h + (x - h);
}

template <int D, int MODE, bool CAUSAL>
__global__ __launch_bounds__(NT) void fwd_f32_kernel(FwdArgs a) {
    constexpr int DL = D / 4;  // head-dim elements per lane
    __shared__ float Ks[BC * D];
    __shared__ float Vs[BC * D];

    const int tid = threadIdx.x;
    const int part = tid & 3;
    const int wg = blockIdx.x;
    const int qt = wg % a.n_qtiles;
    const int bh = wg / a.n_qtiles;
    const int h = bh % a.H, b = bh / a.H;
    const int g = h / a.group;
    const int64_t q = (int64_t)qt * BR + (tid >> 2);
    const bool qvalid = q < a.l_q;
    const int64_t qrow = (int64_t)bh * a.l_q + q;
    const float *Kh = (const float *)a.K + b * a.kv_batch_stride + g * a.kv_head_stride;
    const float *Vh = (const float *)a.V + b * a.kv_batch_stride + g * a.kv_head_stride;

    // lane owns head-dim elements 4*jj + part
    float qv[DL], o[DL];
    for (int jj = 0; jj < DL; ++jj) {
        qv[jj] = qvalid ? ((const float *)a.Q)[qrow * D + 4 * jj + part] : 0.f;
        o[jj] = 0.f;
    }
    float lsum = 0.f, R = -INFINITY, m_nat = -INFINITY;
    if constexpr (MODE == MODE_STEP) {
        if (qvalid) {
            m_nat = a.m[qrow];
            R = m_nat * kLog2e;
            lsum = a.l[qrow];
            for (int jj = 0; jj < DL; ++jj) o[jj] = a.O[qrow * D + 4 * jj + part];
        }
    }
    const float c = a.scale_log2;
    const int64_t qpos =
        CAUSAL ? token_position(a.layout, a.rank, a.n_blocks, a.blk_rows, q) : 0;
    const int64_t tiles_per_blk = (a.blk_rows + BC - 1) / BC;
    const int64_t n_tiles = tiles_per_blk * a.n_blocks;

    for (int64_t it = 0; it < n_tiles; ++it) {
        const int64_t t = it / tiles_per_blk;
        const int64_t tin = it - t * tiles_per_blk;
        int64_t j = (int64_t)a.rank - t;
        if (j < 0) j += a.n_blocks;
        if constexpr (MODE == MODE_SHARE) {
            if (a.trace && tin == 0 && wg == 0 && tid == 0) a.trace[t] = (int32_t)j;
        }
        const int64_t row0 = j * a.blk_rows + tin * BC;
        const int64_t nvalid = a.blk_rows - tin * BC;
        __syncthreads();  // previous tile fully consumed
        for (int e = tid; e < BC * D; e += NT) {
            const int r = e / D;
            const bool ok = r < nvalid;
            Ks[e] = ok ? Kh[(row0 + r) * D + (e % D)] : 0.f;
            Vs[e] = ok ? Vh[(row0 + r) * D + (e % D)] : 0.f;
        }
        __syncthreads();

        float s[BC];
        float mx = -INFINITY;
#pragma unroll
        for (int k = 0; k < BC; ++k) {
            float part_dot = 0.f;
#pragma unroll
            for (int jj = 0; jj < DL; ++jj)
                part_dot = __builtin_fmaf(qv[jj], Ks[k * D + 4 * jj + part], part_dot);
            part_dot += __shfl_xor(part_dot, 1);
            part_dot += __shfl_xor(part_dot, 2);
            bool keep = k < nvalid;
            if constexpr (CAUSAL)
                keep = keep && token_position(a.layout, j, a.n_blocks, a.blk_rows,
                                              tin * BC + k) <= qpos;
            s[k] = keep ? part_dot : -INFINITY;
            mx = fmaxf(mx, s[k]);
        }
        m_nat = fmaxf(m_nat, mx * a.scale);
        const float Rn = fmaxf(R, mx * c);
        const float alpha = __builtin_amdgcn_exp2f(R - Rn);
        R = Rn;
        lsum *= alpha;
#pragma unroll
        for (int jj = 0; jj < DL; ++jj) o[jj] *= alpha;
#pragma unroll
        for (int k = 0; k < BC; ++k) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k], c, -R));
            lsum += p;
#pragma unroll
            for (int jj = 0; jj < DL; ++jj)
                o[jj] = __builtin_fmaf(p, Vs[k * D + 4 * jj + part], o[jj]);
        }
    }

    if (!qvalid || n_tiles == 0) return;
    if constexpr (MODE == MODE_SHARE) {
        for (int jj = 0; jj < DL; ++jj) {
            const float v = o[jj] / lsum;
            a.O[qrow * D + 4 * jj + part] = v;
            if (a.O_cast) ((float *)a.O_cast)[qrow * D + 4 * jj + part] = v;
        }
        if (part == 0) {
            if (a.m) a.m[qrow] = m_nat;
            if (a.l) a.l[qrow] = lsum * __builtin_amdgcn_exp2f(R - m_nat * kLog2e);
        }
    } else {
        const float f = __builtin_amdgcn_exp2f(R - m_nat * kLog2e);
        for (int jj = 0; jj < DL; ++jj) a.O[qrow * D + 4 * jj + part] = o[jj] * f;
        if (part == 0) {
            a.m[qrow] = m_nat;
            a.l[qrow] = lsum * f;
        }
    }
}

template <int D, int MODE, bool CAUSAL = false>
hipError_t launch(const FwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((fwd_f32_kernel<D, MODE, CAUSAL>), dim3(a.n_wg), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, int B, int d, int mode, hipStream_t st) {
    (void)B;
    if (a.layout != kNoCausal) {  // causal shares only
        if (mode != MODE_SHARE) return hipErrorInvalidValue;
        if (d == 128) return launch<128, MODE_SHARE, true>(a, st);
        if (d == 64) return launch<64, MODE_SHARE, true>(a, st);
        return hipErrorInvalidValue;
    }
    if (d == 128) return mode == MODE_SHARE ? launch<128, MODE_SHARE>(a, st)
                                            : launch<128, MODE_STEP>(a, st);
    if (d == 64) return mode == MODE_SHARE ? launch<64, MODE_SHARE>(a, st)
                                           : launch<64, MODE_STEP>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace ra
