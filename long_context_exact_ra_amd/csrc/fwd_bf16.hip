// fwd_bf16.hip -- blockwise exact attention for one ring member's share, bf16
// inputs, gfx950 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 statistics.
//
// What one work-group computes (slowleelab "Ring Attention" page, 4.2 and 4.3;
// aliyun FlashAttention explainer, section 2, tiling with Br x d query tiles and
// Bc x d key/value tiles and running max / sum statistics):
//   for every K/V block in ring order, for every Bc-key tile of that block:
//     S     = Q_tile K_tile^T            (raw dot products, fp32)
//     m_new = max(m, row max S)          (per query row)
//     O    <- exp(m - m_new) O + exp(S*scale - m_new) V_tile
//     l    <- exp(m - m_new) l + row sum exp(S*scale - m_new)
//   and, for a whole share, O / l once at the end.
//
// MI355X mapping
//  * One work-group = 8 waves (2 per SIMD) = 256 query rows of one (batch, head);
//    each wave owns 32 query rows for the whole launch, with its Q fragment
//    resident in VGPRs.
//  * Scores are computed transposed, S^T = K Q^T, so the 32x32 MFMA output puts one
//    query row in each lane (lanes l and l+32 hold 16 keys each of that row).  Row
//    max and row sum are therefore in-lane, plus one v_permlane32_swap.
//  * The exponentials P^T, packed to bf16, are directly the B operand of
//    O^T = V^T P^T: no cross-lane shuffle of P.  The key order inside each
//    16-deep contraction is permuted to match the score layout, and V^T is read
//    from LDS with ds_read_b64_tr_b16 transpose loads using the same permutation.
//  * K/V tiles (64 keys) are double-buffered in LDS: the next tile's global loads
//    are issued before the current tile's math and written to the other buffer
//    after it; one barrier per tile.  Row pitches are padded against bank
//    conflicts (K: +16 B for the 16-byte row reads, V: +32 B for the 4-row
//    transpose reads).
//  * The exponent reference is updated lazily: the O / l rescale only runs when
//    some row's maximum grew by more than 2^kTau (a wave-uniform branch), so
//    exp2(s*c - R) stays <= 2^kTau.  The true running maximum is tracked
//    separately, and the state is converted to it at the end, so outputs obey
//    m = exact running maximum.
//  * Work-group ids are remapped so each XCD (8 per chip, one L2 each) works on a
//    contiguous range of (batch, head, query tile): the work-groups sharing a K/V
//    head stream the same tiles through one L2 at about the same time.
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BR = kBf16QueryTile;  // query rows per work-group
constexpr int BC = 64;              // keys per K/V tile
constexpr int NT = 512;             // threads per work-group (8 waves)
constexpr float kTau = 8.0f;        // lazy-rescale slack, in log2 units
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ int xcd_remap(int wg, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = wg % 8, slot = wg / 8;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Value of x in lane (lane ^ 32), via the gfx950 half-swap.
__device__ __forceinline__ float other_half(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // lanes 0..31: r[1] holds lane+32; lanes 32..63: r[0] holds lane-32
    const unsigned o = (threadIdx.x & 32) ? r[0] : r[1];
    return __builtin_bit_cast(float, o);
}

__device__ __forceinline__ bf16x4 tr_read(const bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (bf16x4 __attribute__((address_space(3))) *)(p));
}

template <int D>
struct Tile {
    static constexpr int KP = D + 8;       // K row pitch (elements)
    static constexpr int VP = D + 16;      // V row pitch (elements)
    static constexpr int CPR = D / 8;      // 16-byte chunks per row
    static constexpr int PT = BC * CPR / NT;  // chunks per thread per tensor
    static_assert(PT >= 1 && BC * CPR % NT == 0, "tile split");
};

template <int D, int MODE>
__global__ __launch_bounds__(NT) void fwd_bf16_kernel(FwdArgs a) {
    using T = Tile<D>;
    constexpr int KP = T::KP, VP = T::VP, PT = T::PT, CPR = T::CPR;
    constexpr int NKK = D / 16;  // 16-deep contractions over the head dimension
    constexpr int NDT = D / 32;  // 32-wide output tiles over the head dimension

    __shared__ __attribute__((aligned(16))) bf16 Ks[2][BC * KP];
    __shared__ __attribute__((aligned(16))) bf16 Vs[2][BC * VP];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int hf = lane >> 5, ln = lane & 31;
    const int g16 = lane >> 4, i16 = lane & 15;

    const int wg = xcd_remap(blockIdx.x, a.n_wg);
    const int qt = wg % a.n_qtiles;
    const int bh = wg / a.n_qtiles;
    const int h = bh % a.H, b = bh / a.H;
    const int g = h / a.group;

    const int64_t q = (int64_t)qt * BR + wave * 32 + ln;
    const bool qvalid = q < a.l_q;
    const int64_t qrow = (int64_t)bh * a.l_q + q;  // flat row of Q / O / m / l

    const bf16 *Kh = (const bf16 *)a.K + b * a.kv_batch_stride + g * a.kv_head_stride;
    const bf16 *Vh = (const bf16 *)a.V + b * a.kv_batch_stride + g * a.kv_head_stride;

    // Resident Q fragment: B operand of S^T = K Q^T, lane holds Q[q][16kk+8hf .. +7].
    bf16x8 qf[NKK];
    {
        const bf16 *qp = (const bf16 *)a.Q + qrow * D + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (qvalid) qf[kk] = *(const bf16x8 *)(qp + 16 * kk);
            else qf[kk] = bf16x8{};
        }
    }

    // Running state per lane (query row ln; lane halves hold different d / keys).
    f32x16 o[NDT];
    float lsum = 0.f;            // this half's partial row sum, relative to R
    float R = -INFINITY;         // exponent reference, log2 units
    float m_nat = -INFINITY;     // exact running max of scale * S
    if constexpr (MODE == MODE_STEP) {
        if (qvalid) {
            m_nat = a.m[qrow];
            R = m_nat * kLog2e;
            if (hf == 0) lsum = a.l[qrow];
            const float *op = a.O + qrow * D + 4 * hf;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 v = *(const f32x4 *)(op + 32 * dt + 8 * i4);
                    o[dt][4 * i4 + 0] = v[0];
                    o[dt][4 * i4 + 1] = v[1];
                    o[dt][4 * i4 + 2] = v[2];
                    o[dt][4 * i4 + 3] = v[3];
                }
        } else {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
        }
    } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] = f32x16{};
    }

    const float c = a.scale_log2;
    const int64_t tiles_per_blk = (a.blk_rows + BC - 1) / BC;
    const int64_t n_tiles = tiles_per_blk * a.n_blocks;

    // Global -> register staging of one K/V tile.
    uint4 kreg[PT], vreg[PT];
    auto load_tile = [&](int64_t it) {
        const int64_t t = it / tiles_per_blk;
        const int64_t tin = it - t * tiles_per_blk;
        int64_t j = (int64_t)a.rank - t;
        if (j < 0) j += a.n_blocks;
        const int64_t row0 = j * a.blk_rows + tin * BC;
        const int64_t nvalid = a.blk_rows - tin * BC;
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int cidx = tid + NT * p;
            const int r = cidx / CPR, cc = cidx % CPR;
            if (r < nvalid) {
                const int64_t off = (row0 + r) * D + cc * 8;
                kreg[p] = *(const uint4 *)(Kh + off);
                vreg[p] = *(const uint4 *)(Vh + off);
            } else {
                kreg[p] = make_uint4(0, 0, 0, 0);
                vreg[p] = make_uint4(0, 0, 0, 0);
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int cidx = tid + NT * p;
            const int r = cidx / CPR, cc = cidx % CPR;
            *(uint4 *)(&Ks[buf][r * KP + cc * 8]) = kreg[p];
            *(uint4 *)(&Vs[buf][r * VP + cc * 8]) = vreg[p];
        }
    };

    if (n_tiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    for (int64_t it = 0; it < n_tiles; ++it) {
        const int buf = (int)(it & 1);
        const int64_t t = it / tiles_per_blk;
        const int64_t tin = it - t * tiles_per_blk;
        if constexpr (MODE == MODE_SHARE) {
            if (a.trace && tin == 0 && wg == 0 && tid == 0) {
                int64_t j = (int64_t)a.rank - t;
                if (j < 0) j += a.n_blocks;
                a.trace[t] = (int32_t)j;
            }
        }
        if (it + 1 < n_tiles) load_tile(it + 1);

        // ---- S^T = K Q^T: two 32-key blocks, lane = query, 16 keys per lane each.
        const bf16 *kt = Ks[buf];
        f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const bf16x8 k0 = *(const bf16x8 *)(kt + ln * KP + 16 * kk + 8 * hf);
            const bf16x8 k1 = *(const bf16x8 *)(kt + (32 + ln) * KP + 16 * kk + 8 * hf);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qf[kk], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qf[kk], s1, 0, 0, 0);
        }
        // s0[i] / s1[i]: key 8*(i/4) + 4*hf + i%4 (+32 for s1) of this tile.
        const int64_t nvalid = a.blk_rows - tin * BC;
        if (nvalid < BC) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 8 * (i >> 2) + 4 * hf + (i & 3);
                if (key >= nvalid) s0[i] = -INFINITY;
                if (key + 32 >= nvalid) s1[i] = -INFINITY;
            }
        }

        // ---- row maximum (in-lane over 32 keys, then across the lane halves)
        float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s0[i], s1[i]));
        mx = fmaxf(mx, other_half(mx));
        m_nat = fmaxf(m_nat, mx * a.scale);
        const float my = mx * c;
        if (__builtin_amdgcn_ballot_w64(my > R + kTau)) {
            const float Rn = fmaxf(R, my);
            const float alpha = __builtin_amdgcn_exp2f(R - Rn);  // R = -inf gives 0
            R = Rn;
            lsum *= alpha;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        }

        // ---- P^T = exp2(S^T c - R), row sums, bf16 packing into PV operands
        const float nR = -R;
        bf16x8 pb[4];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[i], c, nR));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, nR));
            lsum += p0 + p1;
            pb[i >> 3][i & 7] = (bf16)p0;
            pb[2 + (i >> 3)][i & 7] = (bf16)p1;
        }

        // ---- O^T += V^T P^T; contraction c4 covers keys 16*c4 + 8*(j/4) + 4*hf + j%4
        const bf16 *vt = Vs[buf];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16 *vp = vt + (16 * c4 + 4 * hf + (i16 >> 2)) * VP + 32 * dt +
                                 16 * (g16 & 1) + 4 * (i16 & 3);
                const bf16x4 lo = tr_read(vp);
                const bf16x4 hi = tr_read(vp + 8 * VP);
                const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c4], o[dt], 0, 0, 0);
            }
        }

        if (it + 1 < n_tiles) store_tile(buf ^ 1);
        __syncthreads();
    }

    if (!qvalid || n_tiles == 0) return;
    const float ltot = lsum + other_half(lsum);
    // o[dt][4*i4 + e]: head-dim index 32*dt + 8*i4 + 4*hf + e
    if constexpr (MODE == MODE_SHARE) {
        float *op = a.O + qrow * D + 4 * hf;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v = {o[dt][4 * i4] / ltot, o[dt][4 * i4 + 1] / ltot,
                           o[dt][4 * i4 + 2] / ltot, o[dt][4 * i4 + 3] / ltot};
                *(f32x4 *)(op + 32 * dt + 8 * i4) = v;
                if (a.O_cast) {
                    bf16x4 cv = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                    *(bf16x4 *)((bf16 *)a.O_cast + qrow * D + 4 * hf + 32 * dt + 8 * i4) = cv;
                }
            }
        if (hf == 0) {
            if (a.m) a.m[qrow] = m_nat;
            if (a.l) a.l[qrow] = ltot * __builtin_amdgcn_exp2f(R - m_nat * kLog2e);
        }
    } else {
        // Re-express the state relative to the exact running maximum.
        const float f = __builtin_amdgcn_exp2f(R - m_nat * kLog2e);
        float *op = a.O + qrow * D + 4 * hf;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v = {o[dt][4 * i4] * f, o[dt][4 * i4 + 1] * f, o[dt][4 * i4 + 2] * f,
                           o[dt][4 * i4 + 3] * f};
                *(f32x4 *)(op + 32 * dt + 8 * i4) = v;
            }
        if (hf == 0) {
            a.m[qrow] = m_nat;
            a.l[qrow] = ltot * f;
        }
    }
}

template <int D, int MODE>
hipError_t launch(const FwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE>), dim3(a.n_wg), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, int B, int d, int mode, hipStream_t st) {
    (void)B;
    if (d == 128) return mode == MODE_SHARE ? launch<128, MODE_SHARE>(a, st)
                                            : launch<128, MODE_STEP>(a, st);
    if (d == 64) return mode == MODE_SHARE ? launch<64, MODE_SHARE>(a, st)
                                           : launch<64, MODE_STEP>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace ra
