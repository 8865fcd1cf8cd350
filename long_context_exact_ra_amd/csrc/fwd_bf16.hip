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
//  * Software pipeline inside each wave, three tiles deep: A(t) = scores of tile t,
//    B(t) = row max, exp2 and bf16 packing of tile t, C(t) = the P V products of
//    tile t.  Iteration j runs A(j+2), C(j) and B(j+1) stage by stage (one 16-deep
//    slice of each per stage), so the matrix-core work of one wave always has
//    independent vector-ALU work beside it; the second wave on the SIMD fills the
//    remaining gaps.
//  * K and V tiles (64 keys) are double-buffered in LDS, K two tiles ahead of V.
//    Each iteration starts the global loads of K(j+3) and V(j+1) straight into LDS
//    (buffer loads with the LDS bit, no staging registers) and ends with one barrier.  Rows are
//    stored unpadded with XOR swizzles of their 16-byte chunks, chosen so that both
//    the 16-byte K fragment reads and the 4-row V transpose reads are free of bank
//    conflicts.
//  * The exponent reference is updated lazily: the O / l rescale only runs when
//    some row's scaled maximum (log2 units) passed the reference R by more than
//    kTau (a wave-uniform branch), so exp2(s*c - R) stays <= 2^kTau.  The true running maximum is tracked
//    separately and the state is converted to it at the end, so outputs obey
//    m = exact running maximum.
//  * Work-group ids are remapped so each XCD (8 per chip, one L2 each) works on a
//    contiguous range of (batch, head, query tile): the work-groups sharing a K/V
//    head stream the same tiles through one L2 at about the same time.
#include "causal_map.h"
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 8;               // waves per work-group (32 query rows each)
constexpr int BR = 32 * NW;         // query rows per work-group
constexpr int BC = 64;              // keys per K/V tile
constexpr int NH = BC / 32;         // 32-key halves of a tile (one 32x32 score block each)
constexpr int NSTAGE = 2 * NH;      // pipeline stages per tile = 16-key P V contractions
constexpr int NT = 64 * NW;         // threads per work-group
constexpr float kTau = 8.0f;        // lazy-rescale slack, in log2 units
constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw (stride 0) buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, no thread-id addressing; reads past num_records return zero.
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ int xcd_remap(int wg, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = wg % 8, slot = wg / 8;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Ring order: at step t, member `rank` works on block (rank - t) mod n.
__device__ __forceinline__ int64_t ring_block(int32_t rank, int64_t t, int32_t n) {
    int64_t j = (int64_t)rank - t;
    return j < 0 ? j + n : j;
}

// max(x, x in lane ^ 32) in every lane: swapping the upper half of one copy of x with
// the lower half of another leaves (x_lo, x_lo) in one register and (x_hi, x_hi) in the
// other, so their maximum is the both-halves maximum in every lane.
__device__ __forceinline__ float both_halves_max(float x) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]),
                 __builtin_bit_cast(float, (unsigned)r[1]));
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

// Position of one K/V tile in the ring walk, advanced without divisions.
// Blocks may contribute fewer tiles than they hold (a causal share skips key tiles
// that no query of the work-group may attend to); act is the number of tiles of the
// current block that are visited, always a prefix of the block.
struct TileCursor {
    int32_t t;    // ring step
    int32_t tin;  // tile index inside the block
    int32_t act;  // tiles of block j(t) that are visited
    template <typename ActOf>
    __device__ __forceinline__ void next(const ActOf &act_of, int32_t n_blocks) {
        if (++tin == act) {
            tin = 0;
            do {
                ++t;
                act = t < n_blocks ? act_of(t) : 0;
            } while (t < n_blocks && act == 0);
        }
    }
};

template <int D>
struct Tile {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int RPL = 64 / CPR;              // rows filled by one wave-wide load
    static constexpr int WAVE_LOADS = BC * CPR / 64;  // wave-wide loads per K or V tile
    static constexpr int LOADERS = WAVE_LOADS < NW ? WAVE_LOADS : NW;  // waves that load
    static constexpr int ROUND = RPL * LOADERS;       // rows filled by one load per loader
    static constexpr int LOADS = BC / ROUND;          // loads per loading wave per tensor
    static_assert(LOADS >= 1 && BC % ROUND == 0 && LOADS * LOADERS == WAVE_LOADS, "tile split");
};

// LDS tile layouts: rows of D bf16 without padding; the 16-byte chunk c of row r
// sits at position c ^ swz(r).  The LDS serves 256 bytes per clock, so the
// swizzles spread each read's lanes over distinct bytes of a 256-byte window:
//  * K rows are read 16 bytes per lane by consecutive rows at one chunk: with 256-B
//    rows (d = 128) swz_k = r & 15 puts 16 rows on 16 distinct 16-byte slots; with
//    128-B rows (d = 64) rows alternate window halves and swz_k = (r >> 1) & 7.
//  * V rows are read by 4-row transpose loads of 64 bytes (a chunk quad) per row: swz_v
//    moves whole quads (XOR of chunk bits 2-3) so the 4 rows hit 4 distinct 64-byte
//    windows: quad ^ (r & 3) for d = 128, quad ^ ((r >> 1) & 1) for d = 64.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

template <int D, int MODE, bool CAUSAL>
__global__ __launch_bounds__(NT) void fwd_bf16_kernel(FwdArgs a) {
    using T = Tile<D>;
    constexpr int CPR = T::CPR, RPL = T::RPL, ROUND = T::ROUND, LOADS = T::LOADS;
    constexpr int LOADERS = T::LOADERS;
    constexpr int NKK = D / 16;  // 16-deep contractions over the head dimension
    constexpr int NDT = D / 32;  // 32-wide output tiles over the head dimension
    constexpr int TILE = BC * D;  // elements per K or V tile

    __shared__ __attribute__((aligned(1024))) bf16 K0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 K1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 V0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 V1[TILE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep in SGPRs
    const int hf = lane >> 5, ln = lane & 31;
    const int g16 = lane >> 4, i16 = lane & 15;

    // Work-group coordinates are uniform; integer division would otherwise leave them
    // in VGPRs.
    const int wg = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, a.n_wg));
    // A causal share gives later query tiles more keys: start those first.
    const int qt = __builtin_amdgcn_readfirstlane(
        CAUSAL ? a.n_qtiles - 1 - wg % a.n_qtiles : wg % a.n_qtiles);
    const int bh = __builtin_amdgcn_readfirstlane(wg / a.n_qtiles);
    const int h = __builtin_amdgcn_readfirstlane(bh % a.H);
    const int b = __builtin_amdgcn_readfirstlane(bh / a.H);
    const int g = __builtin_amdgcn_readfirstlane(h / a.group);

    // Flat row of Q / O / m / l = row_base (uniform) + qloc (this lane's row).
    const int64_t row_base = (int64_t)bh * a.l_q + (int64_t)qt * BR;
    const int qloc = wave * 32 + ln;
    const bool qvalid = (int64_t)qt * BR + qloc < a.l_q;

    const bf16 *Kh = (const bf16 *)a.K + b * a.kv_batch_stride + g * a.kv_head_stride;
    const bf16 *Vh = (const bf16 *)a.V + b * a.kv_batch_stride + g * a.kv_head_stride;

    // Resident Q fragment: B operand of S^T = K Q^T, lane holds Q[q][16kk+8hf .. +7].
    bf16x8 qf[NKK];
    {
        const bf16 *qp = (const bf16 *)a.Q + row_base * D + (qloc * D + 8 * hf);
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (qvalid) qf[kk] = *(const bf16x8 *)(qp + 16 * kk);
            else qf[kk] = bf16x8{};
        }
    }

    // Running state per lane (query row ln; lane halves hold different d / keys).
    f32x16 o[NDT];
    float lsum = 0.f;         // this half's partial row sum, relative to R
    float tsum = 0.f;         // the same over the current tile only (blocked summation)
    float R = -INFINITY;      // exponent reference, log2 units
    float m_nat = -INFINITY;  // exact running max of scale * S
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        o[dt] = f32x16{};
        asm volatile("" : "+v"(o[dt]));  // no special-cased first products
    }
    if constexpr (MODE == MODE_STEP) {
        if (qvalid) {
            m_nat = a.m[row_base + qloc];
            R = m_nat * kLog2e;
            if (hf == 0) lsum = a.l[row_base + qloc];
            const float *op = a.O + row_base * D + (qloc * D + 4 * hf);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const f32x4 v = *(const f32x4 *)(op + 32 * dt + 8 * i4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[dt][4 * i4 + e] = v[e];
                }
        }
    }

    const float c = a.scale_log2;
    // The host guarantees the tile count of a launch fits in int32.
    const int32_t tiles_per_blk = (int32_t)((a.blk_rows + BC - 1) / BC);
    const CausalMap cmap{a.layout, a.rank, a.n_blocks, (int32_t)a.blk_rows};
    // Last valid local query of the work-group (uniform); positions grow with it.
    const int64_t a_end = (int64_t)(qt + 1) * BR;
    const int32_t a_max = (int32_t)((a.l_q < a_end ? a.l_q : a_end) - 1);
    auto act_of = [&](int32_t t) -> int32_t {
        if constexpr (!CAUSAL) return tiles_per_blk;
        else return cmap.active_tiles((int32_t)ring_block(a.rank, t, a.n_blocks), a_max, BC,
                                      tiles_per_blk);
    };
    int32_t n_tiles = tiles_per_blk * a.n_blocks;
    if constexpr (CAUSAL) {
        n_tiles = 0;
        for (int32_t t = 0; t < a.n_blocks; ++t) n_tiles += act_of(t);
    }

    // ---- direct global -> LDS tile loads (no staging registers), through buffer
    // resources over this work-group's K and V heads.  The buffer form (rather than
    // global_load_lds) keeps LDS reads countable in order: with a flat-encoded LDS DMA
    // in flight every LDS wait degenerates to lgkmcnt(0), which serialises each matrix
    // product behind the most recent fragment read.  Load p of wave w fills tile rows
    // p*ROUND + w*RPL + lane/CPR; lane % CPR is the chunk slot.  One per-lane byte
    // offset per tensor serves every load (loads are ROUND >= 32 rows apart and the
    // swizzles repeat every 16 rows); the row base goes in the scalar offset.
    const int head_bytes = (int)((int64_t)a.n_blocks * a.blk_rows * (D * 2));  // host: < 2^31
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)Kh, 0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)Vh, 0, head_bytes, kRsrcWord3);
    const int lrow = wave * RPL + lane / CPR;  // row of load 0
    const uint32_t koff_g = (uint32_t)(lrow * D + ((lane % CPR) ^ swz_k<D>(lrow)) * 8) * 2;
    const uint32_t voff_g = (uint32_t)(lrow * D + ((lane % CPR) ^ swz_v<D>(lrow)) * 8) * 2;
    auto load_tile = [&](__amdgpu_buffer_rsrc_t rs, const TileCursor &cur, bf16 *dst,
                         uint32_t off, bool is_v) {
        if (LOADERS < NW && wave >= LOADERS) return;  // the tile needs fewer waves
        const int64_t row0 =
            ring_block(a.rank, cur.t, a.n_blocks) * a.blk_rows + (int64_t)cur.tin * BC;
        const int64_t left = a.blk_rows - (int64_t)cur.tin * BC;  // keys left in the block
        const uint32_t soff = (uint32_t)(row0 * (D * 2));           // wave-uniform
        bf16 *ldst = dst + wave * RPL * D;
        if (left >= BC) {
#pragma unroll
            for (int p = 0; p < LOADS; ++p)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (void __attribute__((address_space(3))) *)(ldst + p * ROUND * D), 16,
                    (int)off, (int)(soff + (uint32_t)(p * ROUND * D * 2)), 0, 0);
        } else {
            // Ragged tail: rows past the block end repeat its last row; those keys are
            // masked, so their probabilities are exactly 0.
            const int last = (int)left - 1;
            int ln2 = lane;
            asm volatile("" : "+v"(ln2));  // recompute the slot here (rare path)
            const int lr = wave * RPL + ln2 / CPR;
            const int slot = (ln2 % CPR) ^ (is_v ? swz_v<D>(lr) : swz_k<D>(lr));
#pragma unroll
            for (int p = 0; p < LOADS; ++p) {
                const int r = p * ROUND + lr;
                const int rr = r < last ? r : last;
                const uint32_t o2 = (uint32_t)(rr * D + slot * 8) * 2;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (void __attribute__((address_space(3))) *)(ldst + p * ROUND * D), 16,
                    (int)o2, (int)soff, 0, 0);
            }
        }
    };

    // ---- S^T = K Q^T for one tile: lane = query, 16 keys per lane per 32-key block.
    // sc.h[b][i] holds key 32*b + 8*(i/4) + 4*hf + i%4 of the tile.  Two score sets
    // alternate: one is consumed by the softmax while the next tile's products
    // accumulate into the other.
    struct Scores {
        f32x16 h[NH];
    };
    Scores sx, sy;
    // K fragment addresses: row ln (+32*b, same swizzle), chunk (2*kk + hf) ^ sw.
    // Element offset 8*((2*kk + hf) ^ sw) = 16*(kk ^ (sw >> 1)) + 8*(hf ^ (sw & 1)), so
    // with kbase holding the sw terms the read for kk is at kbase ^ (16*kk): the kk bits
    // (4..6) are disjoint from the row and half bits.
    const int kbase = [&] {
        const int sw = swz_k<D>(ln);
        return ln * D + 8 * (hf ^ (sw & 1)) + 16 * (sw >> 1);
    }();
    // Byte offsets of the K fragment reads, one per 16-deep contraction, computed once and
    // kept in registers (opaque to the compiler, so it does not re-derive them per tile).
    uint32_t kob[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
        kob[kk] = (uint32_t)(kbase ^ (16 * kk)) * 2u;
        asm volatile("" : "+v"(kob[kk]));
    }
    constexpr int KK_STAGE = NKK / NSTAGE;  // contractions per pipeline stage
    static_assert(KK_STAGE >= 1 && NKK % NSTAGE == 0, "stage split");
    auto scores_stage = [&](const bf16 *kt, Scores &d, int stage) {
#pragma unroll
        for (int u = 0; u < KK_STAGE; ++u) {
            const int kk = stage * KK_STAGE + u;
            const bf16 *kp = (const bf16 *)((const char *)kt + kob[kk]);
#pragma unroll
            for (int b = 0; b < NH; ++b) {
                const bf16x8 kf = *(const bf16x8 *)(kp + 32 * b * D);
                d.h[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], d.h[b], 0, 0, 0);
            }
        }
    };
    auto zero_scores = [&](Scores &d) {
#pragma unroll
        for (int b = 0; b < NH; ++b) d.h[b] = f32x16{};
    };
    auto scores_full = [&](const bf16 *kt, Scores &d) {
        zero_scores(d);
#pragma unroll
        for (int stage = 0; stage < NSTAGE; ++stage) {
            scores_stage(kt, d, stage);
            __builtin_amdgcn_sched_barrier(0);  // bound operand prefetch
        }
    };
    // Row max of a score set (raw dot units), both lane halves combined.
    auto row_max = [&](const Scores &d) {
        float ma = d.h[0][0], mb = d.h[0][1];
#pragma unroll
        for (int b = 0; b < NH; ++b)
#pragma unroll
            for (int i = (b == 0 ? 2 : 0); i < 16; i += 4) {
                ma = fmaxf(fmaxf(ma, d.h[b][i]), d.h[b][i + 2]);
                mb = fmaxf(fmaxf(mb, d.h[b][i + 1]), d.h[b][i + 3]);
            }
        return both_halves_max(fmaxf(ma, mb));
    };

    // Keys past the end of a partial tile, and keys a causal share may not attend to,
    // get score -inf.
    const int32_t a_lane = qt * BR + qloc;  // this lane's local query index
    // mx holds the row maximum of d taken before masking; a tile that needs masking gets
    // it taken again afterwards.
    auto mask_scores = [&](Scores &d, const TileCursor &cur, float &mx) {
        const int64_t nvalid = a.blk_rows - (int64_t)cur.tin * BC;
        int keys = nvalid < BC ? (int)nvalid : BC;  // admissible prefix of the tile
        bool partial = keys < BC;
        if constexpr (CAUSAL) {
            const int32_t j = (int32_t)ring_block(a.rank, cur.t, a.n_blocks);
            keys = min(keys, max(cmap.allowed(a_lane, j, cur.tin * BC), 0));
            partial = __builtin_amdgcn_ballot_w64(keys < BC) != 0;  // wave-uniform
        }
        if (partial) {
            // key index = 32*b + 8*(i/4) + i%4 + 4*hf: compare the constant part with a
            // per-lane limit (no per-key registers).
            const int lim = keys - 4 * hf;
#pragma unroll
            for (int b = 0; b < NH; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * b + 8 * (i >> 2) + (i & 3) >= lim) d.h[b][i] = -INFINITY;
            mx = row_max(d);
        }
    };

    // Softmax numerators of a score set, packed into the PV operands.  Operand c4
    // covers keys 16*c4 + 8*(j/4) + 4*hf + j%4, j = 0..7, i.e. elements 8*(c4%2) + j of
    // score block c4/2.
    const bf16x2 ones = {(bf16)1.0f, (bf16)1.0f};
    auto softmax_part = [&](const Scores &d, bf16x8 *pb, int part) {
        const float nR = -R;
        const f32x16 &sv = d.h[part >> 1];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const int i = 8 * (part & 1) + e;
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c, nR));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i + 1], c, nR));
            const bf16x2 pk = {(bf16)p0, (bf16)p1};
            // Each tile's 16 probabilities per lane are summed on their own and the tile
            // sum is then added to the running sum: the rounding error grows with the
            // number of tiles, not the number of keys.
            tsum = __builtin_amdgcn_fdot2_f32_bf16(ones, pk, (part | e) == 0 ? 0.f : tsum, false);
            pb[part][e] = pk[0];
            pb[part][e + 1] = pk[1];
        }
    };

    // O^T += V^T P^T for contraction c4 of a tile.  The 16 lanes of group g16 read
    // rows 16*c4 + 4*hf + 0..3 (then +8) and head-dim columns 32*dt + 16*(g16&1) + 0..15,
    // i.e. chunk 4*dt + x with x = 2*(g16&1) + (i16&3)/2 of quad dt, stored in quad
    // dt ^ (swz_v / 4).  Element offset 32*(dt ^ s) + 8*x + 4*(i16&1) = vbase ^ (32*dt).
    const int vbase = [&] {
        const int vrow = 4 * hf + (i16 >> 2);  // row within each 16-row contraction
        const int sq = swz_v<D>(vrow) >> 2;    // rows 16*c4 + vrow (+8) share it
        const int x = 2 * (g16 & 1) + ((i16 & 3) >> 1);
        return vrow * D + 32 * sq + 8 * x + 4 * (i16 & 1);
    }();
    uint32_t vob[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        vob[dt] = (uint32_t)(vbase ^ (32 * dt)) * 2u;
        asm volatile("" : "+v"(vob[dt]));
    }
    auto pv_part = [&](const bf16 *vt, const bf16x8 *pb, int c4) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const bf16 *vp = (const bf16 *)((const char *)vt + vob[dt]) + 16 * c4 * D;
            const bf16x4 lo = tr_read(vp);
            const bf16x4 hi = tr_read(vp + 8 * D);
            const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[c4], o[dt], 0, 0, 0);
        }
    };

    // Raise the exponent reference to cover a new row maximum (raw units), lazily: only
    // when some row of the wave grew past R + kTau.  Returns the factor alpha that the
    // running output must be multiplied by once the products issued under the old
    // reference are done (1 when nothing changed); the row sum is rescaled here.
    auto update_reference = [&](float mx, bool &changed) {
        m_nat = fmaxf(m_nat, mx * a.scale);
        changed = __builtin_amdgcn_ballot_w64(mx * c > R + kTau) != 0;
        float alpha = 1.0f;
        if (changed) {
            const float Rn = fmaxf(R, mx * c);
            alpha = __builtin_amdgcn_exp2f(R - Rn);  // R = -inf gives 0
            R = Rn;
            lsum *= alpha;
        }
        return alpha;
    };
    auto rescale_output = [&](float alpha) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    };

    // Pipeline per tile t: A(t) scores, B(t) max + softmax, C(t) P V.  Iteration j
    // runs A(j+2), B(j+1) and C(j), which are independent, stage by stage.
    // Buffers: K(t) lives in K[t & 1], V(t) in V[t & 1]; S(t) in score set t & 1.
    const int32_t act0 = act_of(0);  // the member's own block: its first tile always counts
    TileCursor cK{0, 0, act0}, cV{0, 0, act0}, cM{0, 0, act0};  // next K/V load, next softmax

    // ---- prologue: K(0), K(1), V(0) into LDS; A(0), B(0), A(1); then K(2).
    load_tile(krs, cK, K0, koff_g, false);
    cK.next(act_of, a.n_blocks);
    load_tile(vrs, cV, V0, voff_g, true);
    cV.next(act_of, a.n_blocks);
    if (n_tiles > 1) {
        load_tile(krs, cK, K1, koff_g, false);
        cK.next(act_of, a.n_blocks);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads landed
    __syncthreads();

    bf16x8 pp[NSTAGE];  // packed softmax numerators of the tile whose P V product is next
    // Row maximum of the score set the next iteration consumes, taken before masking (the
    // mask takes it again on the tiles that need one).
    float mx_next = -INFINITY;
    {
        scores_full(K0, sx);
        float mx0 = row_max(sx);
        mask_scores(sx, cM, mx0);
        cM.next(act_of, a.n_blocks);
        bool changed;
        const float alpha = update_reference(mx0, changed);
        if (changed) rescale_output(alpha);
#pragma unroll
        for (int part = 0; part < NSTAGE; ++part) softmax_part(sx, pp, part);
        lsum += tsum;
        if (n_tiles > 1) {
            scores_full(K1, sy);
            mx_next = row_max(sy);
        }
    }
    __syncthreads();  // every wave is done with K buffer 0
    if (n_tiles > 2) {
        load_tile(krs, cK, K0, koff_g, false);
        cK.next(act_of, a.n_blocks);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

    // Iteration j with A(j+2): consumes S(j+1) from cs, accumulates S(j+2) into ns from
    // K[j & 1], multiplies P(j) by V[j & 1]; loads K(j+3) into K[(j+1) & 1] and V(j+1)
    // into V[(j+1) & 1].
    auto full_iteration = [&](int32_t j, Scores &cs, Scores &ns, const bf16 *kcur, bf16 *knext,
                              const bf16 *vcur, bf16 *vnext) {
        if (j + 3 < n_tiles) {
            load_tile(krs, cK, knext, koff_g, false);
            cK.next(act_of, a.n_blocks);
        }
        load_tile(vrs, cV, vnext, voff_g, true);
        cV.next(act_of, a.n_blocks);
        mask_scores(cs, cM, mx_next);
        cM.next(act_of, a.n_blocks);
        bool changed;
        const float alpha = update_reference(mx_next, changed);
        zero_scores(ns);
#pragma unroll
        for (int stage = 0; stage < NSTAGE; ++stage) {
            scores_stage(kcur, ns, stage);
            pv_part(vcur, pp, stage);
            softmax_part(cs, pp, stage);  // P(j+1) replaces P(j) after its product
        }
        lsum += tsum;
        // The row maximum of tile j+2 here, before the barrier, so that the next iteration
        // can start its exponentials while its first fragment reads land.
        mx_next = row_max(ns);
        // Keep the numerators of tile j+1 (and that maximum) in this block.  Left alone,
        // the compiler sinks them past the rescale branch into the next iteration's block,
        // so every other block has all the exponentials and the others have none beside
        // their products.
        asm volatile("" ::"v"(pp[0]), "v"(pp[1]), "v"(pp[2]), "v"(pp[3]), "v"(lsum),
                     "v"(mx_next));
        if (changed) rescale_output(alpha);  // after the old-reference products
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads landed
        __syncthreads();
    };
    // Iteration j without a next score tile (the last but one tile).
    auto tail_iteration = [&](Scores &cs, const bf16 *vcur, bf16 *vnext) {
        load_tile(vrs, cV, vnext, voff_g, true);
        cV.next(act_of, a.n_blocks);
        mask_scores(cs, cM, mx_next);
        cM.next(act_of, a.n_blocks);
        bool changed;
        const float alpha = update_reference(mx_next, changed);
#pragma unroll
        for (int stage = 0; stage < NSTAGE; ++stage) {
            pv_part(vcur, pp, stage);
            softmax_part(cs, pp, stage);
        }
        lsum += tsum;
        if (changed) rescale_output(alpha);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    int32_t j = 0;
    for (; j + 3 < n_tiles; j += 2) {  // iterations j and j+1 both have a score stage
        full_iteration(j, sy, sx, K0, K1, V0, V1);
        full_iteration(j + 1, sx, sy, K1, K0, V1, V0);
    }
    if (j + 2 < n_tiles) {  // j even
        full_iteration(j, sy, sx, K0, K1, V0, V1);
        ++j;
    }
    if (j + 1 < n_tiles) {
        if (j & 1) tail_iteration(sx, V1, V0);
        else tail_iteration(sy, V0, V1);
        ++j;
    }
    // Last tile: its P V product only.
#pragma unroll
    for (int c4 = 0; c4 < NSTAGE; ++c4) pv_part((j & 1) ? V1 : V0, pp, c4);

    if constexpr (MODE == MODE_SHARE) {
        // The ring order the loads above followed, one entry per step.
        if (a.trace && wg == 0)
            for (int t = tid; t < a.n_blocks; t += NT)
                a.trace[t] = (int32_t)ring_block(a.rank, t, a.n_blocks);
    }
    if (!qvalid) return;
    const float ltot = lsum + other_half(lsum);
    const int ooff = qloc * D + 4 * hf;  // this lane's output offset past row_base * D
    // o[dt][4*i4 + e]: head-dim index 32*dt + 8*i4 + 4*hf + e
    if constexpr (MODE == MODE_SHARE) {
        float *op = a.O + row_base * D + ooff;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v = {o[dt][4 * i4] / ltot, o[dt][4 * i4 + 1] / ltot,
                           o[dt][4 * i4 + 2] / ltot, o[dt][4 * i4 + 3] / ltot};
                *(f32x4 *)(op + 32 * dt + 8 * i4) = v;
                if (a.O_cast) {
                    bf16x4 cv = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                    *(bf16x4 *)((bf16 *)a.O_cast + row_base * D + ooff + 32 * dt + 8 * i4) = cv;
                }
            }
        if (hf == 0) {
            if (a.m) a.m[row_base + qloc] = m_nat;
            if (a.l) a.l[row_base + qloc] = ltot * __builtin_amdgcn_exp2f(R - m_nat * kLog2e);
        }
    } else {
        // Re-express the state relative to the exact running maximum.
        const float f = __builtin_amdgcn_exp2f(R - m_nat * kLog2e);
        float *op = a.O + row_base * D + ooff;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                f32x4 v = {o[dt][4 * i4] * f, o[dt][4 * i4 + 1] * f, o[dt][4 * i4 + 2] * f,
                           o[dt][4 * i4 + 3] * f};
                *(f32x4 *)(op + 32 * dt + 8 * i4) = v;
            }
        if (hf == 0) {
            a.m[row_base + qloc] = m_nat;
            a.l[row_base + qloc] = ltot * f;
        }
    }
}

template <int D, int MODE, bool CAUSAL = false>
hipError_t launch(const FwdArgs &a, hipStream_t st) {
    hipLaunchKernelGGL((fwd_bf16_kernel<D, MODE, CAUSAL>), dim3(a.n_wg), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int bf16_query_tile() { return BR; }

hipError_t launch_fwd_bf16(const FwdArgs &a, int B, int d, int mode, hipStream_t st) {
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
