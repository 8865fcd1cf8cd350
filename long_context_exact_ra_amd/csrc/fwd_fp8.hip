// fwd_fp8.hip -- one ring member's attention share from FP8 (OCP e4m3) inputs, gfx950
// matrix cores (v_mfma_f32_32x32x64_f8f6f4), fp32 statistics.
//
// Same blockwise algorithm as the bf16 share (slowleelab "Ring Attention" page, 4.2 and
// 4.3; aliyun FlashAttention explainer, section 2), with both products on the FP8 matrix
// path and block-quantized inputs (the FlashAttention-3 paragraph of the aliyun page):
//   score s = scale * qs * ks * (q8 . k8)      qs per 64 query rows, ks per 64-key tile
//   P = e4m3(exp2(s log2e - R))               the probabilities are themselves FP8
//   O = vs * (sum P v8) / (sum P)              vs per channel, applied at the end
// The row sum runs on the matrix core too (a product with a matrix of ones), so it sums
// exactly the FP8 probabilities that weight the values.
//
// MI355X mapping (differences from the bf16 kernel):
//  * One 32x32x64 product contracts 64 keys (or 64 head-dim entries) at once, so P of a
//    whole tile feeds each P V product: P is double-buffered across tiles.
//  * K tile rows are stored in LDS in a permuted order so that the score layout gives
//    each lane 16 *consecutive* keys per 32-key block (lane half hf holds keys
//    16 hf .. 16 hf + 15): the packed P bytes are then contiguous key ranges, and the
//    matching V^T operand is two 16-byte LDS reads of a transposed V tile.  V arrives
//    already transposed per tile (the quantizer writes it so), so no transpose loads.
//  * LDS rows are padded by 16 bytes instead of swizzled: conflict-free, and every
//    fragment address is one base register plus a constant.
//  * Exponent reference: a new reference puts the row maximum at 2^4 and is raised only
//    when the maximum grows past 2^8, so P stays below the E4M3 limit 448 and ordinary
//    probabilities stay clear of the format's subnormal range.
//  * Each tile's K scale reaches the lanes with a vector buffer load issued a tile ahead
//    (a scalar load would force waits on every outstanding LDS read).
#include "causal_map.h"
#include "ra_internal.h"

namespace ra {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16;
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 8;           // waves per work-group (32 query rows each)
constexpr int BR = 32 * NW;     // query rows per work-group
constexpr int BC = 64;          // keys per tile
constexpr int NT = 64 * NW;
constexpr float kSlack = 8.0f;  // P <= 2^8 between reference updates
constexpr float kHead = 4.0f;   // a new reference maps the row maximum to 2^4
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFltMin = 1.17549435e-38f;
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOnes = 0x38383838;  // four E4M3 ones

__device__ __forceinline__ int xcd_remap(int wg, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = wg % 8, slot = wg / 8;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

__device__ __forceinline__ int32_t ring_block(int32_t rank, int32_t t, int32_t n) {
    const int32_t j = rank - t;
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

__device__ __forceinline__ f32x16 mfma8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    // e4m3 x e4m3, no block scales (scale operands 0 select the unscaled instruction)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 join(const i32x4 &lo, const i32x4 &hi) {
    return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// LDS row r of a K tile holds key perm(r): inside each 32-row block, row 8a + 4h + b
// (the score layout's row for lane half h, element 4a + b) holds key 16h + 4a + b.
__device__ __forceinline__ int key_of_row(int r) {
    return 32 * (r >> 5) + 16 * ((r >> 2) & 1) + 4 * ((r >> 3) & 3) + (r & 3);
}

// Ring step t, tile tin of block j(t); act = tiles of that block that are visited (all
// of them, or for a causal share the prefix some query of the work-group may see).
struct Cursor {
    int32_t t, tin, act;
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

template <int D, bool CAUSAL>
__global__ __launch_bounds__(NT) void fwd_fp8_kernel(Fp8Args a) {
    constexpr int NKK = D / 64;        // 64-deep contractions over the head dimension
    constexpr int NDT = D / 32;        // 32-wide output tiles over the head dimension
    constexpr int TB = BC * D;         // bytes per K tile and per V^T tile in HBM
    // LDS rows are padded by 16 bytes, which spreads 16 consecutive rows over distinct
    // 16-byte slots of the 256-byte LDS window (row strides of 9 or 5 slots), so every
    // fragment read is a base register plus a constant offset.
    constexpr int KROW = D + 16, VROW = BC + 16;
    constexpr int KTB = BC * KROW, VTB = D * VROW;       // padded tile bytes in LDS
    constexpr int KLD = KTB / 1024, VLD = VTB / 1024;    // 1 KB loads per tile
    static_assert(KTB % 1024 == 0 && VTB % 1024 == 0 && KLD <= 2 * NW && VLD <= 2 * NW, "loads");

    // One array per buffer: the compiler tells the tile loads into one buffer apart from
    // the fragment reads of the other only when they are distinct __shared__ objects, and
    // otherwise waits for the loads (vmcnt) before every read.
    __shared__ __attribute__((aligned(1024))) uint8_t Ks0[KTB];
    __shared__ __attribute__((aligned(1024))) uint8_t Ks1[KTB];
    __shared__ __attribute__((aligned(1024))) uint8_t Vs0[VTB];
    __shared__ __attribute__((aligned(1024))) uint8_t Vs1[VTB];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, ln = lane & 31;

    const int wg = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, a.n_wg));
    // A causal share gives later query tiles more keys: start those first.
    const int qt = __builtin_amdgcn_readfirstlane(
        CAUSAL ? a.n_qtiles - 1 - wg % a.n_qtiles : wg % a.n_qtiles);
    const int bh = __builtin_amdgcn_readfirstlane(wg / a.n_qtiles);
    const int h = __builtin_amdgcn_readfirstlane(bh % a.H);
    const int b = __builtin_amdgcn_readfirstlane(bh / a.H);
    const int g = __builtin_amdgcn_readfirstlane(h / a.group);
    const int32_t T = a.n_tiles_blk;
    const int32_t N = a.n_blocks;
    const int64_t l = a.l_q;

    const int64_t row_base = (int64_t)bh * l + (int64_t)qt * BR;
    const int qloc = wave * 32 + ln;
    const int64_t qrow = (int64_t)qt * BR + qloc;  // local query index
    const bool qvalid = qrow < l;

    // Resident Q fragment: lane (ln, hf) holds bytes 64 kk + 32 hf .. + 31 of its row.
    i32x8 qf[NKK];
    float c_lane = 0.f;  // scale * log2(e) * (this row's Q descale)
    {
        const uint8_t *qp = a.Q8 + (row_base + qloc) * D + 32 * hf;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            if (qvalid) qf[kk] = join(*(const i32x4 *)(qp + 64 * kk), *(const i32x4 *)(qp + 64 * kk + 16));
            else qf[kk] = i32x8{};
        }
        const float qs = qvalid ? a.qs[(int64_t)bh * T + qrow / BC] : 1.f;
        c_lane = a.scale * kLog2e * qs;
    }

    f32x16 o[NDT], lacc;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        o[dt] = f32x16{};
        asm volatile("" : "+v"(o[dt]));
    }
    lacc = f32x16{};
    asm volatile("" : "+v"(lacc));
    float Rp = -INFINITY;     // exponent reference, log2 units
    float m_nat = -INFINITY;  // exact running max of the natural scores

    // ---- tile loads straight into LDS (buffer loads with the LDS bit)
    const int64_t kvh = (int64_t)b * a.H_kv + g;  // K/V head
    const uint8_t *Kh = a.K8 + kvh * (int64_t)N * l * D;
    const uint8_t *Vh = a.V8 + kvh * (int64_t)N * T * TB;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)Kh, 0, (int)((int64_t)N * l * D), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)Vh, 0, (int)((int64_t)N * T * TB), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t srs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(a.ks + kvh * (int64_t)N * T), 0, (int)((int64_t)N * T * 4), kRsrcWord3);
    // Load i (wave i % NW) fills LDS bytes 1024 i + 16 lane of a tile: K row r = that /
    // KROW holds key key_of_row(r), byte q = that % KROW of it (q >= D: padding, filled
    // with any in-range bytes); V^T row d = that / VROW, byte q of the stored row.
    auto k_slot = [&](int i, int &key, int &q) {
        const int o = 1024 * i + 16 * lane;
        key = key_of_row(o / KROW);
        q = o % KROW;
        if (q >= D) q = 0;
    };
    auto v_slot = [&](int i) {
        const int o = 1024 * i + 16 * lane, q = o % VROW;
        return (o / VROW) * BC + (q < BC ? q : 0);
    };
    int k_key0, k_q0, k_key1 = 0, k_q1 = 0;
    k_slot(wave, k_key0, k_q0);
    if (wave + NW < KLD) k_slot(wave + NW, k_key1, k_q1);
    const int v_off0 = v_slot(wave), v_off1 = wave + NW < VLD ? v_slot(wave + NW) : 0;

    auto load_k = [&](const Cursor &cu, uint8_t *dst) {
        const int32_t j = ring_block(a.rank, cu.t, N);
        const int64_t row0 = (int64_t)j * l + (int64_t)cu.tin * BC;
        const int64_t left = l - (int64_t)cu.tin * BC;
        auto one = [&](int i, int key, int q) {
            if (left < BC && key >= left) key = (int)left - 1;  // ragged: repeat the last row
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                krs, (void __attribute__((address_space(3))) *)(dst + 1024 * i), 16,
                key * D + q, (int)(row0 * D), 0, 0);
        };
        if (wave < KLD) one(wave, k_key0, k_q0);
        if (wave + NW < KLD) one(wave + NW, k_key1, k_q1);
    };
    auto load_v = [&](const Cursor &cu, uint8_t *dst) {
        const int32_t j = ring_block(a.rank, cu.t, N);
        const int64_t tile = (int64_t)j * T + cu.tin;
        if (wave < VLD)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrs, (void __attribute__((address_space(3))) *)(dst + 1024 * wave), 16, v_off0,
                (int)(tile * TB), 0, 0);
        if (wave + NW < VLD)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                vrs, (void __attribute__((address_space(3))) *)(dst + 1024 * (wave + NW)), 16,
                v_off1, (int)(tile * TB), 0, 0);
    };
    auto load_scale = [&](const Cursor &cu) {
        const int32_t j = ring_block(a.rank, cu.t, N);
        return __builtin_bit_cast(
            float, __builtin_amdgcn_raw_buffer_load_b32(srs, 0, (int)(((int64_t)j * T + cu.tin) * 4), 0));
    };

    // ---- products
    struct Scores {
        f32x16 h[2];  // h[kb][i]: key 32 kb + 16 hf + i of the tile
    };
    // Score product s of a tile (s = 0 .. NDT-1): block kb = s / NKK, contraction kk.
    const int kbase = ln * KROW + 32 * hf;  // row ln, bytes 32 hf .. of each 64-byte step
    auto k_frag = [&](const uint8_t *kt, int kb0, int s) {
        const uint8_t *p = kt + kb0 + (s / NKK) * 32 * KROW + 64 * (s % NKK);
        return join(*(const i32x4 *)p, *(const i32x4 *)(p + 16));
    };
    auto score_mfma = [&](const uint8_t *kt, int kb0, Scores &d, int s) {
        const int kb = s / NKK, kk = s % NKK;
        if (kk == 0) d.h[kb] = f32x16{};
        d.h[kb] = mfma8(k_frag(kt, kb0, s), qf[kk], d.h[kb]);
    };
    auto laundered = [](int x) {
        asm volatile("" : "+v"(x));  // derive read offsets where used, not kept live
        return x;
    };
    auto scores = [&](const uint8_t *kt, Scores &d) {
        const int kb0 = laundered(kbase);
#pragma unroll
        for (int st = 0; st < NDT; ++st) score_mfma(kt, kb0, d, st);
    };
    const int vbase = ln * VROW + 16 * hf;  // row ln: keys 16 hf .. and 32 + 16 hf ..
    auto v_frag = [&](const uint8_t *vt, int vb, int dt) {
        const uint8_t *p = vt + vb + 32 * VROW * dt;
        return join(*(const i32x4 *)p, *(const i32x4 *)(p + 32));
    };
    auto pv_mfma = [&](const uint8_t *vt, int vb, const i32x8 &pb, int dt) {
        o[dt] = mfma8(v_frag(vt, vb, dt), pb, o[dt]);
    };
    // Kept resident: rebuilt before each use, the eight moves would sit right before
    // the product that reads them and stall it (measured: 12 % of the kernel's time).
    i32x8 ones = {kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes, kOnes};
    asm volatile("" : "+v"(ones));
    auto sum_mfma = [&](const i32x8 &pb) {  // row sums of the FP8 probabilities
        lacc = mfma8(ones, pb, lacc);
    };
    auto pv = [&](const uint8_t *vt, const i32x8 &pb) {
        const int vb = laundered(vbase);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) pv_mfma(vt, vb, pb, dt);
        sum_mfma(pb);
    };

    // ---- softmax pieces
    // Rare paths (a ragged last tile, a raised reference) stay behind real branches: the
    // empty volatile asm keeps the compiler from turning them into selects and multiplies
    // executed on every tile.
    // Keys past a block's end and, for a causal share, keys after this lane's query get
    // score -inf (the limit is per lane; the branch is wave-uniform).
    const CausalMap cmap{a.layout, a.rank, N, (int32_t)l};
    auto mask_scores = [&](Scores &d, const Cursor &cu) {
        const int64_t left = l - (int64_t)cu.tin * BC;
        int keys = left < BC ? (int)left : BC;
        bool partial = keys < BC;
        if constexpr (CAUSAL) {
            const int32_t j = ring_block(a.rank, cu.t, N);
            keys = min(keys, max(cmap.allowed((int32_t)qrow, j, cu.tin * BC), 0));
            partial = __builtin_amdgcn_ballot_w64(keys < BC) != 0;
        }
        if (!partial) return;
        asm volatile("" ::: "memory");
        const int lim = keys - 16 * hf;  // key = 32 kb + 16 hf + i
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (32 * kb + i >= lim) d.h[kb][i] = -INFINITY;
    };
    auto row_max = [&](const Scores &d) {
        float ma = fmaxf(d.h[0][0], d.h[0][1]), mb = fmaxf(d.h[1][0], d.h[1][1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) {
            ma = fmaxf(fmaxf(ma, d.h[0][i]), d.h[0][i + 1]);
            mb = fmaxf(fmaxf(mb, d.h[1][i]), d.h[1][i + 1]);
        }
        const float mx = fmaxf(ma, mb);
        return both_halves_max(mx);
    };
    // Raise the reference when some row of the wave would exceed 2^kSlack; returns the
    // factor for the output and row sums accumulated under the old reference.
    auto update_reference = [&](float mx, float ct, bool &changed) {
        const float mc = mx * ct;  // log2 units
        m_nat = fmaxf(m_nat, mc * kLn2);
        changed = __builtin_amdgcn_ballot_w64(mc > Rp + kSlack) != 0;
        float alpha = 1.0f;
        if (changed) {
            const float Rn = fmaxf(Rp, mc - kHead);
            alpha = __builtin_amdgcn_exp2f(Rp - Rn);  // Rp = -inf gives 0
            Rp = Rn;
        }
        return alpha;
    };
    // Probabilities of dword q4 (elements 4 (q4 % 4) .. + 3 of block q4 / 4) as E4M3.
    auto softmax_dw = [&](const Scores &d, i32x8 &pb, int q4, float ct) {
        const f32x16 &sv = d.h[q4 >> 2];
        const int i0 = 4 * (q4 & 3);
        const float nR = -Rp;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i0], ct, nR));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i0 + 1], ct, nR));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i0 + 2], ct, nR));
        const float p3 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i0 + 3], ct, nR));
        // Both halves of the word are written, so its previous contents (this operand's
        // P of the tile before, already consumed) only name the register.
        const int w = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pb[q4], false);
        pb[q4] = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, w, true);
    };
    auto rescale = [&](float alpha) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
        lacc *= alpha;
    };
    auto tile_scale = [&](float ks) { return fmaxf(c_lane * ks, kFltMin); };

    // ---- pipeline (as the bf16 kernel): iteration j computes the scores of tile j+2,
    // the softmax of tile j+1 and the P V products of tile j.  K(t) in Ks0 / Ks1 and V(t)
    // in Vs0 / Vs1 by the parity of t, P(t) in pb[t & 1]; ks_cur is the K scale of tile
    // j+1, ks_nxt that of tile j+2 (loaded during iteration j).
    // Last valid local query of the work-group (uniform); positions grow with it.
    const int64_t a_end = (int64_t)(qt + 1) * BR;
    const int32_t a_max = (int32_t)((l < a_end ? l : a_end) - 1);
    auto act_of = [&](int32_t t) -> int32_t {
        if constexpr (!CAUSAL) return T;
        else return cmap.active_tiles(ring_block(a.rank, t, N), a_max, BC, T);
    };
    int32_t n_tiles = T * N;
    if constexpr (CAUSAL) {
        n_tiles = 0;
        for (int32_t t = 0; t < N; ++t) n_tiles += act_of(t);
    }
    // The member's own block comes first and its first tile is always visited (every
    // query sees its own block's first key), so each row's reference is finite from then.
    const int32_t act0 = act_of(0);
    Cursor cK{0, 0, act0}, cV{0, 0, act0}, cM{0, 0, act0}, cS{0, 0, act0};
    load_k(cK, Ks0);
    cK.next(act_of, N);
    load_v(cV, Vs0);
    cV.next(act_of, N);
    float ks_cur = load_scale(cS);
    cS.next(act_of, N);
    float ks_nxt = 1.f;
    if (n_tiles > 1) {
        load_k(cK, Ks1);
        cK.next(act_of, N);
        ks_nxt = load_scale(cS);
        cS.next(act_of, N);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();

    Scores sx, sy;
    i32x8 pb[2];
    {
        scores(Ks0, sx);
        mask_scores(sx, cM);
        cM.next(act_of, N);
        const float ct = tile_scale(ks_cur);
        bool changed;
        const float alpha = update_reference(row_max(sx), ct, changed);
        (void)alpha;  // nothing accumulated yet
#pragma unroll
        for (int q4 = 0; q4 < 8; ++q4) softmax_dw(sx, pb[0], q4, ct);
        if (n_tiles > 1) scores(Ks1, sy);
        ks_cur = ks_nxt;
    }
    __syncthreads();  // every wave is done with K buffer 0
    if (n_tiles > 2) {
        load_k(cK, Ks0);
        cK.next(act_of, N);
        ks_nxt = load_scale(cS);
        cS.next(act_of, N);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

    // Iteration j (j + 2 < n_tiles): cs = S(j+1), ns receives S(j+2) from kcur; P(j) in
    // pcur is multiplied by V(j) from vcur; P(j+1) goes to pnxt.
    auto full_iteration = [&](int32_t j, Scores &cs, Scores &ns, const uint8_t *kcur,
                              uint8_t *knext, const uint8_t *vcur, uint8_t *vnext,
                              const i32x8 &pcur, i32x8 &pnxt) {
        const bool more = j + 3 < n_tiles;
        if (more) load_k(cK, knext);
        load_v(cV, vnext);
        cV.next(act_of, N);
        float ks_new = 1.f;
        if (more) {
            cK.next(act_of, N);
            ks_new = load_scale(cS);
            cS.next(act_of, N);
        }
        mask_scores(cs, cM);
        cM.next(act_of, N);
        const float ct = tile_scale(ks_cur);
        bool changed;
        const float alpha = update_reference(row_max(cs), ct, changed);
        // Stage st: one score product of tile j+2, one P V product of tile j and an
        // equal share of the softmax of tile j+1 (independent work side by side).
        const int kb0 = laundered(kbase), vb = laundered(vbase);
        // The K and V^T fragments of stage st + 1 are read during stage st.
        i32x8 kfr = k_frag(kcur, kb0, 0), vfr = v_frag(vcur, vb, 0);
#pragma unroll
        for (int st = 0; st < NDT; ++st) {
            i32x8 kn = kfr, vn = vfr;
            if (st + 1 < NDT) {
                kn = k_frag(kcur, kb0, st + 1);
                vn = v_frag(vcur, vb, st + 1);
            }
            if (st % NKK == 0) ns.h[st / NKK] = f32x16{};
            ns.h[st / NKK] = mfma8(kfr, qf[st % NKK], ns.h[st / NKK]);
            o[st] = mfma8(vfr, pcur, o[st]);
#pragma unroll
            for (int q = 0; q < 8 / NDT; ++q) {
                softmax_dw(cs, pnxt, st * (8 / NDT) + q, ct);
                // keep this stage's exponentials here, beside its products (otherwise the
                // compiler sinks them towards their first use in the next iteration)
                asm volatile("" :: "v"(pnxt[st * (8 / NDT) + q]));
            }
            __builtin_amdgcn_sched_barrier(0);  // bound operand prefetch
            kfr = kn;
            vfr = vn;
        }
        sum_mfma(pcur);
        if (changed) rescale(alpha);  // after the products under the old reference
        ks_cur = ks_nxt;
        ks_nxt = ks_new;
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };
    // Iteration j = n_tiles - 2: no further scores.
    auto tail_iteration = [&](Scores &cs, const uint8_t *vcur, uint8_t *vnext, const i32x8 &pcur,
                              i32x8 &pnxt) {
        load_v(cV, vnext);
        cV.next(act_of, N);
        mask_scores(cs, cM);
        cM.next(act_of, N);
        const float ct = tile_scale(ks_cur);
        bool changed;
        const float alpha = update_reference(row_max(cs), ct, changed);
        const int vb = laundered(vbase);
#pragma unroll
        for (int st = 0; st < NDT; ++st) {
            pv_mfma(vcur, vb, pcur, st);
#pragma unroll
            for (int q = 0; q < 8 / NDT; ++q) softmax_dw(cs, pnxt, st * (8 / NDT) + q, ct);
            __builtin_amdgcn_sched_barrier(0);
        }
        sum_mfma(pcur);
        if (changed) rescale(alpha);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    };

    int32_t j = 0;
    for (; j + 3 < n_tiles; j += 2) {
        full_iteration(j, sy, sx, Ks0, Ks1, Vs0, Vs1, pb[0], pb[1]);
        full_iteration(j + 1, sx, sy, Ks1, Ks0, Vs1, Vs0, pb[1], pb[0]);
    }
    if (j + 2 < n_tiles) {  // j even
        full_iteration(j, sy, sx, Ks0, Ks1, Vs0, Vs1, pb[0], pb[1]);
        ++j;
    }
    // The last one or two tiles; every branch names its buffers statically.
    if (j + 1 < n_tiles) {
        if (j & 1) {
            tail_iteration(sx, Vs1, Vs0, pb[1], pb[0]);
            pv(Vs0, pb[0]);
        } else {
            tail_iteration(sy, Vs0, Vs1, pb[0], pb[1]);
            pv(Vs1, pb[1]);
        }
    } else if (j & 1) {
        pv(Vs1, pb[1]);
    } else {
        pv(Vs0, pb[0]);
    }

    if (!qvalid) return;
    const float ltot = lacc[0];  // every row of the ones product holds the row sum
    const int ooff = qloc * D + 4 * hf;
    const float *vs = a.vs + kvh * D + 4 * hf;
    float *op = a.O + row_base * D + ooff;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            // o[dt][4 i4 + e]: head-dim index 32 dt + 8 i4 + 4 hf + e
            const f32x4 sc = *(const f32x4 *)(vs + 32 * dt + 8 * i4);
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = o[dt][4 * i4 + e] * sc[e] / ltot;
            *(f32x4 *)(op + 32 * dt + 8 * i4) = v;
            if (a.O_cast) {
                bf16x4 cv = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
                *(bf16x4 *)((bf16 *)a.O_cast + row_base * D + ooff + 32 * dt + 8 * i4) = cv;
            }
        }
    if (hf == 0) {
        if (a.m) a.m[row_base + qloc] = m_nat;
        if (a.l) a.l[row_base + qloc] = ltot * __builtin_amdgcn_exp2f(Rp - m_nat * kLog2e);
    }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8Args &a, hipStream_t st) {
    hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(a.n_wg), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace

int fp8_query_tile() { return BR; }

hipError_t launch_fwd_fp8(const Fp8Args &a, int d, hipStream_t st) {
    const bool causal = a.layout != kNoCausal;
    if (d == 128) return causal ? launch<128, true>(a, st) : launch<128, false>(a, st);
    if (d == 64) return causal ? launch<64, true>(a, st) : launch<64, false>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace ra
