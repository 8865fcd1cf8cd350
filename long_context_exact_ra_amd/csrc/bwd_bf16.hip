// bwd_bf16.hip -- gradients of one ring member's attention share, bf16 inputs, gfx950
// matrix cores, fp32 accumulation.
//
// The backward pass recomputes the scores from the stored softmax statistics instead of
// keeping the attention matrix (aliyun FlashAttention explainer, section 2: recompute in
// the backward pass from O and the logsumexp).  With lse = m + ln l from the forward
// pass, per query row r and key k of the share:
//   P[r,k]  = exp(scale * q_r . k_k - lse_r)
//   dP[r,k] = dO_r . v_k
//   dS[r,k] = P[r,k] * (dP[r,k] - D_r),   D_r = dO_r . O_r   (= sum_k P dP)
//   dQ_r = scale * sum_k dS[r,k] k_k,  dK_k += scale * sum_r dS[r,k] q_r,
//   dV_k += sum_r P[r,k] dO_r.
// Two kernels avoid atomics: bwd_dq_kernel owns query rows and walks every key tile;
// bwd_dkdv_kernel owns key rows and walks every query tile of every query head that
// shares the K/V head.  bwd_prep_kernel first turns (O, dO, m, l) into (D, lse2) per
// row, lse2 = lse * log2(e), so probabilities are exp2(s * scale * log2(e) - lse2).
//
// MI355X mapping (both kernels share it, with the roles of queries and keys exchanged):
//  * The operand that stays put (Q and dO for dQ; K and V for dK / dV) is held in
//    VGPRs as the B operand of v_mfma_f32_32x32x16_bf16, 32 rows per wave.
//  * The streamed pair (K, V tiles; or Q, dO tiles) goes HBM -> LDS by buffer loads with
//    the LDS bit and is read twice: row-wise (16-byte reads) as the A operand of the
//    score-like products, and transposed (ds_read_b64_tr_b16) as the A operand of the
//    gradient products.  One XOR swizzle of 16-byte chunks keeps both read patterns free
//    of bank conflicts (see swz).
//  * Products are computed transposed so that one lane holds one owned row: the
//    elementwise P / dS work is in-lane, and the bf16-packed P and dS are directly the B
//    operands of the gradient products (the key / query order inside each 16-deep
//    contraction is permuted to match, as in the forward kernel).
//  * dK/dV splits each 32-key group between two waves of one SIMD: a producer (K, V
//    resident; score products and exponentials) and a consumer (dK, dV accumulators;
//    gradient products), with P and dS handed over through LDS once per query tile.
//    Each wave then fits in half the register file, and the SIMD holds a wave of matrix
//    products beside a wave of vector work.
//
// Causal shares (one K/V block per ring member, token positions from the layout): the
// dQ kernel walks only the key tiles of each block that some query of its tile may
// attend to (a prefix of the block); the dK/dV kernel walks only the query tiles from the
// first one holding a query at or after its first key (a suffix).  Excluded pairs (and
// rows past a block's end) get score -inf on the few tiles that hold any, by a per-lane
// limit, so ordinary tiles pay nothing for masking.  Work-groups with the most work are
// dispatched first.
#include <type_traits>

#include "causal_map.h"
#include "ra_internal.h"

namespace ra {
namespace {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit format; reads past the end give 0

__device__ __forceinline__ int xcd_remap(int wg, int n) {
    const int per = n / 8, rem = n % 8;
    const int xcd = wg % 8, slot = wg / 8;
    return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

template <int V>
using IC = std::integral_constant<int, V>;

// Buffer B of a tile ring held as separate __shared__ arrays.  The compiler separates
// the direct-to-LDS tile loads into one buffer from the reads of another only when the
// two are distinct __shared__ objects named at compile time; otherwise it waits for the
// loads (vmcnt) before every LDS read that follows them.
template <int B, typename T>
__device__ __forceinline__ T *pick(T *b0, T *b1, T *b2 = nullptr) {
    if constexpr (B == 0) return b0;
    else if constexpr (B == 1) return b1;
    else return b2;
}

__device__ __forceinline__ bf16x4 tr_read(const bf16 *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (bf16x4 __attribute__((address_space(3))) *)(p));
}

// Chunk swizzle of a streamed tile: the 16-byte chunk c of row r sits at c ^ swz(r).
// Row reads fetch one chunk of 16 consecutive rows (must hit 16 distinct 16-byte slots
// of a 256-byte window); transposed reads fetch one 64-byte quad of 4 consecutive rows
// (must hit 4 distinct quads).  d = 128 (256-byte rows): swz = 4*(r&3) | ((r>>2)&3)
// moves each row's quads by r&3 and its chunks within a quad by (r>>2)&3.  d = 64
// (two rows per window): swz = 4*((r>>1)&1) | ((r>>2)&3).
template <int D>
__device__ __forceinline__ int swz(int r) {
    return D == 128 ? (4 * (r & 3) | ((r >> 2) & 3)) : (4 * ((r >> 1) & 1) | ((r >> 2) & 3));
}

// Element offset of the 16-byte row read (row ln [+32 b], chunk 2 kk + hf) is
// rbase ^ (16 kk) [+ 32 b D]: the kk bits are disjoint from the row and half bits.
template <int D>
__device__ __forceinline__ int row_base(int ln, int hf) {
    const int f = swz<D>(ln);
    return ln * D + 8 * (hf ^ (f & 1)) + 16 * (f >> 1);
}

// Element offsets of the transposed reads.  Lane (g16, i16) of a 16-lane group reads
// rows 16 c4 + vrow (lo) and 16 c4 + vrow + 8 (hi), vrow = 4 hf + i16/4, columns
// 32 dt + 8 x + 4 (i16 & 1) with x = 2 (g16 & 1) + (i16 & 3) / 2; the swizzle of both
// rows is independent of c4, and dt enters as ^ (32 dt).
template <int D>
__device__ __forceinline__ int tr_base(int lane, int hi) {
    const int hf = lane >> 5, g16 = lane >> 4, i16 = lane & 15;
    const int r = 4 * hf + (i16 >> 2) + 8 * hi;
    const int f = swz<D>(r);
    const int x = 2 * (g16 & 1) + ((i16 & 3) >> 1);
    return r * D + 32 * (f >> 2) + 8 * (x ^ (f & 3)) + 4 * (i16 & 1);
}

// Direct global -> LDS loads of a tile of `rows` rows (of d bf16) starting at byte
// offset soff of buffer resource rs, by the first `nw` waves of the work-group.  Load p
// of wave w fills tile rows p*ROUND + w*RPL + lane/CPR; rows at or past `valid` repeat
// row valid-1 (their products are masked by the caller).
template <int D, int ROWS, int NWL>
struct TileLoad {
    static constexpr int CPR = D / 8;
    static constexpr int RPL = 64 / CPR;
    static constexpr int WAVE_LOADS = ROWS * CPR / 64;
    static constexpr int LOADERS = WAVE_LOADS < NWL ? WAVE_LOADS : NWL;
    static constexpr int ROUND = RPL * LOADERS;
    static constexpr int LOADS = ROWS / ROUND;
    static_assert(LOADS >= 1 && ROWS % ROUND == 0 && LOADS * LOADERS == WAVE_LOADS, "split");

    __device__ __forceinline__ static void run(__amdgpu_buffer_rsrc_t rs, uint32_t soff,
                                               int valid, bf16 *dst, int wave, int lane) {
        if (wave >= LOADERS) return;
        const int lr = wave * RPL + lane / CPR;
        const int slot = (lane % CPR) ^ swz<D>(lr);  // rows p*ROUND + lr share it (ROUND >= 16)
        bf16 *ldst = dst + wave * RPL * D;
#pragma unroll
        for (int p = 0; p < LOADS; ++p) {
            const int r = p * ROUND + lr;
            const int rr = r < valid ? r : valid - 1;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (void __attribute__((address_space(3))) *)(ldst + p * ROUND * D), 16,
                (int)((rr * D + slot * 8) * 2), (int)soff, 0, 0);
        }
    }
};

// ------------------------------------------------------------------ prep

// D = dO . O and lse2 = (m + ln l) * log2(e) = m log2(e) + log2(l), per row.
// 16 lanes per row, d / 16 elements each.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const float *O, const bf16 *dO,
                                                       const float *m, const float *l,
                                                       f32x2 *ws, int64_t rows) {
    constexpr int PER = D / 16;
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
    const int part = threadIdx.x & 15;
    float s = 0.f;
    if (row < rows) {
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int64_t i = row * D + part * PER + e;
            s = __builtin_fmaf((float)dO[i], O[i], s);
        }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) s += __shfl_xor(s, off);
    if (row < rows && part == 0)
        ws[row] = f32x2{s, m[row] * kLog2e + __builtin_amdgcn_logf(l[row])};
}

// ------------------------------------------------------------------ dQ

constexpr int QW = 8;         // waves per dQ work-group, 32 query rows each
constexpr int QBR = 32 * QW;  // query rows per dQ work-group
constexpr int KBC = 64;       // keys per streamed K/V tile

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * QW) void bwd_dq_kernel(BwdArgs a) {
    constexpr int NKK = D / 16, NDT = D / 32, TILE = KBC * D;
    using TL = TileLoad<D, KBC, QW>;
    __shared__ __attribute__((aligned(1024))) bf16 Kt0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Kt1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Vt0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Vt1[TILE];
    auto Kt = [&](auto b) { return pick<decltype(b)::value>(Kt0, Kt1); };
    auto Vt = [&](auto b) { return pick<decltype(b)::value>(Vt0, Vt1); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hf = lane >> 5, ln = lane & 31;
    const int wg = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, a.n_wg));
    // Causal: the last query tiles of a head see the most keys; they go first.
    const int qt = __builtin_amdgcn_readfirstlane(
        CAUSAL ? a.n_qtiles - 1 - wg % a.n_qtiles : wg % a.n_qtiles);
    const int bh = __builtin_amdgcn_readfirstlane(wg / a.n_qtiles);
    const int h = __builtin_amdgcn_readfirstlane(bh % a.H);
    const int b = __builtin_amdgcn_readfirstlane(bh / a.H);
    const int g = __builtin_amdgcn_readfirstlane(h / a.group);

    const int64_t rowb = (int64_t)bh * a.l_q + (int64_t)qt * QBR;  // first row of the tile
    const int qloc = wave * 32 + ln;
    const bool qvalid = (int64_t)qt * QBR + qloc < a.l_q;

    // Resident B operands: Q and dO rows (lane ln, head-dim chunk 16 kk + 8 hf).
    bf16x8 qf[NKK], dof[NKK];
    {
        const int64_t off = (rowb + qloc) * D + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            qf[kk] = qvalid ? *(const bf16x8 *)((const bf16 *)a.Q + off + 16 * kk) : bf16x8{};
            dof[kk] = qvalid ? *(const bf16x8 *)((const bf16 *)a.dO + off + 16 * kk) : bf16x8{};
        }
    }
    float Dr = 0.f, lse2 = 0.f;
    if (qvalid) {
        const f32x2 w = ((const f32x2 *)a.ws)[rowb + qloc];
        Dr = w[0];
        lse2 = w[1];
    }
    f32x16 dq[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        dq[dt] = f32x16{};
        asm volatile("" : "+v"(dq[dt]));
    }

    const int head_bytes = (int)(a.L * D * 2);  // host: < 2^31
    const bf16 *Kh = (const bf16 *)a.K + b * a.kv_batch_stride + g * a.kv_head_stride;
    const bf16 *Vh = (const bf16 *)a.V + b * a.kv_batch_stride + g * a.kv_head_stride;
    const __amdgpu_buffer_rsrc_t krs =
        __builtin_amdgcn_make_buffer_rsrc((void *)Kh, 0, head_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)Vh, 0, head_bytes, kRsrcWord3);
    // Key tiles: tile tin of block j holds keys j*kblk + tin*KBC ... (never two blocks).
    const int32_t kblk = (int32_t)a.kblk_rows;  // host: a head's rows fit in int32
    const int32_t tiles_per_blk = (kblk + KBC - 1) / KBC;
    const CausalMap cmap{a.layout, a.rank, a.n_kblocks, kblk};
    const int32_t a_end = (int32_t)(a.l_q < (int64_t)(qt + 1) * QBR ? a.l_q : (qt + 1) * QBR);
    auto act_of = [&](int32_t j) -> int32_t {  // active tiles of block j (a prefix)
        if constexpr (!CAUSAL) return tiles_per_blk;
        else return cmap.active_tiles(j, a_end - 1, KBC, tiles_per_blk);
    };
    int32_t n_tiles = tiles_per_blk * a.n_kblocks;
    if constexpr (CAUSAL) {
        n_tiles = 0;
        for (int32_t j = 0; j < a.n_kblocks; ++j) n_tiles += act_of(j);
    }
    struct Cursor {
        int32_t j, tin, act;
    };
    auto advance = [&](Cursor &cu) {
        if (++cu.tin < cu.act) return;
        cu.tin = 0;
        do {
            ++cu.j;
        } while (cu.j < a.n_kblocks && (cu.act = act_of(cu.j)) == 0);
    };
    auto tile_rows = [&](const Cursor &cu) {
        const int32_t left = kblk - cu.tin * KBC;
        return left < KBC ? left : KBC;
    };
    auto load = [&](const Cursor &cu, auto buf) {
        const int64_t r0 = (int64_t)cu.j * kblk + (int64_t)cu.tin * KBC;
        const uint32_t soff = (uint32_t)(r0 * D * 2);
        TL::run(krs, soff, tile_rows(cu), Kt(buf), wave, lane);
        TL::run(vrs, soff, tile_rows(cu), Vt(buf), wave, lane);
    };

    const int rb = row_base<D>(ln, hf);
    const int tb_lo = tr_base<D>(lane, 0), tb_hi = tr_base<D>(lane, 1);
    const float c = a.scale_log2;

    const int32_t qa = qt * QBR + qloc;  // this lane's local query
    Cursor lc{-1, 0, 0}, cc;             // next tile to load; tile being computed
    advance(lc);
    cc = lc;
    if (n_tiles > 0) {
        load(lc, IC<0>{});
        advance(lc);
    }
    // Tile t in buffer t & 1, fixed at compile time (the loop is unrolled by two).
    auto step = [&](auto buf, int32_t t) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t landed (this wave's part)
        __syncthreads();                     // ... everyone's part; tile t-1 fully read
        if (t + 1 < n_tiles) {
            load(lc, IC<1 - decltype(buf)::value>{});
            advance(lc);
        }
        const bf16 *kt = Kt(buf), *vt = Vt(buf);

        // S^T = K Q^T and dP^T = V dO^T: lane = query ln, 16 keys per 32-key block.
        f32x16 s[2], dp[2];
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
            s[k2] = f32x16{};
            dp[k2] = f32x16{};
        }
        int kb = rb;
        asm volatile("" : "+v"(kb));
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int off = (kb ^ (16 * kk)) + 32 * k2 * D;
                const bf16x8 kf = *(const bf16x8 *)(kt + off);
                const bf16x8 vf = *(const bf16x8 *)(vt + off);
                s[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[k2], 0, 0, 0);
                dp[k2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[kk], dp[k2], 0, 0, 0);
            }
        }
        // dS = P (dP - D), P = exp2(s c - lse2); keys past the end of the block (and,
        // causal, keys after this lane's query) get P = 0.  Packed in the contraction
        // order of the dQ product: operand c4 holds keys 16 c4 + 8 (j/4) + 4 hf + j%4,
        // i.e. elements 8 (c4%2) + j of block c4/2.
        int keys = tile_rows(cc);
        if constexpr (CAUSAL) {
            const int allow = cmap.allowed(qa, cc.j, cc.tin * KBC);
            keys = allow < keys ? (allow > 0 ? allow : 0) : keys;
        }
        advance(cc);
        // Excluded keys get score -inf (so P = 0), on the rare tiles that have any: the
        // empty volatile asm keeps this a branch rather than selects on every tile.
        if (__builtin_amdgcn_ballot_w64(keys < KBC) != 0) {
            asm volatile("" ::: "memory");
            const int lim = keys - 4 * hf;
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                for (int i = 0; i < 16; ++i)  // key 32 k2 + 8 (i/4) + 4 hf + i%4
                    if (32 * k2 + 8 * (i >> 2) + (i & 3) >= lim) s[k2][i] = -INFINITY;
        }
        bf16x8 dsp[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = 8 * (c4 & 1) + j;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[c4 >> 1][i], c, -lse2));
                dsp[c4][j] = (bf16)(p * (dp[c4 >> 1][i] - Dr));
            }
        // dQ^T += K^T dS^T: A = K^T (transposed reads, rows = keys of the contraction).
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x4 lo = tr_read(kt + (tb_lo ^ (32 * dt)) + 16 * c4 * D);
                const bf16x4 hi = tr_read(kt + (tb_hi ^ (32 * dt)) + 16 * c4 * D);
                const bf16x8 ka = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, dsp[c4], dq[dt], 0, 0, 0);
            }
    };
    for (int32_t t = 0; t < n_tiles; t += 2) {
        step(IC<0>{}, t);
        if (t + 1 >= n_tiles) break;
        step(IC<1>{}, t + 1);
    }

    if (!qvalid) return;
    // dq[dt][4 i4 + e]: head-dim 32 dt + 8 i4 + 4 hf + e of this lane's query row.
    float *op = a.dQ + (rowb + qloc) * D + 4 * hf;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
            *(f32x4 *)(op + 32 * dt + 8 * i4) =
                f32x4{dq[dt][4 * i4] * a.scale, dq[dt][4 * i4 + 1] * a.scale,
                      dq[dt][4 * i4 + 2] * a.scale, dq[dt][4 * i4 + 3] * a.scale};
}

// ------------------------------------------------------------------ dK, dV

constexpr int KW = 4;          // key groups per dK/dV work-group, 32 keys each
constexpr int KBR = 32 * KW;   // key rows per work-group
constexpr int QBC = 64;        // query rows per streamed Q / dO tile
constexpr int KWAVES = 2 * KW; // dK/dV waves: producers 0 .. KW-1, consumers KW .. 2 KW-1
constexpr int kReadAhead = 3;  // dK/dV: fragment reads this many product steps ahead

// Causal: key tile i of a (batch, kv head) in order of its first key's position (the
// earliest keys are seen by the most queries, so they go first).  Zigzag lists the first
// halves of the blocks, then the second halves from the last block down.
__device__ __forceinline__ void key_tile_of(int32_t i, int32_t layout, int32_t N, int32_t kpb,
                                            int32_t &j, int32_t &u) {
    if (layout == kLayoutContiguous) {
        j = i / kpb;
        u = i - j * kpb;
    } else if (layout == kLayoutStriped) {
        u = i / N;
        j = i - u * N;
    } else {
        const int32_t ka = (kpb + 1) / 2, kb = kpb - ka;
        if (i < N * ka) {
            j = i / ka;
            u = i - j * ka;
        } else {
            const int32_t r = i - N * ka, jj = r / kb;
            j = N - 1 - jj;
            u = ka + (r - jj * kb);
        }
    }
}

// The dK/dV work of a key group is split between two waves on one SIMD.  The producer
// holds the group's K and V rows and turns each query tile into P and dS (score
// products, exponentials); the consumer holds the dK and dV accumulators and runs the
// gradient products.  P and dS pass through LDS, one tile per barrier pair: while the
// consumer works on tile t the producer computes tile t+1, so the SIMD has a wave of
// matrix products beside the wave of vector work.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * KWAVES) void bwd_dkdv_kernel(BwdArgs a) {
    constexpr int NKK = D / 16, NDT = D / 32, TILE = QBC * D;
    using TL = TileLoad<D, QBC, KWAVES>;
    // Three Q / dO tile buffers: tile t is read by the gradient products while tile t+1 is
    // read by the score products and tile t+2 is being loaded.
    __shared__ __attribute__((aligned(1024))) bf16 Qt0[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Qt1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Qt2[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Ot0[TILE];  // dO tiles
    __shared__ __attribute__((aligned(1024))) bf16 Ot1[TILE];
    __shared__ __attribute__((aligned(1024))) bf16 Ot2[TILE];
    __shared__ __attribute__((aligned(16))) f32x2 Wt0[QBC];    // (D, lse2) of the rows
    __shared__ __attribute__((aligned(16))) f32x2 Wt1[QBC];
    __shared__ __attribute__((aligned(16))) f32x2 Wt2[QBC];
    // P and dS of one tile: per key group 8 operands (P, then dS, for c4 = 0..3) of 16
    // bytes per lane, lane-contiguous.
    __shared__ __attribute__((aligned(1024))) bf16x8 Xs[KW * 8 * 64];
    auto Qt = [&](auto b) { return pick<decltype(b)::value>(Qt0, Qt1, Qt2); };
    auto Ot = [&](auto b) { return pick<decltype(b)::value>(Ot0, Ot1, Ot2); };
    auto Wt = [&](auto b) { return pick<decltype(b)::value>(Wt0, Wt1, Wt2); };

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave < KW;
    const int kg = producer ? wave : wave - KW;  // key group (uniform)
    const int hf = lane >> 5, ln = lane & 31;
    const int wg = __builtin_amdgcn_readfirstlane(xcd_remap(blockIdx.x, a.n_wg));
    const int kt_i = __builtin_amdgcn_readfirstlane(wg % a.n_ktiles);
    const int bg = __builtin_amdgcn_readfirstlane(wg / a.n_ktiles);
    const int g = __builtin_amdgcn_readfirstlane(bg % a.H_kv);
    const int b = __builtin_amdgcn_readfirstlane(bg / a.H_kv);

    // Key tile kt_i is tile u of key block j; this lane's key is local key bl of block j.
    int32_t j = 0, u = kt_i;
    if constexpr (CAUSAL) key_tile_of(kt_i, a.layout, a.n_kblocks, a.n_ktiles_blk, j, u);
    j = __builtin_amdgcn_readfirstlane(j);
    u = __builtin_amdgcn_readfirstlane(u);
    const int32_t kblk = (int32_t)a.kblk_rows;
    const int32_t bl = u * KBR + kg * 32 + ln;
    const int64_t key = (int64_t)j * kblk + bl;  // this lane's key row
    const bool kvalid = bl < kblk;
    const int64_t kvoff = b * a.kv_batch_stride + g * a.kv_head_stride;

    const int head_bytes = (int)(a.l_q * D * 2);
    const int32_t tiles_per_head = (int32_t)((a.l_q + QBC - 1) / QBC);
    // Causal: only queries at or after a key's position see it; query tiles from s_min on
    // hold all the queries that see a key of this work-group; fq is the first query that
    // sees this lane's key (positions grow with the local index in every layout).
    const CausalMap cmap{a.layout, a.rank, a.n_kblocks, kblk};
    int32_t s_min = 0, fq = 0, fq_wave = 0;  // fq_wave: the largest fq of the key group
    if constexpr (CAUSAL) {
        const int32_t last = kblk - 1, wlast = u * KBR + kg * 32 + 31;
        s_min = __builtin_amdgcn_readfirstlane(cmap.first_query(cmap.pos(j, u * KBR)) / QBC);
        fq = cmap.first_query(cmap.pos(j, bl < last ? bl : last));
        fq_wave = __builtin_amdgcn_readfirstlane(
            cmap.first_query(cmap.pos(j, wlast < last ? wlast : last)));
    }
    const int32_t act_per_head = tiles_per_head - s_min;
    const int32_t n_tiles = act_per_head * a.group;
    if (n_tiles == 0) return;  // no query of this share sees these keys (uniform)
    // Tile t: query head g*group + t / act_per_head, rows (s_min + t % act_per_head) * QBC
    auto tile_of = [&](int32_t t, int32_t &hh) {
        hh = t / act_per_head;
        return s_min + (t - hh * act_per_head);
    };
    auto load = [&](int32_t t, auto buf) {
        int32_t hh;
        const int32_t s = tile_of(t, hh);
        const int64_t bh = (int64_t)b * a.H + (int64_t)g * a.group + hh;
        const int64_t r0 = (int64_t)s * QBC;
        const int64_t left = a.l_q - r0;
        const int valid = left < QBC ? (int)left : QBC;
        const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const bf16 *)a.Q + bh * a.l_q * D), 0, head_bytes, kRsrcWord3);
        const __amdgpu_buffer_rsrc_t ors = __builtin_amdgcn_make_buffer_rsrc(
            (void *)((const bf16 *)a.dO + bh * a.l_q * D), 0, head_bytes, kRsrcWord3);
        const uint32_t soff = (uint32_t)(r0 * D * 2);
        TL::run(qrs, soff, valid, Qt(buf), wave, lane);
        TL::run(ors, soff, valid, Ot(buf), wave, lane);
        if (wave == KWAVES - 1 && lane < QBC / 2) {  // 64 (D, lse2) pairs = 512 bytes
            const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)((const f32x2 *)a.ws + bh * a.l_q), 0, (int)(a.l_q * 8), kRsrcWord3);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wrs, (void __attribute__((address_space(3))) *)(Wt(buf)), 16, lane * 16,
                (int)(r0 * 8), 0, 0);
        }
    };
    bf16x8 *xs = Xs + kg * 8 * 64 + lane;  // operand v of this lane at xs[64 v]
    // Fragment reads run kReadAhead steps ahead of their products.  The fences keep the
    // reads and the products in this order and let vector and scalar work move across.
    auto fence = [] { __builtin_amdgcn_sched_barrier(0x0406); };

    load(0, IC<0>{});
    if (n_tiles > 1) load(1, IC<1>{});
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();

    if (producer) {
        // Resident B operands: K and V rows of this lane's key.
        bf16x8 kf[NKK], vf[NKK];
        {
            const int64_t off = kvoff + key * D + 8 * hf;
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) {
                kf[kk] = kvalid ? *(const bf16x8 *)((const bf16 *)a.K + off + 16 * kk) : bf16x8{};
                vf[kk] = kvalid ? *(const bf16x8 *)((const bf16 *)a.V + off + 16 * kk) : bf16x8{};
            }
        }
        const int rb = row_base<D>(ln, hf);
        const float c = a.scale_log2;
        // S = Q K^T and dP = dO V^T of the tile in buffer `buf`: lane = key ln, 16 queries
        // per 32-query block, element i of block qb = query 32 qb + 8 (i/4) + 4 hf + i%4.
        auto scores = [&](auto buf, f32x16 *sc, f32x16 *dq) {
            const bf16 *qt = Qt(buf), *ot = Ot(buf);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                sc[qb] = f32x16{};
                dq[qb] = f32x16{};
            }
            int kb = rb;
            asm volatile("" : "+v"(kb));
            constexpr int NS = 2 * NKK;  // steps (kk, qb)
            bf16x8 qa[NS], oa[NS];
            auto rd = [&](int st) {
                const int kk = st / 2, qb = st % 2;
                const int off = (kb ^ (16 * kk)) + 32 * qb * D;
                qa[st] = *(const bf16x8 *)(qt + off);
                oa[st] = *(const bf16x8 *)(ot + off);
            };
            fence();
#pragma unroll
            for (int st = 0; st < kReadAhead; ++st) rd(st);
#pragma unroll
            for (int st = 0; st < NS; ++st) {
                fence();
                if (st + kReadAhead < NS) rd(st + kReadAhead);
                const int kk = st / 2, qb = st % 2;
                sc[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], kf[kk], sc[qb], 0, 0, 0);
                dq[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[st], vf[kk], dq[qb], 0, 0, 0);
            }
            fence();
        };
        // Excluded pairs (rows past the end of the block; causal, queries before this
        // lane's first query fq) get score -inf, so P = 0 and dS = 0.  Only tiles that
        // have any are touched, behind a wave-uniform branch kept real by an empty
        // volatile asm.
        auto mask_tile = [&](int32_t t, f32x16 *sc) {
            int32_t hh;
            const int32_t s_idx = tile_of(t, hh);
            const bool ragged = (int64_t)(s_idx + 1) * QBC > a.l_q;
            if (!(ragged || (CAUSAL && fq_wave > s_idx * QBC))) return;
            asm volatile("" ::: "memory");
            const int64_t left = a.l_q - (int64_t)s_idx * QBC;
            const int qlim = (left < QBC ? (int)left : QBC) - 4 * hf;  // valid query rows
            const int qthr = CAUSAL ? fq - s_idx * QBC - 4 * hf : -QBC;  // first seeing query
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int q = 32 * qb + 8 * (i >> 2) + (i & 3);  // query minus 4 hf
                    if (q >= qlim || q < qthr) sc[qb][i] = -INFINITY;
                }
        };
        // P and dS, packed in the contraction order of the gradient products (operand c4:
        // queries 16 c4 + 8 (j/4) + 4 hf + j%4 = elements 8 (c4%2) + j of block c4/2).
        auto softmax = [&](auto buf, const f32x16 *sc, const f32x16 *dq, bf16x8 *pp,
                           bf16x8 *dsp) {
            int wo = 4 * hf;
            asm volatile("" : "+v"(wo));
            const f32x2 *w = Wt(buf) + wo;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4)
#pragma unroll
                for (int j4 = 0; j4 < 2; ++j4) {
                    // queries q0 .. q0 + 3, q0 = 16 c4 + 8 j4 + 4 hf: two 16-byte LDS reads
                    const int q0 = 16 * c4 + 8 * j4;  // minus 4 hf
                    const f32x4 w01 = *(const f32x4 *)(w + q0);
                    const f32x4 w23 = *(const f32x4 *)(w + q0 + 2);
                    const float Dq[4] = {w01[0], w01[2], w23[0], w23[2]};
                    const float Lq[4] = {w01[1], w01[3], w23[1], w23[3]};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int jj = 4 * j4 + e, i = 8 * (c4 & 1) + jj;
                        const float p =
                            __builtin_amdgcn_exp2f(__builtin_fmaf(sc[c4 >> 1][i], c, -Lq[e]));
                        pp[c4][jj] = (bf16)p;
                        dsp[c4][jj] = (bf16)(p * (dq[c4 >> 1][i] - Dq[e]));
                    }
                }
        };
        f32x16 sc[2], dq[2];
        bf16x8 pp[4], dsp[4];
        scores(IC<0>{}, sc, dq);
        mask_tile(0, sc);
        softmax(IC<0>{}, sc, dq, pp, dsp);
        // Iteration t (tile t in buffer t % 3, fixed at compile time: the loop is unrolled
        // by three): publish P and dS of tile t, then compute those of tile t+1.
        auto iteration = [&](auto buf, int32_t t) {
            constexpr int bb = decltype(buf)::value;
            const IC<(bb + 1) % 3> nb;   // tile t + 1
            const IC<(bb + 2) % 3> nnb;  // tile t + 2 (held tile t - 1)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                xs[64 * v] = pp[v];
                xs[64 * (4 + v)] = dsp[v];
            }
            __syncthreads();  // P and dS of tile t published
            if (t + 2 < n_tiles) load(t + 2, nnb);
            if (t + 1 < n_tiles) {
                scores(nb, sc, dq);
                mask_tile(t + 1, sc);
                softmax(nb, sc, dq, pp, dsp);
            }
            __builtin_amdgcn_s_waitcnt(0x0F70);  // tile t + 2 landed (this wave's part)
            __syncthreads();                     // everyone's part; tile t fully read
        };
        for (int32_t t = 0;; t += 3) {
            iteration(IC<0>{}, t);
            if (t + 1 >= n_tiles) break;
            iteration(IC<1>{}, t + 1);
            if (t + 2 >= n_tiles) break;
            iteration(IC<2>{}, t + 2);
            if (t + 3 >= n_tiles) break;
        }
        return;
    }

    // Consumer.
    f32x16 dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
        dk[dt] = f32x16{};
        dv[dt] = f32x16{};
        asm volatile("" : "+v"(dk[dt]), "+v"(dv[dt]));
    }
    const int tb_lo0 = tr_base<D>(lane, 0), tb_hi0 = tr_base<D>(lane, 1);
    // dV^T += dO^T P and dK^T += Q^T dS: A = transposed reads of the dO / Q tiles.
    auto grads = [&](auto buf, const bf16x8 *pp, const bf16x8 *dsp) {
        const bf16 *qt = Qt(buf), *ot = Ot(buf);
        int tb_lo = tb_lo0, tb_hi = tb_hi0;  // derived where used, not kept live per buffer
        asm volatile("" : "+v"(tb_lo), "+v"(tb_hi));
        constexpr int NS = 4 * NDT;  // steps (c4, dt)
        bf16x8 oa[NS], qa[NS];
        auto rd = [&](int st) {
            const int c4 = st / NDT, dt = st % NDT;
            const int olo = (tb_lo ^ (32 * dt)) + 16 * c4 * D;
            const int ohi = (tb_hi ^ (32 * dt)) + 16 * c4 * D;
            const bf16x4 a0 = tr_read(ot + olo), a1 = tr_read(ot + ohi);
            const bf16x4 b0 = tr_read(qt + olo), b1 = tr_read(qt + ohi);
            oa[st] = bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            qa[st] = bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
        };
        fence();
#pragma unroll
        for (int st = 0; st < kReadAhead; ++st) rd(st);
#pragma unroll
        for (int st = 0; st < NS; ++st) {
            fence();
            if (st + kReadAhead < NS) rd(st + kReadAhead);
            const int c4 = st / NDT, dt = st % NDT;
            dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa[st], pp[c4], dv[dt], 0, 0, 0);
            dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[st], dsp[c4], dk[dt], 0, 0, 0);
        }
        fence();
    };
    auto iteration = [&](auto buf, int32_t t) {
        constexpr int bb = decltype(buf)::value;
        const IC<(bb + 2) % 3> nnb;  // tile t + 2 (held tile t - 1)
        __syncthreads();  // P and dS of tile t published
        if (t + 2 < n_tiles) load(t + 2, nnb);
        bf16x8 pp[4], dsp[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            pp[v] = xs[64 * v];
            dsp[v] = xs[64 * (4 + v)];
        }
        grads(buf, pp, dsp);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // tile t + 2 landed (this wave's part)
        __syncthreads();                     // everyone's part; tile t fully read
    };
    for (int32_t t = 0;; t += 3) {
        iteration(IC<0>{}, t);
        if (t + 1 >= n_tiles) break;
        iteration(IC<1>{}, t + 1);
        if (t + 2 >= n_tiles) break;
        iteration(IC<2>{}, t + 2);
        if (t + 3 >= n_tiles) break;
    }

    if (!kvalid) return;
    // dk[dt][4 i4 + e]: head-dim 32 dt + 8 i4 + 4 hf + e of this lane's key row; the
    // gradients are added to what the caller's buffers hold.
    const int64_t ro = kvoff + key * D + 4 * hf;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            f32x4 *pk = (f32x4 *)(a.dK + ro + 32 * dt + 8 * i4);
            f32x4 *pv = (f32x4 *)(a.dV + ro + 32 * dt + 8 * i4);
            f32x4 xk = *pk, xv = *pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xk[e] = __builtin_fmaf(dk[dt][4 * i4 + e], a.scale, xk[e]);
                xv[e] += dv[dt][4 * i4 + e];
            }
            *pk = xk;
            *pv = xv;
        }
}

template <int D, bool CAUSAL>
hipError_t launch_all(const BwdArgs &a, const float *O, const void *dO, const float *m,
                      const float *l, int64_t rows, hipStream_t st) {
    const int64_t prep_blocks = (rows * 16 + 255) / 256;
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)prep_blocks), dim3(256), 0, st, O,
                       (const bf16 *)dO, m, l, (f32x2 *)a.ws, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3(a.n_wg), dim3(64 * QW), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    BwdArgs k = a;
    k.n_wg = a.n_kv_wg;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3(k.n_wg), dim3(64 * KWAVES), 0, st, k);
    return hipGetLastError();
}

}  // namespace

int bwd_query_tile() { return QBR; }
int bwd_key_tile() { return KBR; }

hipError_t launch_bwd_bf16(const BwdArgs &a, const float *O, const void *dO, const float *m,
                           const float *l, int64_t rows, int d, hipStream_t st) {
    const bool causal = a.layout != kNoCausal;
    if (d == 128)
        return causal ? launch_all<128, true>(a, O, dO, m, l, rows, st)
                      : launch_all<128, false>(a, O, dO, m, l, rows, st);
    if (d == 64)
        return causal ? launch_all<64, true>(a, O, dO, m, l, rows, st)
                      : launch_all<64, false>(a, O, dO, m, l, rows, st);
    return hipErrorInvalidValue;
}

}  // namespace ra
