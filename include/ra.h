/*
 * ra.h -- C ABI of the ring-attention share library for AMD MI355X (gfx950).
 *
 * The method (slowleelab "Ring Attention" page, L3 definition and L4 section 4.2):
 * a sequence of L tokens is split into N equal blocks of l = L / N tokens; ring
 * member i keeps its query block Q_i resident and, at step t = 0 .. N-1, works on
 * the K/V block (i - t) mod N, which arrives from member i-1 and is passed on to
 * member i+1.  Each step is one blockwise, FlashAttention-style merge with online
 * softmax (same page, 4.3): a running row maximum m, a running sum l of
 * exp(s - m) and an unnormalised output O are rescaled and accumulated per block,
 * and O is divided by l once after the last block.  After the N steps, Q_i's
 * output is exact attention softmax(Q_i K^T / sqrt(d)) V over the whole sequence.
 * On one GPU the arrival of blocks over the ring is replaced by a rotating index
 * over K/V blocks that are already resident in device memory.
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers owned by the caller, in memory of the
 *    current HIP device (hipSetDevice), on which every call launches; the library
 *    allocates no device memory and keeps no state between calls, except a
 *    per-device record of whether the device is supported.
 *  - Layouts are row-major: Q_i and outputs O are [B, H, l_q, d]; K and V are
 *    [B, H_kv, rows, d]; m and l are fp32 [B, H, l_q]; O_acc is always fp32.
 *  - Grouped-query attention (lnwmold page, section 2.2): query head h reads K/V
 *    head h / (H / H_kv); H must be a multiple of H_kv.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *    compute call only enqueues work on that stream and returns; errors inside a
 *    kernel surface at the caller's next synchronisation.
 *  - Return value: RA_OK, or an ra_status code.  Arguments are validated before
 *    anything is enqueued, so an RA_EINVAL / RA_ENOTSUP return means no device
 *    memory was written.  Input VALUES are not checked: NaN and Inf propagate.
 *  - Supported: d in {64, 128}; dtype RA_F32 or RA_BF16; scale finite and > 0;
 *    device pointers 16-byte aligned.  Any N >= 1 is allowed (the slowleelab page,
 *    pitfall 6, notes the ring works for any GPU count).
 *  - With RA_BF16, one K (or V) head of the call, rows * d * 2 bytes, must stay
 *    below 2^31 bytes (the kernel addresses a head through a 32-bit buffer range);
 *    larger heads return RA_ENOTSUP.
 *  - Sizes whose tensors or grids the kernels cannot address (a byte size beyond
 *    int64, a grid beyond 2^31 - 1 work-groups) return RA_ENOTSUP; the checks
 *    saturate rather than overflow, so no argument value makes them wrap round.
 */
#ifndef RA_H
#define RA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ra_status {
    RA_OK = 0,
    RA_EINVAL = 1,  /* bad argument; nothing was enqueued */
    RA_ENOTSUP = 2, /* current device is not gfx950, or an unsupported size */
    RA_EHIP = 3,    /* a HIP runtime call failed; see ra_last_hip_error() */
    RA_ESCRATCH = 4 /* ra_share_backward_noalloc: the problem needs more than
                       RA_NOALLOC_SCRATCH_BYTES of workspace; nothing was enqueued */
} ra_status;

typedef enum ra_dtype {
    RA_F32 = 0,  /* fp32 Q/K/V; fp32 arithmetic throughout */
    RA_BF16 = 1  /* bf16 Q/K/V; bf16 matrix-core products, fp32 accumulation and statistics */
} ra_dtype;

/*
 * Shape of one step's operands.
 *   B, H, H_kv, d   batch, query heads, K/V heads, head dimension
 *   l_q             rows of the resident query block Q_i
 *   l_kv            rows (keys) of the K/V block merged by this step
 *   kv_head_stride  elements between consecutive K/V heads of K_blk / V_blk;
 *                   0 means l_kv * d (a contiguous [B, H_kv, l_kv, d] block, as
 *                   received over a ring); L * d addresses a block inside a full
 *                   [B, H_kv, L, d] tensor.  Must be a multiple of 8.
 *   kv_batch_stride elements between batches of K_blk / V_blk; 0 means
 *                   H_kv * kv_head_stride.  Must be a multiple of 8.
 *   dtype           an ra_dtype for Q_i, K_blk and V_blk
 */
typedef struct ra_shape {
    int32_t B, H, H_kv, d;
    int64_t l_q, l_kv;
    int64_t kv_head_stride, kv_batch_stride;
    int32_t dtype;
} ra_shape;

/*
 * K/V block that ring member `rank` uses at step t: (rank - t) mod N, always in
 * [0, N).  slowleelab page, L3 ("at step t GPU i receives K_(i-t)%N, V_(i-t)%N
 * from GPU i-1 ... then sends it to GPU i+1") and the N = 4 table in 4.2.
 * Host only.  Returns -RA_EINVAL if N < 1, rank outside [0, N) or t outside [0, N).
 */
int32_t ra_ring_block(int32_t rank, int32_t N, int32_t t);

/*
 * Fills host array out[0 .. N-1] with ra_ring_block(rank, N, t).  Host only.
 * Returns RA_EINVAL (and writes nothing) on bad rank / N or a NULL `out`.
 */
int ra_ring_schedule(int32_t rank, int32_t N, int32_t *out);

/*
 * K/V head read by query head h under grouped-query attention with contiguous
 * groups of H / H_kv heads (lnwmold page, sections 2.2 and 3.1).  Host only.
 * Returns -RA_EINVAL if H % H_kv != 0 or h is outside [0, H).
 */
int32_t ra_kv_head(int32_t h, int32_t H, int32_t H_kv);

/*
 * Initial running state before the first step: O_acc = 0, m = -inf, l = 0.
 * (The slowleelab page's step pseudocode, 4.3, leaves the initial state
 * unstated; this is the state for which merging one block gives that block's
 * own attention.)  O_acc is [B, H, l_q, d] fp32; m and l are [B, H, l_q] fp32.
 * Uses shape fields B, H, d, l_q.  l_q == 0 is a no-op.
 */
int ra_state_init(float *O_acc, float *m, float *l, const ra_shape *s, void *stream);

/*
 * One ring step: merges the K/V block (K_blk, V_blk) into the running state of
 * the resident block Q_i, in place (slowleelab page, 4.3, ring_attention_step):
 *     s      = scale * Q_i K_blk^T                (per query row, per key)
 *     m_new  = max(m, row max of s)
 *     l     <- exp(m - m_new) * l + row sum of exp(s - m_new)
 *     O_acc <- exp(m - m_new) * O_acc + exp(s - m_new) V_blk
 *     m     <- m_new
 * Division by l is NOT done here (it is the final rescale, ra_finalize).  After
 * the call, m is exactly the running row maximum of the fp32 scores seen so far.
 * Blocks may be merged in any order; the finalised result does not depend on it.
 * Q_i is [B, H, l_q, d] contiguous; K_blk / V_blk are [B, H_kv, l_kv, d] with the
 * strides in *s.  l_q == 0 or l_kv == 0 is a no-op.  scale is normally 1/sqrt(d).
 */
int ra_step(const void *Q_i, const void *K_blk, const void *V_blk, float *O_acc,
            float *m, float *l, float scale, const ra_shape *s, void *stream);

/*
 * Final rescale after the last step (slowleelab page, 4.3, "O_i / l_new"):
 * O_acc <- O_acc / l per row, in place.  If O_out is not NULL it also receives the
 * result in s->dtype (bf16 rounded to nearest even, or an fp32 copy).  Uses shape
 * fields B, H, d, l_q, dtype.  Defined only after at least one step (l > 0).
 */
int ra_finalize(float *O_acc, const float *l, const ra_shape *s, void *O_out, void *stream);

/*
 * The whole share of ring member `rank` in one launch: all N blocks of the
 * sequence, visited in the order ra_ring_schedule(rank, N), merged with online
 * softmax and finalised.
 *   L          sequence length; must be a multiple of N; l = L / N
 *   Q_i        [B, H, l, d] in `dtype`, the resident query block
 *   K, V       [B, H_kv, L, d] in `dtype`, the full sequence; block j is rows
 *              j*l .. (j+1)*l - 1
 *   O          [B, H, l, d] fp32, the finalised attention output (required)
 *   m_out      nullable [B, H, l] fp32: row maximum of the scaled scores
 *   l_out      nullable [B, H, l] fp32: sum over all keys of exp(s - m_out)
 *   O_cast     nullable [B, H, l, d] in `dtype` (bf16 rounded to nearest even)
 *   sched_trace nullable device int32[N]: the block index used at each step t
 * L == 0 is a no-op.
 */
int ra_share_forward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                     int32_t d, int32_t B, int32_t dtype, const void *Q_i, const void *K,
                     const void *V, float scale, float *O, float *m_out, float *l_out,
                     void *O_cast, int32_t *sched_trace, void *stream);

/*
 * How the tokens of the sequence are assigned to ring members, for the causal share.
 * Member r holds l = L / N tokens; its local token x sits at global position
 *   RA_LAYOUT_CONTIGUOUS  r*l + x                       (the plain split of the
 *                         sequence into N consecutive blocks, slowleelab page, L2)
 *   RA_LAYOUT_STRIPED     x*N + r                       (Striped Attention's
 *                         interleaved assignment, slowleelab page, 4.8)
 *   RA_LAYOUT_ZIGZAG      with h = l/2: r*h + x for x < h, (2N-1-r)*h + (x-h) after:
 *                         chunks r and 2N-1-r of 2N equal chunks (the zigzag ring
 *                         named in 4.5; this chunk pairing is the library's reading)
 */
typedef enum ra_layout {
    RA_LAYOUT_CONTIGUOUS = 0,
    RA_LAYOUT_STRIPED = 1,
    RA_LAYOUT_ZIGZAG = 2
} ra_layout;

/*
 * Causal share of ring member `rank` in one launch (slowleelab page, 4.5 limitation 2:
 * under causal attention a query may only attend to keys at or before its own
 * position).  Same computation as ra_share_forward except that a key enters a query's
 * softmax only if its global position (per `layout`) is <= the query's.  Q_i holds the
 * member's tokens in local order; K and V hold the whole sequence in member-major
 * order: rows j*l .. (j+1)*l - 1 are member j's tokens, local order.
 * Key tiles with no admissible key for any query of a work-group are skipped, so the
 * work follows the layout: growing with the rank for RA_LAYOUT_CONTIGUOUS (the 50 %
 * waste of 4.5), nearly equal across members for the striped and zigzag layouts.
 * Every query has at least one admissible key (itself), so the output is defined.
 *   layout   an ra_layout; RA_LAYOUT_ZIGZAG needs l to be a multiple of 128 (each
 *            half-block a whole number of 64-key tiles), else RA_EINVAL
 *   O, m_out, l_out, O_cast as in ra_share_forward (m and l over admissible keys).
 * L == 0 is a no-op.  Other arguments and errors as in ra_share_forward.
 */
int ra_causal_share_forward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                            int32_t d, int32_t B, int32_t dtype, int32_t layout,
                            const void *Q_i, const void *K, const void *V, float scale,
                            float *O, float *m_out, float *l_out, void *O_cast, void *stream);

/*
 * Number of (query, key) pairs member `rank`'s causal share evaluates per (batch,
 * head): the sum over its queries of the keys at or before each.  Host only; exact.
 * Returns -RA_EINVAL for bad N, rank, L (L % N != 0, L < 0) or layout (zigzag: odd l),
 * -RA_ENOTSUP if the count exceeds INT64_MAX.
 */
int64_t ra_causal_pairs(int32_t rank, int32_t N, int64_t L, int32_t layout);

/*
 * Gradients of ring member `rank`'s (non-causal) share, bf16 inputs
 * (aliyun FlashAttention explainer, section 2: the backward pass recomputes the scores
 * from the stored output O and the softmax statistics instead of storing the attention
 * matrix).  With lse = m + ln(l) from ra_share_forward and D_r = dO_r . O_r:
 *     P  = exp(scale Q_i K^T - lse),   dS = P * (dO_i V^T - D)
 *     dQ_i = scale dS K,   dK += scale dS^T Q_i,   dV += P^T dO_i
 * over all L keys of the sequence (a share's softmax runs over every block, so the ring
 * order does not enter the gradient).
 *   Q_i, K, V  as in ra_share_forward (dtype must be RA_BF16, else RA_ENOTSUP)
 *   O          fp32 [B, H, l, d]: the forward output of the same share
 *   dO         [B, H, l, d] in `dtype`: the gradient of the loss with respect to O
 *   m, l       fp32 [B, H, l]: the forward's m_out and l_out
 *   dQ         fp32 [B, H, l, d], written
 *   dK, dV     fp32 [B, H_kv, L, d], ADDED to (zero them first; a ring passes them
 *              along with their K/V block and every member adds its part)
 *   workspace  device buffer of ra_share_backward_workspace(B, H, L / N) bytes, 16-byte
 *              aligned, owned by the caller; its contents are scratch
 * L == 0 is a no-op.  Other arguments and errors as in ra_share_forward.
 */
int ra_share_backward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv, int32_t d,
                      int32_t B, int32_t dtype, const void *Q_i, const void *K, const void *V,
                      const float *O, const void *dO, const float *m, const float *l,
                      float scale, float *dQ, float *dK, float *dV, void *workspace,
                      void *stream);

/*
 * Gradients of ring member `rank`'s causal share (the share of ra_causal_share_forward:
 * each query's softmax runs over the keys at or before its position, slowleelab "Ring
 * Attention" page, 4.5 limitation 2; positions from `layout` as there).  Same formulas
 * as ra_share_backward with P = 0 on the excluded pairs; key rows no query of the share
 * sees get nothing added.  The kernels skip the key tiles (for dQ) and query tiles (for
 * dK, dV) that hold no admissible pair.
 *   layout   an ra_layout; RA_LAYOUT_ZIGZAG needs l to be a multiple of 128, else
 *            RA_EINVAL
 *   O, m, l  the outputs of ra_causal_share_forward for the same share and layout
 * Other arguments, ownership and errors as in ra_share_backward.
 */
int ra_causal_share_backward(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                             int32_t d, int32_t B, int32_t dtype, int32_t layout,
                             const void *Q_i, const void *K, const void *V, const float *O,
                             const void *dO, const float *m, const float *l, float scale,
                             float *dQ, float *dK, float *dV, void *workspace, void *stream);

/* Bytes of workspace ra_share_backward (and ra_causal_share_backward) needs for B x H query rows of length l_q:
 * 8 * B * H * l_q (two floats per row).  Returns -RA_EINVAL for negative sizes,
 * -RA_ENOTSUP if the byte count does not fit int64. */
int64_t ra_share_backward_workspace(int32_t B, int32_t H, int64_t l_q);

/* Size of the static device scratch of ra_share_backward_noalloc: 8 MiB per GPU, enough
 * for B * H * l <= 1048576 query rows (the 128K / N = 8, H = 32 share needs 524288). */
#define RA_NOALLOC_SCRATCH_BYTES (8 << 20)

/*
 * ra_share_backward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * results and errors as ra_share_backward, without `workspace`: the per-row workspace
 * lives in a static device array of RA_NOALLOC_SCRATCH_BYTES that each GPU holds from
 * the first call on it until the process ends.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 *   - A problem whose ra_share_backward_workspace(B, H, L / N) exceeds
 *     RA_NOALLOC_SCRATCH_BYTES returns RA_ESCRATCH, after the usual argument checks and
 *     before any device work.
 *   - The array is shared by every call on one GPU and keeps the last call's contents
 *     (each call writes every entry it reads, so nothing needs clearing).  Calls that
 *     overlap on one GPU (other streams, other host threads) race on it: serialise them.
 */
int ra_share_backward_noalloc(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                              int32_t d, int32_t B, int32_t dtype, const void *Q_i,
                              const void *K, const void *V, const float *O, const void *dO,
                              const float *m, const float *l, float scale, float *dQ,
                              float *dK, float *dV, void *stream);

/*
 * FP8 (OCP E4M3) inputs with block quantization (aliyun FlashAttention explainer,
 * section 2, FlashAttention-3: the forward products run on FP8 matrix units and block
 * quantization limits the precision lost).  The pages fix neither the format nor the
 * blocks; this library uses OCP E4M3 (bias 7, largest value 448, no infinities) and:
 *   descale = max(amax / 448, 2^-126)      per block, fp32, amax = largest |x|
 *   code    = E4M3(x * (1 / descale))      round to nearest even, fp32 arithmetic
 * and a code stands for descale * value(code).  T(seg) = ceil(seg / 64).
 */
typedef enum ra_fp8_kind {
    RA_FP8_ROWS = 0, /* Q, K: one scale per 64-row block of each segment; codes keep the
                        input layout [B, Hx, n_seg*seg, d]; descale [B, Hx, n_seg, T] */
    RA_FP8_VT = 1    /* V: one scale per channel over all n_seg*seg rows, descale
                        [B, Hx, d]; codes stored per 64-row tile transposed,
                        [B, Hx, n_seg, T, d, 64], columns past a segment's end zero */
} ra_fp8_kind;

/* T(seg) = ceil(seg / 64); -RA_EINVAL for seg < 0.  Host only. */
int64_t ra_fp8_tiles(int64_t seg);

/*
 * Quantizes x (bf16 [B, Hx, n_seg*seg, d], device) to E4M3 codes and descales as above.
 * For a share, Q is one segment of l rows (n_seg = 1) and K, V are N segments of l rows
 * (the ring members' blocks).  Pointers: device, 16-byte aligned, caller-owned; the
 * call writes `codes` and `descale` only (RA_FP8_VT uses descale as scratch for the
 * maxima before finalising it in place).  seg == 0 is a no-op.  Errors: RA_EINVAL for
 * a bad kind, B, Hx, n_seg, seg, d (64 or 128) or pointer; RA_ENOTSUP for grids beyond
 * 2^31 - 1 work-groups or a device other than gfx950.
 */
int ra_quantize_fp8(int32_t kind, int32_t B, int32_t Hx, int32_t n_seg, int64_t seg, int32_t d,
                    const void *x, void *codes, float *descale, void *stream);

/*
 * Incoherent processing, then block quantization, for the query and key sides of the FP8
 * share (aliyun FlashAttention explainer, section 2, FlashAttention-3: block quantization
 * and incoherent processing limit the error of FP8 products).  Each row x of
 * x [B, Hx, n_seg * seg, d] (bf16) becomes x diag(signs) H_d, H_d the Sylvester Hadamard
 * matrix with entries +-1 (H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]), computed in fp32 by
 * the fast transform (for h = 1, 2, ..., d/2, each pair of entries (i, i + h) with
 * i & h == 0 becomes (a + b, a - b)), and is then quantized exactly as RA_FP8_ROWS does.
 * Since (Q S H)(K S H)^T = d Q K^T, quantize Q with query_side = 1 (its descales are
 * multiplied by 1/d, exact) and K with query_side = 0, with the same signs; the FP8 share
 * over those inputs then takes the usual scale and computes the same attention.  V is
 * quantized as before (RA_FP8_VT), unrotated.
 *   signs   device fp32 [d], normally random +-1 (drawn by the caller; other values are
 *           applied as given)
 *   codes, descale  as ra_quantize_fp8 with RA_FP8_ROWS
 * seg == 0 is a no-op.  Errors as ra_quantize_fp8 (RA_EINVAL also for a NULL signs).
 */
int ra_quantize_fp8_hadamard(int32_t B, int32_t Hx, int32_t n_seg, int64_t seg, int32_t d,
                             const void *x, const float *signs, int32_t query_side,
                             void *codes, float *descale, void *stream);

/*
 * Rank `rank`'s non-causal share (as ra_share_forward) from FP8 inputs, products on the
 * gfx950 FP8 matrix path, fp32 statistics:
 *   Q8 [B, H, l, d] codes with q_descale [B, H, T(l)]          (RA_FP8_ROWS, n_seg = 1)
 *   K8 [B, H_kv, L, d] codes with k_descale [B, H_kv, N, T(l)] (RA_FP8_ROWS, n_seg = N)
 *   V8t [B, H_kv, N, T(l), d, 64] codes with v_descale [B, H_kv, d]   (RA_FP8_VT)
 * computes O = softmax(scale * Qd Kd^T) Vd over the dequantized values, with the
 * probabilities themselves rounded to E4M3 before they weight V (and the row sum summing
 * those rounded probabilities).  O fp32 [B, H, l, d]; m_out, l_out as in
 * ra_share_forward (nullable); O_cast nullable bf16 [B, H, l, d].  Descales must be
 * positive and finite.  Errors as ra_share_forward; RA_ENOTSUP also when one K head
 * (L*d bytes) or V head (N*T(l)*64*d bytes) reaches 2^31 bytes.
 */
int ra_share_forward_fp8(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                         int32_t d, int32_t B, const void *Q8, const float *q_descale,
                         const void *K8, const float *k_descale, const void *V8t,
                         const float *v_descale, float scale, float *O, float *m_out,
                         float *l_out, void *O_cast, void *stream);

/*
 * Rank `rank`'s causal share (as ra_causal_share_forward: each query attends to the keys
 * at or before its position, slowleelab "Ring Attention" page, 4.5 limitation 2; token
 * positions from `layout`) from FP8 inputs laid out as for ra_share_forward_fp8.  Key
 * tiles that no query of a work-group may see are skipped.  RA_LAYOUT_ZIGZAG needs l to be
 * a multiple of 128, else RA_EINVAL.  Other arguments and errors as ra_share_forward_fp8.
 */
int ra_causal_share_forward_fp8(int32_t rank, int32_t N, int64_t L, int32_t H, int32_t H_kv,
                                int32_t d, int32_t B, int32_t layout, const void *Q8,
                                const float *q_descale, const void *K8, const float *k_descale,
                                const void *V8t, const float *v_descale, float scale, float *O,
                                float *m_out, float *l_out, void *O_cast, void *stream);

/* Static description of a status code. */
const char *ra_strerror(int status);

/* The hipError_t of the last failing HIP call on this thread (0 if none). */
int ra_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
