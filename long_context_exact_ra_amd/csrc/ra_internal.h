// ra_internal.h -- shared declarations between the C ABI layer and the kernel
// translation units of the ring-attention share library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

// Work description for one launch of the forward kernels.
//
// The launch covers every (batch, query head, query tile) of the resident block.
// Each work-group walks the K/V blocks in ring order: at step t it reads block
// j(t) = (rank - t) mod n_blocks (slowleelab "Ring Attention" page, L3 and 4.2),
// i.e. rows j*blk_rows .. (j+1)*blk_rows - 1 of the K/V head it is mapped to.
// A single ring step (ra_step) is n_blocks = 1, rank = 0 over a block pointer.
struct FwdArgs {
    const void *Q;   // [B, H, l_q, D] contiguous
    const void *K;   // head (b, g) starts at K + b*kv_batch_stride + g*kv_head_stride
    const void *V;
    float *O;        // share: finalised output; step: running O_acc (in/out)
    float *m;        // share: row max out (nullable); step: running max (in/out)
    float *l;        // share: row sum out (nullable); step: running sum (in/out)
    void *O_cast;    // share only, nullable: output in the input dtype
    int32_t *trace;  // share only, nullable: block index used at each step
    int64_t l_q;
    int64_t blk_rows;
    int64_t kv_head_stride;
    int64_t kv_batch_stride;
    int32_t n_blocks;
    int32_t rank;
    int32_t H;
    int32_t H_kv;
    int32_t group;     // H / H_kv
    int32_t n_qtiles;  // query tiles per (batch, head)
    int32_t n_wg;      // total work-groups of the launch
    float scale;       // score scale (normally 1/sqrt(d))
    float scale_log2;  // scale * log2(e): exponentials are taken as exp2
    int32_t layout;    // causal token layout (ra_layout), or kNoCausal
};

constexpr int32_t kNoCausal = -1;

// Work description of the backward kernels (one share's gradients).
struct BwdArgs {
    const void *Q;    // [B, H, l_q, D] contiguous
    const void *K;    // head (b, g) at K + b*kv_batch_stride + g*kv_head_stride, L rows
    const void *V;
    const void *dO;   // [B, H, l_q, D] contiguous, same dtype as Q
    float *ws;        // [B, H, l_q] pairs (D = dO . O, lse * log2(e)), written by prep
    float *dQ;        // [B, H, l_q, D] written
    float *dK;        // [B, H_kv, L, D] (kv strides) added to
    float *dV;
    int64_t l_q;
    int64_t L;
    int64_t kv_head_stride;
    int64_t kv_batch_stride;
    int32_t H;
    int32_t H_kv;
    int32_t group;      // H / H_kv
    int32_t n_qtiles;   // dQ: query tiles per (batch, head)
    int32_t n_wg;       // dQ work-groups
    int32_t n_ktiles;   // dK/dV: key tiles per (batch, kv head)
    int32_t n_kv_wg;    // dK/dV work-groups
    // Key tiling: n_kblocks blocks of kblk_rows keys each (block j = rows j*kblk_rows ...);
    // tiles never straddle two blocks.  A causal share has one block per ring member
    // (n_kblocks = N, kblk_rows = l_q); otherwise the keys are one block of L rows.
    int32_t n_kblocks;
    int64_t kblk_rows;
    int32_t n_ktiles_blk;  // dK/dV key tiles per block
    int32_t layout;        // ra_layout of a causal share, or kNoCausal
    int32_t rank;          // ring member whose queries these are (causal only)
    float scale;
    float scale_log2;
};

enum Mode : int {
    MODE_SHARE = 0,  // no state in; finalised output out
    MODE_STEP = 1    // running state in and out, no division
};

// Query rows per work-group of each kernel (the host sizes the grid with these).
int bf16_query_tile();
constexpr int kF32QueryTile = 64;

hipError_t launch_fwd_bf16(const FwdArgs &a, int B, int d, int mode, hipStream_t st);
// Rows per work-group of the backward kernels (query rows for dQ, key rows for dK/dV).
int bwd_query_tile();
int bwd_key_tile();
hipError_t launch_bwd_bf16(const BwdArgs &a, const float *O, const void *dO, const float *m,
                           const float *l, int64_t rows, int d, hipStream_t st);
hipError_t launch_fwd_f32(const FwdArgs &a, int B, int d, int mode, hipStream_t st);

// FP8 (OCP e4m3) share: one launch over every (batch, head, query tile), non-causal.
// Byte layouts (T = ceil(l / 64) tiles per member block of l rows):
//   Q8 [B, H, l, D], q_descale [B, H, T]; K8 [B, H_kv, N*l, D], k_descale [B, H_kv, N, T];
//   V8 [B, H_kv, N, T, D, 64] (each 64-key tile stored transposed), v_descale [B, H_kv, D].
struct Fp8Args {
    const uint8_t *Q8;
    const float *qs;
    const uint8_t *K8;
    const float *ks;
    const uint8_t *V8;
    const float *vs;
    float *O;      // [B, H, l, D] finalised output
    float *m;      // nullable
    float *l;      // nullable
    void *O_cast;  // nullable, bf16 [B, H, l, D]
    int64_t l_q;   // rows per member block (= l)
    int32_t n_blocks;
    int32_t rank;
    int32_t H;
    int32_t H_kv;
    int32_t group;
    int32_t n_tiles_blk;  // T
    int32_t n_qtiles;
    int32_t n_wg;
    float scale;
    int32_t layout;  // causal token layout (ra_layout), or kNoCausal
};
int fp8_query_tile();
hipError_t launch_fwd_fp8(const Fp8Args &a, int d, hipStream_t st);

// FP8 quantization (see ra_quantize_fp8): rows mode writes codes in the input layout and
// one descale per 64-row block of each segment; vt mode writes per-channel descales over
// all rows and tile-transposed codes.
hipError_t launch_quant_rows(const void *x, uint8_t *codes, float *descale, int64_t heads,
                             int32_t n_seg, int64_t seg, int d, hipStream_t st);
hipError_t launch_quant_vt(const void *x, uint8_t *codes, float *descale, int64_t heads,
                           int32_t n_seg, int64_t seg, int d, hipStream_t st);
// Rows mode after incoherent processing: each row times diag(signs) H_d (fp32 fast
// Hadamard transform), then quantized; the query side's descales carry a factor 1/d.
hipError_t launch_quant_rows_hadamard(const void *x, const float *signs, bool query_side,
                                      uint8_t *codes, float *descale, int64_t heads,
                                      int32_t n_seg, int64_t seg, int d, hipStream_t st);
hipError_t launch_state_init(float *O_acc, float *m, float *l, int64_t rows, int d,
                             hipStream_t st);

// Device address, on the current device, of the library's static scratch array
// (RA_NOALLOC_SCRATCH_BYTES bytes, 256-byte aligned), looked up once per device.
hipError_t noalloc_scratch(void **ptr);
hipError_t launch_finalize(float *O_acc, const float *l, int64_t rows, int d, int dtype,
                           void *O_out, hipStream_t st);

}  // namespace ra
