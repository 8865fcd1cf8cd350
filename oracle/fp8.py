"""FP8 (OCP E4M3) inputs for a share: block quantization and the attention it defines.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite, the smoke
check and the CPU-baseline leg of the benchmark use it.

FlashAttention-3 runs the forward products on FP8 matrix units and limits the precision
lost in the conversion with block quantization (aliyun FlashAttention explainer,
section 2, the FlashAttention-3 paragraph on low-precision GEMMs).  The pages fix
neither the FP8 format nor the block shapes; the readings taken here are:

* Format: OCP FP8 E4M3 ("e4m3fn"): 1 sign, 4 exponent bits with bias 7, 3 mantissa
  bits; exponent 0 holds the subnormals m/8 * 2^-6; S.1111.111 is NaN; there are no
  infinities and the largest finite value is 448.  Encoding rounds to nearest, ties to
  even; magnitudes at or beyond 464 (half-way to the next, non-existent step) give NaN.
* Blocks: Q and K get one scale per 64-row block of each member's block of rows (a K/V
  tile, or a query tile); V gets one scale per channel (head-dim column) over the
  whole sequence, which can be applied once to the output.
* Scale: descale = max(float32(amax / 448), 2^-126) per block, with amax the largest
  magnitude in the block; a value x is stored as encode(float32(x * float32(1 /
  descale))) and stands for descale * decode(code).  All of that arithmetic is fp32
  with round-to-nearest, as written.
* V is stored tile-transposed: for each member block s and 64-row tile u, a [d, 64]
  byte matrix whose column r is row s*seg + 64u + r (zero past the block end).

The share over such inputs is the plain definition of attention over the dequantized
values (fp64 products descale * decode(code) are exact), evaluated by the same C code as
the bf16 share.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
FLT_MIN = np.float32(2.0 ** -126)
TILE = 64  # rows per scale block of Q and K, keys per stored V tile


def e4m3_decode(codes) -> np.ndarray:
    """fp64 value of each E4M3 code (uint8); NaN for the two NaN codes."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x) -> np.ndarray:
    """E4M3 code (uint8) of each float32 value, round to nearest, ties to even."""
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)  # exact
    a = np.where(np.isfinite(a), a, 1e9)  # non-finite inputs take the NaN code below
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    # subnormal range: multiples of 2^-9 below 2^-6 (q == 8 is the smallest normal)
    q_sub = np.rint(a * 2.0 ** 9).astype(np.int64)
    # normal range: a = (1 + f) 2^e with f in [0, 1); 8 f rounded to an integer
    frac, ex = np.frexp(np.where(a > 0, a, 1.0))  # a = frac * 2^ex, frac in [0.5, 1)
    e = ex.astype(np.int64) - 1
    q = np.rint((frac * 2.0 - 1.0) * 8.0).astype(np.int64)
    carry = q == 8
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 0, q)
    normal = (e + 7) * 8 + q
    over = (e > 8) | ((e == 8) & (q == 7))
    code = np.where(a < 2.0 ** -6, q_sub, np.where(over, 0x7F, normal))
    return (sign | code).astype(np.uint8)


def block_descale(amax) -> np.ndarray:
    """max(float32(amax / 448), 2^-126), elementwise, float32."""
    amax = np.asarray(amax, dtype=np.float32)
    return np.maximum(amax / np.float32(E4M3_MAX), FLT_MIN).astype(np.float32)


def _quantize(x32: np.ndarray, descale: np.ndarray) -> np.ndarray:
    inv = (np.float32(1.0) / descale).astype(np.float32)
    return e4m3_encode((x32 * inv).astype(np.float32))


def _f32(x) -> np.ndarray:
    """bf16 bits (uint16) or float32 values as float32."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32)
    if x.dtype == np.float32:
        return x
    raise TypeError("expected bf16 bits (uint16) or float32")


def quantize_rows(x, n_seg: int, seg: int):
    """Per-block quantization of x [B, Hx, n_seg*seg, d] (bf16 bits or float32): blocks
    of 64 rows inside each of the n_seg segments of seg rows (the last block of a
    segment may be shorter).  Returns (codes uint8 [B, Hx, n_seg*seg, d], descale
    float32 [B, Hx, n_seg, ceil(seg/64)])."""
    x32 = _f32(x)
    B, Hx, R, d = x32.shape
    if R != n_seg * seg:
        raise ValueError("rows must be n_seg * seg")
    T = -(-seg // TILE)
    codes = np.empty(x32.shape, dtype=np.uint8)
    descale = np.empty((B, Hx, n_seg, T), dtype=np.float32)
    for s in range(n_seg):
        for u in range(T):
            r0 = s * seg + u * TILE
            r1 = min(r0 + TILE, (s + 1) * seg)
            blk = x32[:, :, r0:r1, :]
            ds = block_descale(np.abs(blk).max(axis=(2, 3)))  # [B, Hx]
            descale[:, :, s, u] = ds
            codes[:, :, r0:r1, :] = _quantize(blk, ds[:, :, None, None])
    return codes, descale


def quantize_vt(x, n_seg: int, seg: int):
    """Per-channel quantization of x [B, Hx, n_seg*seg, d] over all rows, stored
    tile-transposed.  Returns (codes uint8 [B, Hx, n_seg, T, d, 64], descale float32
    [B, Hx, d]), T = ceil(seg/64); columns past a segment's end hold code 0."""
    x32 = _f32(x)
    B, Hx, R, d = x32.shape
    if R != n_seg * seg:
        raise ValueError("rows must be n_seg * seg")
    T = -(-seg // TILE)
    descale = block_descale(np.abs(x32).max(axis=2))  # [B, Hx, d]
    q = _quantize(x32, descale[:, :, None, :])  # [B, Hx, R, d]
    codes = np.zeros((B, Hx, n_seg, T, d, TILE), dtype=np.uint8)
    for s in range(n_seg):
        for u in range(T):
            r0 = s * seg + u * TILE
            r1 = min(r0 + TILE, (s + 1) * seg)
            codes[:, :, s, u, :, : r1 - r0] = np.swapaxes(q[:, :, r0:r1, :], 2, 3)
    return codes, descale


def dequantize_rows(codes, descale, seg: int) -> np.ndarray:
    """fp64 values of quantize_rows' output (exact)."""
    B, Hx, R, d = codes.shape
    rows = np.arange(R)
    s, u = rows // seg, (rows % seg) // TILE
    ds = np.asarray(descale, dtype=np.float64)[:, :, s, u]  # [B, Hx, R]
    return e4m3_decode(codes) * ds[:, :, :, None]


def dequantize_vt(codes, descale, seg: int) -> np.ndarray:
    """fp64 values [B, Hx, n_seg*seg, d] of quantize_vt's output (exact)."""
    B, Hx, n_seg, T, d, _ = codes.shape
    R = n_seg * seg
    rows = np.arange(R)
    s, u, r = rows // seg, (rows % seg) // TILE, (rows % seg) % TILE
    rows_major = np.swapaxes(codes, 4, 5)  # [B, Hx, n_seg, T, 64, d]
    vals = e4m3_decode(rows_major[:, :, s, u, r, :])  # [B, Hx, R, d]
    return vals * np.asarray(descale, dtype=np.float64)[:, :, None, :]


def share_fp8(Q8, q_descale, K8, k_descale, V8t, v_descale, scale, rank: int, N: int,
              rows=None, nthreads=None):
    """Rank `rank`'s share over FP8 inputs: Q8 [B, H, l, d] with q_descale
    [B, H, 1, ceil(l/64)]; K8 [B, H_kv, L, d] with k_descale [B, H_kv, N, ceil(l/64)];
    V8t [B, H_kv, N, ceil(l/64), d, 64] with v_descale [B, H_kv, d].  The plain
    definition over the dequantized values; returns (O, M, Z) as attention_rows."""
    from . import share
    l = Q8.shape[2]
    Qd = dequantize_rows(Q8, q_descale, l)
    Kd = dequantize_rows(K8, k_descale, l)
    Vd = dequantize_vt(V8t, v_descale, l)
    return share(Qd, Kd, Vd, scale, rank, N, rows=rows, nthreads=nthreads)


def causal_share_fp8(Q8, q_descale, K8, k_descale, V8t, v_descale, scale, rank: int, N: int,
                     layout: str, rows=None, nthreads=None):
    """The causal share (causal_share: keys at or before each query's position under
    `layout`) over the dequantized FP8 inputs of share_fp8."""
    from . import causal_share
    l = Q8.shape[2]
    Qd = dequantize_rows(Q8, q_descale, l)
    Kd = dequantize_rows(K8, k_descale, l)
    Vd = dequantize_vt(V8t, v_descale, l)
    return causal_share(Qd, Kd, Vd, scale, rank, N, layout, rows=rows, nthreads=nthreads)


def error_bounds(Qd, Kd, Vd, scale, rank: int, N: int, O_ref, rows, layout=None):
    """Allowed deviation of an FP8 share from the exact share over the dequantized values
    Qd, Kd, Vd (fp64), for the listed flat rows (O_ref: the exact rows).  Returns
    (bound_O [n, d], bound_m [n], bound_l [n]).

    The rounding steps it allows for, beyond the dequantized inputs themselves:
    * the FP8 matrix instruction's grouped accumulation: each group of 8 consecutive
      products is summed with its terms truncated to 13 fractional bits below the
      group's largest product (measured on gfx950), so a score is off by at most
      ds_k = 2^-10 * scale * sum_d |q_d k_d|, and the P V and row-sum products by 2^-10 of
      their magnitude sums;
    * E4M3 rounding of each probability, taken relative to a reference at least 2^4 below
      the row maximum: relative 2^-4 for P_k >= 2^-10 (row maximum 1), absolute 2^-14
      below;
    * fp32 accumulation over L keys (L * 2^-23 relative to the magnitude sum).
    With e_k = max(2^-4 P_k, 2^-14) + 1.1 P_k expm1(ds_k):
      |O - O_ref| <= 2 sum_k e_k |V_k - O_ref| / Z + (2^-9 + L 2^-23) sum_k P_k |V_k| / Z + 1e-6
      |m - M|     <= max_k ds_k + 1e-6 max(1, |M|)
      |l - Z|     <= 2 sum_k e_k + sum_k P_k expm1(ds_k + max_k ds_k) + (2^-9 + L 2^-23) Z
    (the factor 2 covers the row sum's own deviation in the denominator).  With `layout`,
    the sums run over each row's admissible keys only (the causal share)."""
    # A whole share covers every key; the ring order does not enter the sums.
    B, H, l, d = Qd.shape
    H_kv, L = Kd.shape[1], Kd.shape[2]
    if L != N * l or not 0 <= rank < N:
        raise ValueError("a share covers all N blocks of l keys")
    g = H // H_kv
    acc = 2.0 ** -9 + L * 2.0 ** -23
    if layout is not None:
        from . import layout_positions, token_positions
        kpos = layout_positions(layout, N, L)
        qpos = token_positions(layout, rank, N, l)
    rows = np.asarray(rows, dtype=np.int64)
    bO = np.empty((len(rows), d))
    bm = np.empty(len(rows))
    bl = np.empty(len(rows))
    held = (None, None, None)  # (batch, K/V head), |K|, |V| of the last row's head
    for i, r in enumerate(rows):
        b, h, q = r // (H * l), (r // l) % H, r % l
        k, v = Kd[b, h // g], Vd[b, h // g]
        if held[0] != (b, h // g):  # |K| and |V| once per head, not once per row
            held = ((b, h // g), np.abs(k), np.abs(v))
        ak, av = held[1], held[2]
        if layout is not None:
            keep = kpos <= qpos[q]
            k, v, ak, av = k[keep], v[keep], ak[keep], av[keep]
        s = scale * (k @ Qd[b, h, q])
        ds = 2.0 ** -10 * scale * (ak @ np.abs(Qd[b, h, q]))
        P = np.exp(s - s.max())
        Z = P.sum()
        e = np.maximum(2.0 ** -4 * P, 2.0 ** -14) + 1.1 * P * np.expm1(ds)
        dev = np.subtract(v, O_ref[i])
        np.abs(dev, out=dev)
        bO[i] = (2 * (e @ dev) + acc * (P @ av)) / Z + 1e-6
        bm[i] = ds.max() + 1e-6 * max(1.0, abs(s.max()))
        bl[i] = 2 * e.sum() + P @ np.expm1(ds + ds.max()) + acc * Z
    return bO, bm, bl



# ------------------------------------------------------------------ incoherent processing
#
# The FlashAttention-3 paragraph of the aliyun explainer names a second remedy for the
# error of FP8 products beside block quantization: incoherent processing, i.e. multiplying
# Q and K by the same random orthogonal matrix along the head dimension before quantizing,
# which leaves Q K^T unchanged and spreads any outlier channel over all of them.  The page
# fixes neither the matrix nor the scaling; the reading taken here is the Sylvester
# Hadamard matrix H_d (entries +-1, H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]) times a
# diagonal of random signs S, unnormalised: (Q S H)(K S H)^T = d Q K^T, and the factor 1/d
# (a power of two) goes into Q's descales, so the share over the quantized rotated inputs
# uses the usual scale.


def hadamard(d: int) -> np.ndarray:
    """The Sylvester Hadamard matrix H_d (d a power of two), float64 entries +-1."""
    if d < 1 or d & (d - 1):
        raise ValueError("d must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard_rotate(x, signs) -> np.ndarray:
    """x [..., d] (bf16 bits or float32) times diag(signs) H_d, in float32, by the fast
    transform: after the sign flips (exact), for h = 1, 2, 4, ..., d/2 every pair of
    entries (i, i + h) with i & h == 0 becomes (a + b, a - b), each a single float32
    rounding.  (H_d is symmetric, so row vectors times H_d are H_d times columns.)"""
    y = (_f32(x) * np.asarray(signs, dtype=np.float32)).astype(np.float32)
    d = y.shape[-1]
    if d & (d - 1):
        raise ValueError("d must be a power of two")
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :], y[..., 1, :]
        y = np.stack([(a + b).astype(np.float32), (a - b).astype(np.float32)], axis=-2)
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return y


def quantize_rows_hadamard(x, signs, n_seg: int, seg: int, query_side: bool):
    """Incoherent processing then block quantization: quantize_rows of
    hadamard_rotate(x, signs); for the query side (query_side) the descales are
    multiplied by 1/d (exact: a power of two), so that a share over Q and K quantized
    this way needs no change of scale.  Returns (codes, descale) as quantize_rows."""
    r = hadamard_rotate(x, signs)
    codes, descale = quantize_rows(r, n_seg, seg)
    if query_side:
        descale = (descale * np.float32(1.0 / r.shape[-1])).astype(np.float32)
    return codes, descale
