"""Per-row error bounds of the bf16 share's row statistics (m and lse = m + ln l).

The pages fix a tolerance for the output O only; m and l are this build's outputs, so
their bounds are derived here from the arithmetic the kernel performs, term by term:

  * Scores.  The bf16 matrix instruction multiplies exactly (8-bit significands) and, in
    each group of 8 consecutive head-dimension products, truncates every term toward zero
    24 bits below the group's largest term before summing; group sums enter the fp32
    accumulator with one rounding each (16 per 128-dim score).  This model is pinned
    on the GPU through the library (tests/test_gpu_accumulation.py).  It bounds a raw
    score's error by 8*2^-24 per group maximum plus 16 roundings, below
        E = 2^-19 * S,   S = max_k sum_i |q_i k_ki|
    with S bounded per row by min(|q|_2 max_k |k_k|_2, sum_i |q_i| max_k |k_ki|).
  * Exponent.  exp2 takes fl(s*c~ - R) with c~ = fl(scale * log2 e): the argument is off
    by at most c*E + 2^-24 * c * S (c~) + 2^-24 * 2 c S (the fma), i.e.
    dx <= c * S * (2^-19 + 2^-22), which moves every term by a factor within 2^(+-dx).
  * v_exp_f32.  Taken as accurate to 2^-21 relative (4 ulp; assumed, not measured: the
    library's outputs round every probability to bf16 before it can be observed).
  * bf16 probabilities.  Round to nearest even with 8 significant bits: each summed term
    is within 2^-8 relative of its fp32 value, and in the worst case all in one direction.
  * The row sum.  Each lane half sums a tile's 16 probabilities on its own (16 roundings
    at most, two per packed dot product), adds the tile sum to the running sum (one
    rounding per tile), is rescaled at each reference raise (one rounding; at most
    1 + 2 c S / 8 raises, since the reference only rises, by more than 8 each time, within
    a range of 2 c S), and the two halves are added once:
        (16 + n_tiles + n_raise + 1) * 2^-24 relative.
  * Output.  l_out = ltot * exp2(R - m log2 e) adds exp2's error, one product rounding
    and the argument's rounding (2^-24 * 8 for the difference, 2^-23 |m| log2 e for
    m log2 e with log2 e itself rounded).  The step path does this once per launch, and
    its next launch rebuilds the reference from the stored m (one more exp2 and rounding
    in the first rescale), so these terms count once per step.
Summing (as a bound on |ln(l_gpu / l_exact)| plus the m terms, which cancel in lse up
to the last item):
    |lse - lse_ref| <= ln(1 + 2^-8) + (16 + n_tiles + n_raise + 1) 2^-24
                       + ln2 * c S (2^-19 + 2^-22)
                       + steps * (ln2 (2^-21 + 8 * 2^-24 + 1.5 |M| 2^-23) + 2 * 2^-21 + 4 * 2^-24)
    |m - M| <= scale * E + 2^-23 |M|
where M is the exact row maximum of scale * q.k.  A small 1e-7 is added to both for the
fp64 evaluation of the reference itself.
"""
import math

import numpy as np

TILE_KEYS = 64


def _f32(bits):
    """fp32 values of stored bf16 bits (uint16) or of an fp32 array."""
    a = np.asarray(bits)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32)
    return a.astype(np.float32)


def stat_bounds_bf16(Qh, Kh, shape, scale, rows, M, n_tiles=None, n_steps=1):
    """Bounds (bound_m [n], bound_lse [n]) for the listed flat rows of a bf16 share.

    Qh, Kh: the stored bits (uint16 views of bf16) of Q_i [B, H, l, d] and
    K [B, H_kv, L, d]; shape = (B, H, H_kv, d, l, L); M: the exact row maxima (fp64).
    n_tiles: key tiles the kernel visits (default: N blocks of l keys, each rounded up
    to whole tiles, with N = L / l).  n_steps: separate launches whose state is carried
    through memory (the step path); each adds its own conversion of the state to the
    exact maximum (one exp2 and four roundings)."""
    B, H, H_kv, d, l, L = shape
    rows = np.asarray(rows, dtype=np.int64)
    Q = _f32(Qh).reshape(B * H * l, d)[rows].astype(np.float64)
    K = _f32(Kh).reshape(B, H_kv, L, d)
    g = H // H_kv
    knorm = np.empty((B, H_kv))
    kabs = np.empty((B, H_kv, d))
    for b in range(B):
        for h in range(H_kv):
            kk = K[b, h]
            knorm[b, h] = np.sqrt((kk.astype(np.float64) ** 2).sum(axis=1).max()) if L else 0.0
            kabs[b, h] = np.abs(kk).max(axis=0) if L else 0.0
    heads = (rows // l) % H
    bs = rows // (H * l)
    gk = heads // g
    s_cs = np.sqrt((Q * Q).sum(axis=1)) * knorm[bs, gk]
    s_l1 = (np.abs(Q) * kabs[bs, gk]).sum(axis=1)
    S = np.minimum(s_cs, s_l1)
    scale = float(np.float32(scale))
    c = scale * math.log2(math.e)
    M = np.abs(np.asarray(M, dtype=np.float64))
    if n_tiles is None:
        n_tiles = (L // l) * -(-l // TILE_KEYS) if l else 0
    n_raise = 1.0 + 2.0 * c * S / 8.0
    u = 2.0 ** -24
    ln2 = math.log(2.0)
    b_lse = (math.log1p(2.0 ** -8) + (16 + n_tiles + n_raise + 1) * u
             + ln2 * (c * S * (2.0 ** -19 + 2.0 ** -22))
             + n_steps * (ln2 * (2.0 ** -21 + 8 * u + 1.5 * M * 2.0 ** -23) + 2 * 2.0 ** -21 + 4 * u)
             + 1e-7)
    b_m = scale * S * 2.0 ** -19 + 2.0 ** -23 * M + 1e-7
    return b_m, b_lse
