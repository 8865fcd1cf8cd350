"""Pins of the FP8 oracle (oracle/fp8.py) to things other than itself.

* The E4M3 codec against torch's float8_e4m3fn conversions (a library routine), the OCP
  format's defining values, its round-to-nearest-even ties and its overflow boundary.
* Block quantization against the error bound its definition implies (half a step of
  the format, times the block's scale), the largest element mapping to 448, all-zero
  blocks, and the tile-transposed V layout written out by index.
* The FP8 share against the already pinned bf16/fp32 share on inputs the format holds
  exactly (every block's largest magnitude is 448, so every scale is 1).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import fp8


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_defining_values_of_the_format():
    d = fp8.e4m3_decode
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0          # largest finite
    assert d(0x08) == 2.0 ** -6                            # smallest normal
    assert d(0x07) == 7 * 2.0 ** -9                        # largest subnormal
    assert d(0x01) == 2.0 ** -9                            # smallest subnormal
    assert d(0x38) == 1.0 and d(0xB8) == -1.0 and d(0x40) == 2.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert fp8.e4m3_encode(np.float32(0.3)) == 0x2A        # 0.3 -> 0.3125 = 1.25 * 2^-2


def test_encode_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(300_000) * np.exp2(rng.uniform(-16, 9, 300_000)))
    x = x.astype(np.float32)
    x = x[np.abs(x) < 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_midpoints_round_to_the_even_code_and_codes_round_trip():
    codes = np.array([c for c in range(0x00, 0x7E)], dtype=np.uint8)  # positive finite
    lo, hi = fp8.e4m3_decode(codes), fp8.e4m3_decode(codes + 1)
    mid = ((lo + hi) / 2).astype(np.float32)  # exact: at most 5 significant bits
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)
    got = fp8.e4m3_encode(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1)  # the code with an even mantissa
    assert np.array_equal(got, want)
    # just off the midpoint goes to the nearer code
    up = np.nextafter(mid, np.float32(np.inf))
    assert np.array_equal(fp8.e4m3_encode(up), codes + 1)
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(finite).astype(np.float32)),
                          finite)


def test_overflow_boundary():
    enc = fp8.e4m3_encode
    assert enc(np.float32(463.99)) == 0x7E and enc(np.float32(464.0)) == 0x7E
    assert enc(np.float32(464.01)) == 0x7F and enc(np.float32(-1e6)) == 0xFF
    assert enc(np.float32(np.inf)) == 0x7F


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


@pytest.mark.parametrize("n_seg,seg", [(1, 256), (3, 100), (2, 64), (4, 1)])
def test_quantize_rows_error_bound_and_extremes(n_seg, seg):
    rng = np.random.default_rng(5 + seg)
    B, Hx, d = 2, 3, 16
    x = (rng.standard_normal((B, Hx, n_seg * seg, d)) * np.exp2(rng.uniform(-6, 6, (B, Hx, 1, 1))))
    xb = _bf16_bits(x)
    x32 = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, ds = fp8.quantize_rows(xb, n_seg, seg)
    T = -(-seg // 64)
    assert codes.shape == x32.shape and ds.shape == (B, Hx, n_seg, T)
    deq = fp8.dequantize_rows(codes, ds, seg)
    rows = np.arange(n_seg * seg)
    step = ds.astype(np.float64)[:, :, rows // seg, (rows % seg) // 64][..., None]
    # a normal code is within 2^-4 relative of x / step, a subnormal within 2^-10
    xs = np.abs(x32) / step
    bound = np.where(xs >= 2.0 ** -6, 2.0 ** -4 * xs, 2.0 ** -10) * step * (1 + 1e-6)
    assert np.all(np.abs(deq - x32) <= bound)
    # each block's largest magnitude is stored as +-448
    for s in range(n_seg):
        for u in range(T):
            r0, r1 = s * seg + 64 * u, min(s * seg + 64 * u + 64, (s + 1) * seg)
            blk = np.abs(x32[:, :, r0:r1])
            cb = codes[:, :, r0:r1] & 0x7F
            assert np.all((cb == 0x7E).reshape(B, Hx, -1).any(axis=2))
            assert np.all(cb.reshape(B, Hx, -1)[blk.reshape(B, Hx, -1)
                                                == blk.reshape(B, Hx, -1).max(axis=2,
                                                                               keepdims=True)] == 0x7E)


def test_all_zero_block_gets_the_floor_scale_and_zero_codes():
    x = np.zeros((1, 1, 128, 8), dtype=np.float32)
    x[0, 0, 64:] = 1.5
    codes, ds = fp8.quantize_rows(x, 1, 128)
    assert ds[0, 0, 0, 0] == np.float32(2.0 ** -126) and np.all(codes[0, 0, :64] == 0)
    assert ds[0, 0, 0, 1] == np.float32(1.5) / np.float32(448)
    assert np.all(codes[0, 0, 64:] == 0x7E)


def test_quantize_vt_layout_written_out_by_index():
    rng = np.random.default_rng(3)
    B, Hx, n_seg, seg, d = 1, 2, 2, 70, 4  # two tiles per segment, the second ragged
    x = rng.standard_normal((B, Hx, n_seg * seg, d)).astype(np.float32)
    codes, ds = fp8.quantize_vt(x, n_seg, seg)
    assert codes.shape == (B, Hx, n_seg, 2, d, 64) and ds.shape == (B, Hx, d)
    # channel c of every row uses scale ds[c]; column r of tile u of segment s holds
    # row s*seg + 64u + r, zero past the segment end
    for h in range(Hx):
        for s in range(n_seg):
            for u in range(2):
                for c in range(d):
                    for r in range(64):
                        row = s * seg + 64 * u + r
                        got = codes[0, h, s, u, c, r]
                        if 64 * u + r >= seg:
                            assert got == 0
                        else:
                            inv = np.float32(1) / ds[0, h, c]
                            assert got == fp8.e4m3_encode(np.float32(x[0, h, row, c] * inv))
    deq = fp8.dequantize_vt(codes, ds, seg)
    assert np.all(np.abs(deq - x) <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * ds[:, :, None, :])
    for h in range(Hx):  # each channel's largest magnitude is 448 steps
        for c in range(d):
            k = np.argmax(np.abs(x[0, h, :, c]))
            assert abs(deq[0, h, k, c]) == pytest.approx(abs(x[0, h, k, c]), rel=2 ** -20)


def test_share_fp8_equals_the_plain_share_on_exactly_representable_inputs():
    """Values on the E4M3 grid with +-448 in every scale block: every scale is 1, the
    codes hold the values exactly, and the FP8 share is the (pinned) plain share."""
    rng = np.random.default_rng(9)
    B, H, H_kv, d, N, l = 1, 2, 1, 32, 3, 100
    L = N * l
    grid = fp8.e4m3_decode(np.array([c for c in range(0, 0x7E)], np.uint8))

    def draw(shape):
        v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
        return v.astype(np.float32)

    Q, K, V = draw((B, H, l, d)), draw((B, H_kv, L, d)), draw((B, H_kv, L, d))
    for t in (Q, K):  # first row of every 64-row block of every member block
        for s in range(t.shape[2] // l):
            for u in range(0, l, 64):
                t[:, :, s * l + u, 0] = 448.0
    V[:, :, 0, :] = 448.0
    Q8, qs = fp8.quantize_rows(Q, 1, l)
    K8, ks = fp8.quantize_rows(K, N, l)
    V8, vs = fp8.quantize_vt(V, N, l)
    assert np.all(qs == 1) and np.all(ks == 1) and np.all(vs == 1)
    scale = 2.0 ** -15
    for rank in (0, N - 1):
        O8, M8, Z8 = fp8.share_fp8(Q8, qs, K8, ks, V8, vs, scale, rank, N)
        O, M, Z = oracle.share(Q, K, V, scale, rank, N)
        np.testing.assert_allclose(O8, O, rtol=0, atol=1e-12 * np.abs(O).max())
        np.testing.assert_allclose(M8, M, rtol=1e-15)
        np.testing.assert_allclose(Z8, Z, rtol=1e-12)


def test_error_bounds_cover_a_cpu_model_of_the_kernel_roundings():
    """A numpy model of what the bound allows for (probabilities rounded to E4M3 relative
    to a reference 2^4 below the row maximum, grouped accumulation truncating terms 13
    bits below each group's largest) stays inside oracle.fp8.error_bounds, and a planted
    mistake in the model (a dropped key) does not."""
    rng = np.random.default_rng(21)
    B, H, d, N, l = 1, 1, 64, 2, 96
    L = N * l
    Q = rng.standard_normal((B, H, l, d)) * 2
    K = rng.standard_normal((B, H, L, d)) * 2
    V = rng.standard_normal((B, H, L, d))
    scale = 1 / 8
    rows = np.arange(l)
    O, M, Z = oracle.share(Q.astype(np.float64), K, V, scale, 0, N, rows=rows)
    bO, bm, bl = fp8.error_bounds(Q, K, V, scale, 0, N, O, rows)

    def trunc_group_sum(terms):  # groups of 8, terms truncated 13 bits below the max
        out = 0.0
        for g0 in range(0, len(terms), 8):
            t = terms[g0:g0 + 8]
            e = np.floor(np.log2(np.abs(t).max())) if np.any(t) else 0
            step = 2.0 ** (e - 13)
            out += np.sum(np.trunc(t / step) * step)
        return out

    worst = 0.0
    for r in rows:
        s = np.array([trunc_group_sum(scale * Q[0, 0, r] * K[0, 0, k]) for k in range(L)])
        p = np.exp(s - s.max()) * 16  # reference 2^4 below the maximum
        pq = fp8.e4m3_decode(fp8.e4m3_encode(p.astype(np.float32)))
        o = (pq @ V[0, 0]) / pq.sum()
        worst = max(worst, (np.abs(o - O[r]) / bO[r]).max())
        lq = pq.sum() / 16
        assert abs(lq - Z[r]) <= bl[r] and abs(s.max() - M[r]) <= bm[r]
    assert worst <= 1.0
    # a dropped key (a plausible kernel mistake) is caught for most rows
    caught = 0
    for r in rows[:16]:
        s = scale * (K[0, 0] @ Q[0, 0, r])
        p = np.exp(s - s.max())
        p[np.argmax(p)] = 0.0
        o = (p @ V[0, 0]) / p.sum()
        caught += (np.abs(o - O[r]) > bO[r]).any()
    assert caught >= 12


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_causal_share_fp8_equals_the_plain_causal_share_on_exact_inputs(layout):
    """As for the non-causal share: on exactly representable inputs (every scale 1) the
    FP8 causal share is the pinned causal share of the plain values."""
    rng = np.random.default_rng(31)
    B, H, H_kv, d, N, l = 1, 2, 1, 32, 4, 128
    grid = fp8.e4m3_decode(np.array([c for c in range(0, 0x7E)], np.uint8))

    def draw(shape):
        return (rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)).astype(np.float32)

    Q, K, V = draw((B, H, l, d)), draw((B, H_kv, N * l, d)), draw((B, H_kv, N * l, d))
    for t in (Q, K):
        for s0 in range(0, t.shape[2], 64):
            t[:, :, s0, 0] = 448.0
    V[:, :, 0, :] = 448.0
    Q8, qs = fp8.quantize_rows(Q, 1, l)
    K8, ks = fp8.quantize_rows(K, N, l)
    V8, vs = fp8.quantize_vt(V, N, l)
    assert np.all(qs == 1) and np.all(ks == 1) and np.all(vs == 1)
    for rank in (0, N - 1):
        O8, M8, Z8 = fp8.causal_share_fp8(Q8, qs, K8, ks, V8, vs, 2.0 ** -15, rank, N, layout)
        O, M, Z = oracle.causal_share(Q, K, V, 2.0 ** -15, rank, N, layout)
        np.testing.assert_allclose(O8, O, rtol=0, atol=1e-12 * np.abs(O).max())
        np.testing.assert_allclose(Z8, Z, rtol=1e-12)


# ------------------------------------------------------------------ incoherent processing

def test_hadamard_is_the_library_sylvester_matrix_and_orthogonal():
    import scipy.linalg
    for d in (1, 2, 4, 64, 128):
        H = fp8.hadamard(d)
        assert np.array_equal(H, scipy.linalg.hadamard(d))
        assert np.array_equal(H @ H.T, d * np.eye(d))


def test_fast_rotation_equals_the_matrix_product():
    rng = np.random.default_rng(31)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    # small integers: every float32 sum is exact, so the transform must equal the product
    x = rng.integers(-8, 9, size=(4, 7, 128)).astype(np.float32)
    y = fp8.hadamard_rotate(x, signs)
    assert np.array_equal(y, (x.astype(np.float64) * signs) @ fp8.hadamard(128))
    # general values: within the rounding of 7 butterfly stages
    x = rng.standard_normal((4, 7, 128)).astype(np.float32)
    y = fp8.hadamard_rotate(x, signs)
    ref = (x.astype(np.float64) * signs) @ fp8.hadamard(128)
    assert np.all(np.abs(y - ref) <= 7 * 2.0 ** -24 * 2 * np.abs(x).sum(axis=-1, keepdims=True))


def test_rotation_leaves_the_exact_share_unchanged():
    """(Q S H)(K S H)^T = d Q K^T: the share over rotated Q, K with scale / d is the share."""
    rng = np.random.default_rng(32)
    B, H, d, l, N = 1, 2, 64, 16, 4
    L = N * l
    Q = rng.standard_normal((B, H, l, d))
    K = rng.standard_normal((B, H, L, d))
    V = rng.standard_normal((B, H, L, d))  # all three inputs float64
    signs = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    R = signs[:, None] * fp8.hadamard(d)
    O1, M1, Z1 = oracle.share(Q, K, V, 0.125, 1, N)
    O2, M2, Z2 = oracle.share(Q @ R, K @ R, V, 0.125 / d, 1, N)
    np.testing.assert_allclose(O2, O1, atol=1e-12)
    np.testing.assert_allclose(M2 + np.log(Z2), M1 + np.log(Z1), atol=1e-12)


def test_rotated_quantization_folds_one_over_d_into_query_descales():
    rng = np.random.default_rng(33)
    x = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(5))
    bits = x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    signs = np.where(rng.random(128) < 0.5, -1.0, 1.0)
    ck, dk = fp8.quantize_rows_hadamard(bits, signs, 1, 128, False)
    cq, dq = fp8.quantize_rows_hadamard(bits, signs, 1, 128, True)
    assert np.array_equal(ck, cq)
    assert np.array_equal(dq, (dk / np.float32(128)).astype(np.float32))
    r = fp8.hadamard_rotate(bits, signs)
    rc, rd = fp8.quantize_rows(r, 1, 128)
    assert np.array_equal(ck, rc) and np.array_equal(dk, rd)


def test_rotation_spreads_an_outlier_channel():
    """The point of incoherent processing: with one large channel in Q and K, the FP8
    scores of the rotated pair are closer to the exact ones than without the rotation."""
    g = torch.Generator().manual_seed(6)
    d, n = 128, 256
    q = torch.randn(1, 1, n, d, generator=g)
    k = torch.randn(1, 1, n, d, generator=g)
    q[..., 5] *= 40.0
    k[..., 5] *= 40.0
    qb, kb = (t.to(torch.bfloat16) for t in (q, k))
    Qb, Kb = (t.view(torch.int16).numpy().view(np.uint16) for t in (qb, kb))
    exact = qb.double()[0, 0].numpy() @ kb.double()[0, 0].numpy().T
    cq, dq = fp8.quantize_rows(Qb, 1, n)
    ck, dk = fp8.quantize_rows(Kb, 1, n)
    plain = fp8.dequantize_rows(cq, dq, n)[0, 0] @ fp8.dequantize_rows(ck, dk, n)[0, 0].T
    signs = np.where(np.random.default_rng(34).random(d) < 0.5, -1.0, 1.0)
    cq, dq = fp8.quantize_rows_hadamard(Qb, signs, 1, n, True)
    ck, dk = fp8.quantize_rows_hadamard(Kb, signs, 1, n, False)
    rot = fp8.dequantize_rows(cq, dq, n)[0, 0] @ fp8.dequantize_rows(ck, dk, n)[0, 0].T
    e_plain = np.abs(plain - exact).mean()
    e_rot = np.abs(rot - exact).mean()
    assert e_rot < 0.7 * e_plain, (e_rot, e_plain)
