"""Pins of the share backward oracle (CPU only).

The backward pass of a share (aliyun page, FlashAttention section: recompute the
scores from the stored output and softmax statistics) is the gradient of
O = softmax(scale Q K^T) V.  The oracle writes that gradient out with the softmax
Jacobian; it is pinned here against central finite differences of the forward
definition, against torch autograd in fp64 (a library routine), and against identities
the gradient must satisfy.
"""
import numpy as np
import pytest
import torch

import oracle


def _forward(q, k, v, scale, mask=None):
    """softmax(scale q k^T) v per (b, h), fp64 numpy, GQA by repeated K/V heads."""
    g = q.shape[1] // k.shape[1]
    kk = np.repeat(k, g, axis=1)
    vv = np.repeat(v, g, axis=1)
    S = scale * np.einsum("bhqd,bhkd->bhqk", q, kk)
    if mask is not None:
        S = np.where(mask, S, -np.inf)
    P = np.exp(S - S.max(axis=-1, keepdims=True))
    P /= P.sum(axis=-1, keepdims=True)
    return np.einsum("bhqk,bhkd->bhqd", P, vv)


def _draw(rng, B, H, H_kv, l, L, d):
    f = lambda *s: rng.standard_normal(s).astype(np.float32)
    return f(B, H, l, d), f(B, H_kv, L, d), f(B, H_kv, L, d), f(B, H, l, d)


def test_gradients_match_central_differences():
    rng = np.random.default_rng(5)
    Q, K, V, dO = _draw(rng, 1, 2, 1, 3, 6, 4)
    scale = 0.7
    dQ, dK, dV = oracle.share_backward(Q, K, V, dO, scale)
    q, k, v, do = (x.astype(np.float64) for x in (Q, K, V, dO))
    loss = lambda q_, k_, v_: float(np.sum(_forward(q_, k_, v_, scale) * do))
    eps = 1e-6
    for name, x, grad in (("Q", q, dQ), ("K", k, dK), ("V", v, dV)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = {"Q": (xp, k, v), "K": (q, xp, v), "V": (q, k, xp)}[name]
            args_m = {"Q": (xm, k, v), "K": (q, xm, v), "V": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=1e-7, err_msg=name)


@pytest.mark.parametrize("layout", [None, "contiguous", "striped", "zigzag"])
def test_gradients_match_torch_autograd(layout):
    rng = np.random.default_rng(7)
    B, H, H_kv, d, N, l = 2, 4, 2, 8, 3, 6
    L = N * l
    rank = 1
    Q, K, V, dO = _draw(rng, B, H, H_kv, l, L, d)
    scale = 0.35
    dQ, dK, dV = oracle.share_backward(Q, K, V, dO, scale, rank, N, layout)
    q = torch.tensor(Q, dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K, dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V, dtype=torch.float64, requires_grad=True)
    mask = None
    if layout is not None:
        mask = torch.from_numpy(oracle.layout_positions(layout, N, L)[None, :]
                                <= oracle.token_positions(layout, rank, N, l)[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(H // H_kv, 1), v.repeat_interleave(H // H_kv, 1),
        attn_mask=mask, scale=scale)
    out.backward(torch.from_numpy(dO.astype(np.float64)))
    for got, ref in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=0, atol=1e-12)


def test_gradient_identities():
    rng = np.random.default_rng(9)
    Q, K, V, dO = _draw(rng, 1, 3, 3, 7, 21, 8)
    dQ, dK, dV = oracle.share_backward(Q, K, V, dO, 0.4)
    # each row of dS sums to zero, so the key gradients of a head sum to zero
    assert np.abs(dK.sum(axis=2)).max() < 1e-12
    # dV sums the upstream gradient over queries with softmax weights that sum to one
    np.testing.assert_allclose(dV.sum(axis=2), dO.astype(np.float64).sum(axis=2), atol=1e-12)
    # with every value row equal, the output does not depend on Q or K
    Vc = np.broadcast_to(V[:, :, :1], V.shape).copy()
    dQ, dK, _ = oracle.share_backward(Q, K, Vc, dO, 0.4)
    assert np.abs(dQ).max() < 1e-12 and np.abs(dK).max() < 1e-12


def test_sampled_rows_agree_with_the_dense_gradient():
    rng = np.random.default_rng(13)
    Q, K, V, dO = _draw(rng, 1, 4, 2, 40, 160, 8)
    dQ, dK, dV = oracle.share_backward(Q, K, V, dO, 0.3)
    heads = [(0, 1), (0, 2)]
    q_rows, k_rows = [0, 17, 39], [0, 5, 99, 159]
    res = oracle.share_backward_rows(Q, K, V, dO, 0.3, heads, q_rows, k_rows, chunk=16)
    # contributions of one query head: the dense K/V gradient sums over the group
    dK_h = {}
    for (b, h), (gq, gk, gv) in zip(heads, res):
        np.testing.assert_allclose(gq, dQ[b, h, q_rows], atol=1e-12)
        dK_h[h] = (gk, gv)
    only = oracle.share_backward(Q[:, 2:4], K[:, 1:2], V[:, 1:2], dO[:, 2:4], 0.3)
    np.testing.assert_allclose(dK_h[2][0] + oracle.share_backward_rows(
        Q, K, V, dO, 0.3, [(0, 3)], [], k_rows)[0][1], only[1][0, 0, k_rows], atol=1e-12)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_sampled_causal_rows_agree_with_the_dense_causal_gradient(layout):
    """The chunked, sampled form with a layout against the dense masked gradient (itself
    pinned to autograd and finite differences above), one query head per K/V head so the
    key-row parts are the whole gradient."""
    rng = np.random.default_rng(17)
    N, l, rank = 4, 32, 2
    Q, K, V, dO = _draw(rng, 1, 2, 2, l, N * l, 8)
    dQ, dK, dV = oracle.share_backward(Q, K, V, dO, 0.3, rank, N, layout)
    q_rows, k_rows = [0, 9, 16, 31], [0, 40, 64, 77, 100, 127]
    res = oracle.share_backward_rows(Q, K, V, dO, 0.3, [(0, 0), (0, 1)], q_rows, k_rows,
                                     chunk=8, rank=rank, N=N, layout=layout)
    for h, (gq, gk, gv) in enumerate(res):
        np.testing.assert_allclose(gq, dQ[0, h, q_rows], atol=1e-12)
        np.testing.assert_allclose(gk, dK[0, h, k_rows], atol=1e-12)
        np.testing.assert_allclose(gv, dV[0, h, k_rows], atol=1e-12)
