"""GPU parity of the causal share backward (ra_causal_share_backward) against the fp64
oracle's masked gradient.

The share's softmax runs over the keys at or before each query's position (slowleelab
"Ring Attention" page, 4.5 limitation 2), positions from the contiguous, striped (4.8) or
zigzag assignment of tokens to ring members.  The error model and the bound are those of
the non-causal backward (test_gpu_backward.py), with P = 0 on the excluded pairs; key rows
that no query of the share sees must come out exactly zero.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_ra_amd import ra, synth
from test_gpu_backward import TOL, _bits, _draw, _tile_edge_rows, check, sampled_magnitudes
from test_gpu_parity import _say

pytestmark = pytest.mark.gpu

LAYOUTS = ["contiguous", "striped", "zigzag"]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ra.load()
    return torch.device("cuda:0")


def run_gpu(q, k, v, do, N, rank, layout, scale, dev):
    B, H, l, d = q.shape
    H_kv, L = k.shape[1], k.shape[2]
    qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
    O = torch.empty((B, H, l, d), dtype=torch.float32, device=dev)
    m = torch.empty((B, H, l), dtype=torch.float32, device=dev)
    lo = torch.empty_like(m)
    ra.causal_share_forward(rank, N, L, H, H_kv, d, B, layout, qd, kd, vd, scale, O, m, lo)
    dQ = torch.full((B, H, l, d), float("nan"), dtype=torch.float32, device=dev)
    dK = torch.zeros((B, H_kv, L, d), dtype=torch.float32, device=dev)
    dV = torch.zeros_like(dK)
    ra.causal_share_backward(rank, N, L, H, H_kv, d, B, layout, qd, kd, vd, O, dod, m, lo,
                             scale, dQ, dK, dV)
    torch.cuda.synchronize()
    return dQ.cpu().numpy(), dK.cpu().numpy(), dV.cpu().numpy()


def masked_magnitudes(q, k, v, do, scale, rank, N, layout):
    """Per-element error magnitudes as in test_gpu_backward.magnitudes, over the
    admissible pairs only."""
    Q, K, V, dO = (oracle.bf16_bits_to_f64(_bits(x)) for x in (q, k, v, do))
    B, H, l, d = Q.shape
    L = K.shape[2]
    g = H // K.shape[1]
    allow = (oracle.layout_positions(layout, N, L)[None, :]
             <= oracle.token_positions(layout, rank, N, l)[:, None])
    mq, mk, mv = np.zeros_like(Q), np.zeros_like(K), np.zeros_like(V)
    for b in range(B):
        for h in range(H):
            kk, vv = K[b, h // g], V[b, h // g]
            S = np.where(allow, scale * Q[b, h] @ kk.T, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dP = dO[b, h] @ vv.T
            Dq = np.sum(P * dP, axis=1, keepdims=True)
            Dmag = np.sum(np.abs(dO[b, h]) * (P @ np.abs(vv)), axis=1, keepdims=True)
            A = P * np.abs(dP - Dq)
            mq[b, h] = scale * (A @ np.abs(kk) + Dmag * (P @ np.abs(kk)))
            mk[b, h // g] += scale * ((A + P * Dmag).T @ np.abs(Q[b, h]))
            mv[b, h // g] += P.T @ np.abs(dO[b, h])
    return mq, mk, mv, allow


def compare(q, k, v, do, N, rank, layout, scale, dev, tag):
    dQ, dK, dV = run_gpu(q, k, v, do, N, rank, layout, scale, dev)
    rQ, rK, rV = oracle.share_backward(_bits(q), _bits(k), _bits(v), _bits(do), scale, rank,
                                       N, layout)
    mq, mk, mv, allow = masked_magnitudes(q, k, v, do, scale, rank, N, layout)
    w = [check(n, g_, r_, m_) for n, g_, r_, m_ in
         (("dQ", dQ, rQ, mq), ("dK", dK, rK, mk), ("dV", dV, rV, mv))]
    unseen = ~allow.any(axis=0)  # key rows no query of this share attends to
    assert np.all(dK[:, :, unseen] == 0) and np.all(dV[:, :, unseen] == 0), "unseen keys"
    _say(f"causal backward {tag}: worst err/bound dQ {w[0]:.3f} dK {w[1]:.3f} "
         f"dV {w[2]:.3f}; {int(unseen.sum())} unseen key rows")


# (layout, B, H, H_kv, d, N, l): ragged blocks (contiguous / striped), zigzag half-blocks
# of one and of several tiles, GQA, both head sizes, and blocks shorter than one 32-key group
CASES = [
    ("contiguous", 1, 2, 1, 128, 3, 300),
    ("contiguous", 2, 2, 2, 64, 2, 256),
    ("striped", 2, 4, 2, 64, 4, 200),
    ("striped", 1, 2, 2, 128, 3, 384),
    ("zigzag", 1, 3, 3, 128, 2, 384),
    ("zigzag", 1, 4, 2, 64, 4, 256),
    ("contiguous", 1, 2, 1, 128, 3, 7),
    ("striped", 1, 1, 1, 64, 4, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_every_rank_against_the_oracle(dev, case):
    layout, B, H, H_kv, d, N, l = case
    q, k, v, do = _draw(B, H, H_kv, d, l, N * l, 6000 + l + N)
    for rank in range(N):
        compare(q, k, v, do, N, rank, layout, 1.0 / math.sqrt(d), dev,
                f"{case} rank {rank}")


@pytest.mark.parametrize("layout", LAYOUTS)
def test_large_logits(dev, layout):
    """Q/K with std 3: peaked rows, the diagonal key often dominant."""
    B, H, H_kv, d, N, l = 1, 2, 2, 128, 4, 256
    q, k, v, do = _draw(B, H, H_kv, d, l, N * l, 6300, std=3.0)
    for rank in (0, N - 1):
        compare(q, k, v, do, N, rank, layout, 1.0 / math.sqrt(d), dev,
                f"std 3 {layout} rank {rank}")


def test_single_member_is_the_plain_causal_gradient(dev):
    """N = 1: every layout is the ordinary causal mask; the three agree bit for bit."""
    q, k, v, do = _draw(1, 2, 2, 128, 512, 512, 6400)
    outs = [run_gpu(q, k, v, do, 1, 0, lay, 0.09, dev) for lay in LAYOUTS]
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)
    compare(q, k, v, do, 1, 0, "contiguous", 0.09, dev, "N = 1")


def test_rejects_zigzag_blocks_that_split_tiles(dev):
    q, k, v, do = _draw(1, 1, 1, 64, 192, 384, 6500)
    with pytest.raises(ra.RaError):
        run_gpu(q, k, v, do, 2, 0, "zigzag", 0.1, dev)


@pytest.mark.parametrize("layout", ["contiguous", "zigzag"])
def test_32k_share_sampled_rows(dev, layout):
    """The 32K / N = 8 causal share (H = 32, d = 128) at full size, rank 3; sampled query
    rows (dQ) and key rows (dK, dV) of two heads against the oracle, rows chosen on both
    sides of the mask's edge."""
    w = synth.WORKLOADS["share_L32K_N8"]
    q, k, v = synth.draw_workload(w)
    g = torch.Generator().manual_seed(w.seed + 99)
    do = torch.randn((w.B, w.H, w.l, w.d), generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(w.d)
    _say(f"[causal backward 32K {layout}] running forward + backward")
    dQ, dK, dV = run_gpu(q, k, v, do, w.N, w.rank, layout, scale, dev)
    heads = [(0, 2), (0, 30)]
    q_rows = [0, 63, 64, 2047, 2048, 3000, w.l - 1]
    lq = w.l
    k_rows = [0, 4095, 4096, w.rank * lq, w.rank * lq + 1000, w.rank * lq + lq - 1,
              (w.rank + 1) * lq, w.L - 1]
    _say(f"[causal backward 32K {layout}] oracle and magnitudes on sampled rows")
    bits = [_bits(x) for x in (q, k, v, do)]
    res = oracle.share_backward_rows(*bits, scale, heads, q_rows, k_rows, rank=w.rank, N=w.N,
                                     layout=layout)
    mags = sampled_magnitudes(q, k, v, do, scale, heads, q_rows, k_rows, rank=w.rank, N=w.N,
                              layout=layout)
    for (b, h), (rq, rk, rv), (mq, mk, mv) in zip(heads, res, mags):
        for name, got, ref, mag in (("dQ", dQ[b, h, q_rows], rq, mq),
                                    ("dK", dK[b, h, k_rows], rk, mk),
                                    ("dV", dV[b, h, k_rows], rv, mv)):
            w_ = check(f"32K {layout} head {h} {name}", got, ref, mag)
            _say(f"[causal backward 32K {layout}] head {h} {name}: err/bound {w_:.3f}")
            zero = np.all(ref == 0, axis=1)
            assert np.all(got[zero] == 0), f"head {h} {name}: unseen rows not zero"


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_128k_share_sampled_rows(dev, layout):
    """The 128K / N = 8 causal share the benchmark reports (H = 32, d = 128, rank 3) at full
    size: dQ on query rows at both sides of 256-row tile edges and the ends, dK / dV on key
    rows at both sides of 128-row tile edges, the ends and the edges of the member's own
    block, one head, elementwise within TOL * mag; rows no query of the share sees are
    exactly zero."""
    w = synth.WORKLOADS["share_L128K_N8"]
    q, k, v = synth.draw_workload(w)
    g = torch.Generator().manual_seed(w.seed + 99)
    do = torch.randn((w.B, w.H, w.l, w.d), generator=g).to(torch.bfloat16)
    scale = 1.0 / math.sqrt(w.d)
    _say(f"[causal backward 128K {layout}] running forward + backward")
    dQ, dK, dV = run_gpu(q, k, v, do, w.N, w.rank, layout, scale, dev)
    heads = [(0, 1)]
    q_rows = _tile_edge_rows(w.l, 256)
    lq = w.l
    k_rows = sorted(set(_tile_edge_rows(w.L, 128)) |
                    {w.rank * lq - 1, w.rank * lq, w.rank * lq + lq - 1, (w.rank + 1) * lq})
    _say(f"[causal backward 128K {layout}] oracle and magnitudes on {len(q_rows)} query and "
         f"{len(k_rows)} key rows")
    bits = [_bits(x) for x in (q, k, v, do)]
    res = oracle.share_backward_rows(*bits, scale, heads, q_rows, k_rows, rank=w.rank, N=w.N,
                                     layout=layout)
    mags = sampled_magnitudes(q, k, v, do, scale, heads, q_rows, k_rows, rank=w.rank, N=w.N,
                              layout=layout)
    for (b, h), (rq, rk, rv), (mq, mk, mv) in zip(heads, res, mags):
        for name, got, ref, mag in (("dQ", dQ[b, h, q_rows], rq, mq),
                                    ("dK", dK[b, h, k_rows], rk, mk),
                                    ("dV", dV[b, h, k_rows], rv, mv)):
            w_ = check(f"128K {layout} head {h} {name}", got, ref, mag)
            _say(f"[causal backward 128K {layout}] head {h} {name}: err/bound {w_:.3f}")
            zero = np.all(ref == 0, axis=1)
            assert np.all(got[zero] == 0), f"head {h} {name}: unseen rows not zero"
