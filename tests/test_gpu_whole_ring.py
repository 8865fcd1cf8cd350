"""The whole ring on one GPU: the N members' shares together against plain attention over
the sequence in its own order.

A ring of N members splits one sequence of L tokens. Member i keeps its query block and
meets every key/value block in ring order (slowleelab "Ring Attention" page, 4.2 and 4.3).
So the N shares together are attention over the whole sequence. In the backward pass, each
member adds its part into the key/value gradients that travel with the blocks (aliyun
FlashAttention explainer, section 2: recomputation from the stored statistics).

Here the members run one after another on one GPU, all adding into one dK / dV pair. Their
rows, put back into sequence order, are compared with the oracle's single-member result
(N = 1) on the sequence-ordered inputs. The CPU tests pin that result to torch's
scaled-dot-product attention and its autograd. For a causal share, the tokens are first
given to members by the layout (contiguous, striped or zigzag). That checks the kernels'
position maps against the true order of the sequence, not only against the oracle's own
layout code.

Bounds: the forward uses the share's own bf16 bounds (test_gpu_parity.py). The backward
uses the magnitude bound of test_gpu_backward.py over the whole sequence. Each member's
part of a key gradient stays within 2^-6 of its own magnitude sum, and those sums add up
to the whole sequence's; the absolute floor grows to N * 1e-6.

The FP8 causal share gets the same check against exact causal attention over the
dequantized values in sequence order, within each member's own FP8 bound.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8 as ofp8
from long_context_exact_ra_amd import ra, synth
from test_gpu_backward import TOL, _bits, _draw, magnitudes
from test_gpu_causal_backward import masked_magnitudes
from test_gpu_fp8 import run_fp8_share
from bounds import stat_bounds_bf16
from test_gpu_parity import _say, check_O, check_stats

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ra.load()
    return torch.device("cuda:0")


def run_ring(q, k, v, do, N, layout, scale, dev):
    """Every member's forward and backward, inputs and outputs member-major [.., L, ..]."""
    B, H, L, d = q.shape
    H_kv = k.shape[1]
    l = L // N
    kd, vd = k.to(dev), v.to(dev)
    O = torch.empty((B, H, L, d), dtype=torch.float32)
    m = torch.empty((B, H, L), dtype=torch.float32)
    lo = torch.empty_like(m)
    dQ = torch.empty_like(O)
    dK = torch.zeros((B, H_kv, L, d), dtype=torch.float32, device=dev)
    dV = torch.zeros_like(dK)
    for rank in range(N):
        rows = slice(rank * l, (rank + 1) * l)
        qi = q[:, :, rows].contiguous().to(dev)
        doi = do[:, :, rows].contiguous().to(dev)
        Oi = torch.empty((B, H, l, d), dtype=torch.float32, device=dev)
        mi = torch.empty((B, H, l), dtype=torch.float32, device=dev)
        li = torch.empty_like(mi)
        dQi = torch.full_like(Oi, float("nan"))
        if layout is None:
            ra.share_forward(rank, N, L, H, H_kv, d, B, qi, kd, vd, scale, Oi, mi, li)
            ra.share_backward(rank, N, L, H, H_kv, d, B, qi, kd, vd, Oi, doi, mi, li, scale,
                              dQi, dK, dV)
        else:
            ra.causal_share_forward(rank, N, L, H, H_kv, d, B, layout, qi, kd, vd, scale, Oi,
                                    mi, li)
            ra.causal_share_backward(rank, N, L, H, H_kv, d, B, layout, qi, kd, vd, Oi, doi,
                                     mi, li, scale, dQi, dK, dV)
        torch.cuda.synchronize()
        O[:, :, rows], m[:, :, rows], lo[:, :, rows] = Oi.cpu(), mi.cpu(), li.cpu()
        dQ[:, :, rows] = dQi.cpu()
    return [x.numpy() for x in (O, m, lo, dQ, dK.cpu(), dV.cpu())]


# (layout, B, H, H_kv, d, N, l): None is the non-causal share; ragged blocks (300, 200),
# GQA, both head sizes
CASES = [
    (None, 1, 2, 1, 128, 4, 256),
    (None, 2, 2, 2, 64, 3, 300),
    ("contiguous", 1, 2, 2, 128, 4, 256),
    ("contiguous", 1, 4, 2, 64, 3, 200),
    ("striped", 1, 2, 1, 128, 4, 256),
    ("striped", 2, 2, 2, 64, 3, 200),
    ("zigzag", 1, 2, 2, 128, 4, 256),
    ("zigzag", 1, 4, 2, 64, 2, 384),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_members_together_are_the_whole_sequence(dev, case):
    layout, B, H, H_kv, d, N, l = case
    L = N * l
    scale = 1.0 / math.sqrt(d)
    # the sequence in its own order, then given to members by the layout
    q, k, v, do = _draw(B, H, H_kv, d, L, L, 7000 + l + N, std=1.0)
    pos = oracle.layout_positions(layout or "contiguous", N, L)
    take = torch.from_numpy(pos)
    qm, km, vm, dom = (x[:, :, take].contiguous() for x in (q, k, v, do))
    O, m, lo, dQ, dK, dV = run_ring(qm, km, vm, dom, N, layout, scale, dev)
    back = np.argsort(pos)  # member-major row of each sequence position
    O, m, lo, dQ, dK, dV = (x[:, :, back] for x in (O, m, lo, dQ, dK, dV))

    # plain attention over the sequence order: one member, no ring
    Qs, Ks, Vs, dOs = (_bits(x) for x in (q, k, v, do))
    if layout is None:
        Or, M, Z = oracle.share(Qs, Ks, Vs, scale, 0, 1)
        mq, mk, mv = magnitudes(q, k, v, do, scale)
    else:
        Or, M, Z = oracle.causal_share(Qs, Ks, Vs, scale, 0, 1, "contiguous")
        mq, mk, mv, _ = masked_magnitudes(q, k, v, do, scale, 0, 1, "contiguous")
    rQ, rK, rV = oracle.share_backward(Qs, Ks, Vs, dOs, scale, 0, 1,
                                       None if layout is None else "contiguous")
    what = f"{layout or 'full'} {case[1:]}"
    err = check_O(O.reshape(Or.shape), Or, "bf16", what)
    bnd = stat_bounds_bf16(Qs, Ks, (B, H, H_kv, d, L, L), scale, np.arange(B * H * L), M,
                           n_tiles=N * -(-l // 64))
    check_stats(m.ravel(), lo.ravel(), M, Z, "bf16", what, bounds=bnd)
    worst = {}
    for name, got, ref, mag in (("dQ", dQ, rQ, mq), ("dK", dK, rK, mk), ("dV", dV, rV, mv)):
        assert np.isfinite(got).all(), f"{what} {name}: non-finite values"
        w = (np.abs(got - ref) / (TOL * mag + N * 1e-6)).max()
        assert w <= 1.0, f"{what} {name}: err/bound {w:.3f}"
        worst[name] = w
    _say(f"whole ring {what}: O max abs err {err:.2e}; worst err/bound dQ {worst['dQ']:.3f} "
         f"dK {worst['dK']:.3f} dV {worst['dV']:.3f}")


# ------------------------------------------------------------------ FP8 causal share

# (layout, B, H, H_kv, d, N, l): GQA, both head sizes, a ragged striped block
FP8_CASES = [
    ("contiguous", 1, 2, 1, 128, 3, 256),
    ("striped", 1, 2, 2, 64, 4, 200),
    ("zigzag", 1, 2, 2, 128, 4, 256),
    ("zigzag", 2, 2, 1, 64, 2, 384),
]


@pytest.mark.parametrize("case", FP8_CASES, ids=lambda c: "x".join(map(str, c)))
def test_fp8_causal_members_together_are_the_whole_sequence(dev, case):
    """Every member's FP8 causal share (GPU quantization and kernel) against exact causal
    attention over the dequantized values of the whole sequence in its own order (one
    member, no layout). The allowed deviation is the FP8 share's own bound
    (oracle.fp8.error_bounds, which measures from that exact attention), per member."""
    layout, B, H, H_kv, d, N, l = case
    L = N * l
    scale = 1.0 / math.sqrt(d)
    q, k, v = synth.draw(B, H, H_kv, d, L, L, "bf16", 7500 + l + N)
    pos = oracle.layout_positions(layout, N, L)
    take = torch.from_numpy(pos)
    qm, km, vm = (x[:, :, take].contiguous() for x in (q, k, v))
    O = np.empty((B, H, L, d))
    Qd = np.empty((B, H, L, d))
    for rank in range(N):
        rows = slice(rank * l, (rank + 1) * l)
        qr = qm[:, :, rows].contiguous()
        (Or, _, _, _), _ = run_fp8_share(qr, km, vm, N, rank, scale, dev, layout=layout)
        O[:, :, rows] = Or.double().cpu().numpy()
        q8, qs = ofp8.quantize_rows(_bits(qr), 1, l)
        Qd[:, :, rows] = ofp8.dequantize_rows(q8, qs, l)
    k8, ks = ofp8.quantize_rows(_bits(km), N, l)
    v8, vs = ofp8.quantize_vt(_bits(vm), N, l)
    Kd, Vd = ofp8.dequantize_rows(k8, ks, l), ofp8.dequantize_vt(v8, vs, l)
    back = np.argsort(pos)
    ref, _, _ = oracle.causal_share(Qd[:, :, back], Kd[:, :, back], Vd[:, :, back], scale, 0, 1,
                                    "contiguous")
    ref = ref.reshape(B, H, L, d)[:, :, pos]  # member-major rows
    worst = 0.0
    for rank in range(N):
        rows = slice(rank * l, (rank + 1) * l)
        ref_r = ref[:, :, rows].reshape(-1, d)
        bound, _, _ = ofp8.error_bounds(Qd[:, :, rows], Kd, Vd, scale, rank, N, ref_r,
                                        np.arange(B * H * l), layout=layout)
        got = O[:, :, rows].reshape(-1, d)
        assert np.isfinite(got).all()
        w = (np.abs(got - ref_r) / bound).max()
        assert w <= 1.0, f"fp8 {case} rank {rank}: err/bound {w:.3f}"
        worst = max(worst, w)
    _say(f"whole ring fp8 {case}: worst O err/bound {worst:.3f}")
