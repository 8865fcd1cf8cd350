"""GPU parity of the causal share (ra_causal_share_forward) against the fp64 oracle.

A query attends only to keys at or before its own sequence position (slowleelab "Ring
Attention" page, 4.5 limitation 2), with tokens assigned to ring members contiguously,
striped (4.8) or zigzag.  K and V are member-major: rows j*l .. (j+1)*l - 1 hold member
j's tokens.  Tolerances are those of the non-causal share (test_gpu_parity.py).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_ra_amd import ra, synth
from bounds import stat_bounds_bf16
from test_gpu_parity import _say, check_O, check_stats, flat_rows, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ra.load()
    return torch.device("cuda:0")


def run_causal(q, k, v, rank, N, layout, scale):
    B, H, l, d = q.shape
    _, H_kv, L, _ = k.shape
    dev = q.device
    O = torch.full((B, H, l, d), float("nan"), dtype=torch.float32, device=dev)
    m = torch.full((B, H, l), float("nan"), dtype=torch.float32, device=dev)
    lo = torch.full((B, H, l), float("nan"), dtype=torch.float32, device=dev)
    cast = torch.empty((B, H, l, d), dtype=q.dtype, device=dev)
    ra.causal_share_forward(rank, N, L, H, H_kv, d, B, layout, q, k, v, scale, O, m, lo, cast)
    torch.cuda.synchronize()
    return O, m, lo, cast


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_f32_every_rank(dev, layout):
    B, H, H_kv, d, N, l = 1, 2, 2, 64, 4, 128
    q, k, v = synth.draw(B, H, H_kv, d, N * l, N * l, "f32", 2001)
    scale = 1.0 / math.sqrt(d)
    kd, vd = k.to(dev), v.to(dev)
    K, V = host(k, v)
    for rank in range(N):
        qi = q[:, :, rank * l:(rank + 1) * l].contiguous()
        O, m, lo, cast = run_causal(qi.to(dev), kd, vd, rank, N, layout, scale)
        Or, M, Z = oracle.causal_share(synth.to_oracle_array(qi), K, V, scale, rank, N, layout)
        err = check_O(O.cpu().numpy().reshape(Or.shape), Or, "f32", f"{layout} rank {rank}")
        check_stats(m.cpu().numpy().ravel(), lo.cpu().numpy().ravel(), M, Z, "f32")
        assert torch.equal(cast, O)
        _say(f"causal f32 {layout} rank {rank}: max abs err {err:.2e}")


# (B, H, H_kv, d, N, l): several query tiles, ragged tails, GQA, both head sizes
BF16_CASES = [
    (2, 4, 2, 128, 3, 384),
    (1, 2, 1, 64, 5, 256),
    (1, 3, 3, 128, 4, 300),   # ragged: not a multiple of 64 or 256 (no zigzag)
    (1, 2, 2, 128, 2, 1024),
    (1, 2, 2, 128, 1, 640),   # a single member: plain causal attention
    (1, 2, 1, 128, 3, 5),     # blocks of 5 keys: one ragged tile per block (no zigzag)
]


@pytest.mark.parametrize("case", BF16_CASES, ids=lambda c: "x".join(map(str, c)))
@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_bf16_small_every_rank(dev, layout, case):
    B, H, H_kv, d, N, l = case
    if layout == "zigzag" and l % 128:
        pytest.skip("zigzag needs whole 64-key tiles in each half-block")
    q, k, v = synth.draw(B, H, H_kv, d, N * l, N * l, "bf16", 3000 + l + N)
    scale = 1.0 / math.sqrt(d)
    kd, vd = k.to(dev), v.to(dev)
    K, V = host(k, v)
    for rank in sorted({0, N // 2, N - 1}):
        qi = q[:, :, rank * l:(rank + 1) * l].contiguous()
        O, m, lo, cast = run_causal(qi.to(dev), kd, vd, rank, N, layout, scale)
        Or, M, Z = oracle.causal_share(synth.to_oracle_array(qi), K, V, scale, rank, N, layout)
        what = f"{layout} {case} rank {rank}"
        err = check_O(O.cpu().numpy().reshape(Or.shape), Or, "bf16", what)
        check_O(cast.float().cpu().numpy().reshape(Or.shape), Or, "bf16", what + " cast")
        Qh = synth.to_oracle_array(qi)
        bnd = stat_bounds_bf16(Qh, K, (B, H, H_kv, d, l, N * l), scale, np.arange(B * H * l), M)
        check_stats(m.cpu().numpy().ravel(), lo.cpu().numpy().ravel(), M, Z, "bf16", what,
                    bounds=bnd)
        _say(f"causal bf16 {what}: max abs err {err:.2e}")


def test_single_member_causal_equals_both_layouts(dev):
    """With N = 1 the contiguous and striped layouts are the same sequence order."""
    B, H, d, l = 1, 2, 128, 512
    q, k, v = synth.draw(B, H, H, d, l, l, "bf16", 4001)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O1 = run_causal(qd, kd, vd, 0, 1, "contiguous", 0.1)[0]
    O2 = run_causal(qd, kd, vd, 0, 1, "striped", 0.1)[0]
    assert torch.equal(O1, O2)


@pytest.mark.parametrize("layout", ["contiguous", "striped", "zigzag"])
def test_full_size_causal_sampled_rows(dev, layout):
    """The 128K / N = 8 share with a causal mask, at full size, rank 3 and the last rank."""
    w = synth.WORKLOADS["share_L128K_N8"]
    q, k, v = synth.draw_workload(w)
    scale = 1.0 / math.sqrt(w.d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    Q, K, V = host(q, k, v)
    for rank in (w.rank, w.N - 1):
        _say(f"[causal {layout}] rank {rank} of {w.N}")
        O, m, lo, cast = run_causal(qd, kd, vd, rank, w.N, layout, scale)
        rows = synth.sample_rows(w.B, w.H, w.l, 8, w.seed + rank)
        Or, M, Z = oracle.causal_share(Q, K, V, scale, rank, w.N, layout, rows=rows)
        err = check_O(flat_rows(O, rows).cpu().numpy(), Or, "bf16", f"{layout} rank {rank}")
        bnd = stat_bounds_bf16(Q, K, (w.B, w.H, w.H_kv, w.d, w.l, w.L), scale, rows, M)
        check_stats(flat_rows(m, rows).cpu().numpy(), flat_rows(lo, rows).cpu().numpy(), M, Z,
                    "bf16", f"{layout} rank {rank}", bounds=bnd)
        assert torch.isfinite(O).all()
        _say(f"[causal {layout}] rank {rank}: max abs err {err:.2e} over {len(rows)} rows")
