"""GPU parity of the HIP path against the fp64 CPU oracle, through the C ABI.

Tolerances:
  fp32 inputs: max |O_gpu - O_ref| <= 1e-5 (the target's own bar).
  bf16 inputs: |O_gpu - O_ref| <= 2e-2 + 1e-2 * |O_ref| elementwise (the target's own bar).
  Row statistics (this build's outputs; no bar is given for them):
    fp32: m and lse = m + ln l to 1e-5 (1 + |x|);
    bf16: per-row bounds derived from the kernel's arithmetic in tests/bounds.py: the
    bf16 rounding of the summed probabilities (2^-8 relative, worst case all one way),
    the fp32 row-sum accumulation, the score error of the matrix instruction (its
    grouped truncation is pinned in tests/test_gpu_accumulation.py), the exponent
    argument's roundings and exp2's error.
  The ring schedule trace must match bit-exactly.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from long_context_exact_ra_amd import ra, synth
from bounds import stat_bounds_bf16

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    ra.load()
    return torch.device("cuda:0")


# ------------------------------------------------------------------ comparison helpers

def check_O(gpu, ref, dtype, what=""):
    gpu = np.asarray(gpu, np.float64)
    err = np.abs(gpu - ref)
    if dtype == "f32":
        assert err.max() <= 1e-5, f"{what}: max abs err {err.max():.3e}"
    else:
        bound = 2e-2 + 1e-2 * np.abs(ref)
        worst = (err / bound).max()
        assert worst <= 1.0, f"{what}: err/bound {worst:.3f}, max abs err {err.max():.3e}"
    return float(err.max())


def check_stats(m_gpu, l_gpu, M, Z, dtype, what="", bounds=None):
    """m and lse = m + ln l against the exact row maximum M and M + ln Z; for bf16,
    `bounds` = (bound_m, bound_lse) per row from stat_bounds_bf16."""
    m_gpu = np.asarray(m_gpu, np.float64)
    lse_gpu = m_gpu + np.log(np.asarray(l_gpu, np.float64))
    lse = M + np.log(Z)
    if dtype == "f32":
        assert np.all(np.abs(m_gpu - M) <= 1e-5 * (1 + np.abs(M))), what
        assert np.all(np.abs(lse_gpu - lse) <= 1e-5 * (1 + np.abs(lse))), what
    else:
        b_m, b_lse = bounds
        em, el = np.abs(m_gpu - M), np.abs(lse_gpu - lse)
        assert np.all(em <= b_m), f"{what}: m err/bound {(em / b_m).max():.3f}"
        assert np.all(el <= b_lse), f"{what}: lse err/bound {(el / b_lse).max():.3f}"
        return float((em / b_m).max()), float((el / b_lse).max())


def dt_name(t):
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def run_share(q, k, v, rank, N, scale):
    B, H, l, d = q.shape
    _, H_kv, L, _ = k.shape
    dev = q.device
    O = torch.empty((B, H, l, d), dtype=torch.float32, device=dev)
    m = torch.empty((B, H, l), dtype=torch.float32, device=dev)
    lo = torch.empty((B, H, l), dtype=torch.float32, device=dev)
    cast = torch.empty((B, H, l, d), dtype=q.dtype, device=dev)
    trace = torch.full((N,), -1, dtype=torch.int32, device=dev)
    ra.share_forward(rank, N, L, H, H_kv, d, B, q, k, v, scale, O, m, lo, cast, trace)
    torch.cuda.synchronize()
    return O, m, lo, cast, trace


def host(*ts):
    return [synth.to_oracle_array(t) for t in ts]


def flat_rows(t, rows):
    B, H, l = t.shape[:3]
    return t.reshape(B * H * l, -1)[rows] if t.dim() == 4 else t.reshape(-1)[rows]


# ------------------------------------------------------------------ tiny fp32 workload

def test_tiny_f32_every_rank(dev):
    w = synth.WORKLOADS["tiny_f32_L256_N4"]
    q, k, v = synth.draw_workload(w)
    scale = 1.0 / math.sqrt(w.d)
    kd, vd = k.to(dev), v.to(dev)
    K, V = host(k, v)
    for rank in range(w.N):
        qi = q[:, :, rank * w.l:(rank + 1) * w.l].contiguous()
        O, m, lo, cast, trace = run_share(qi.to(dev), kd, vd, rank, w.N, scale)
        Or, M, Z = oracle.share(synth.to_oracle_array(qi), K, V, scale, rank, w.N)
        err = check_O(O.cpu().numpy().reshape(Or.shape), Or, "f32", f"rank {rank}")
        check_stats(m.cpu().numpy().ravel(), lo.cpu().numpy().ravel(), M, Z, "f32")
        assert trace.cpu().tolist() == oracle.ring_schedule(rank, w.N)
        assert torch.equal(cast, O)
        _say(f"tiny f32 rank {rank}: max abs err {err:.2e}")


def test_tiny_f32_step_path_every_prefix(dev):
    w = synth.WORKLOADS["tiny_f32_L256_N4"]
    q, k, v = synth.draw_workload(w)
    scale = 1.0 / math.sqrt(w.d)
    kd, vd = k.to(dev), v.to(dev)
    K, V = host(k, v)
    for rank in range(w.N):
        qi = q[:, :, rank * w.l:(rank + 1) * w.l].contiguous()
        Qh = synth.to_oracle_array(qi)
        qd = qi.to(dev)
        O_acc = torch.empty((1, w.H, w.l, w.d), dtype=torch.float32, device=dev)
        m = torch.empty((1, w.H, w.l), dtype=torch.float32, device=dev)
        lsum = torch.empty_like(m)
        ra.state_init(O_acc, m, lsum)
        for t, j in enumerate(ra.ring_schedule(rank, w.N)):
            ra.step(qd, kd[:, :, j * w.l:(j + 1) * w.l], vd[:, :, j * w.l:(j + 1) * w.l],
                    O_acc, m, lsum, scale)
            torch.cuda.synchronize()
            Op, Mp, Zp = oracle.share(Qh, K, V, scale, rank, w.N, steps=t + 1)
            Og = (O_acc / lsum[..., None]).cpu().numpy().reshape(Op.shape)
            check_O(Og, Op, "f32", f"rank {rank} step {t}")
            check_stats(m.cpu().numpy().ravel(), lsum.cpu().numpy().ravel(), Mp, Zp, "f32")
        ra.finalize(O_acc, lsum)
        torch.cuda.synchronize()
        Or, _, _ = oracle.share(Qh, K, V, scale, rank, w.N)
        check_O(O_acc.cpu().numpy().reshape(Or.shape), Or, "f32", "finalized")


# ------------------------------------------------------------------ small bf16 cases

SMALL = [  # B, H, H_kv, d, L, N, rank
    (1, 2, 2, 128, 64, 1, 0),
    (2, 4, 2, 128, 300, 3, 1),      # ragged query tile (100 rows) and key tile (100 keys)
    (1, 2, 1, 128, 3500, 5, 2),     # several query tiles + ragged tails on both axes
    (2, 3, 3, 64, 512, 4, 3),
    (1, 6, 2, 64, 1000, 8, 5),      # 125-row blocks
    (1, 2, 2, 128, 7, 7, 3),        # one key per block, one query row
    (1, 1, 1, 128, 4096, 2, 1),     # two full 2048-key blocks
]


@pytest.mark.parametrize("B,H,H_kv,d,L,N,rank", SMALL)
def test_bf16_share_small(dev, B, H, H_kv, d, L, N, rank):
    l = L // N
    q, k, v = synth.draw(B, H, H_kv, d, l, L, "bf16", seed=100 + L + N)
    scale = 1.0 / math.sqrt(d)
    O, m, lo, cast, trace = run_share(q.to(dev), k.to(dev), v.to(dev), rank, N, scale)
    Q, K, V = host(q, k, v)
    Or, M, Z = oracle.share(Q, K, V, scale, rank, N)
    err = check_O(O.cpu().numpy().reshape(Or.shape), Or, "bf16", "O")
    check_O(cast.float().cpu().numpy().reshape(Or.shape), Or, "bf16", "O_cast")
    assert torch.equal(cast, O.to(torch.bfloat16))
    bnd = stat_bounds_bf16(Q, K, (B, H, H_kv, d, l, L), scale, np.arange(B * H * l), M)
    wm, wl = check_stats(m.cpu().numpy().ravel(), lo.cpu().numpy().ravel(), M, Z, "bf16",
                         bounds=bnd)
    assert trace.cpu().tolist() == oracle.ring_schedule(rank, N)
    _say(f"bf16 {B}x{H}/{H_kv} d{d} L{L} N{N} r{rank}: max abs err {err:.2e}, "
         f"m err/bound {wm:.3f}, lse err/bound {wl:.3f}")


@pytest.mark.parametrize("contiguous_blocks", [False, True])
def test_bf16_step_path_every_prefix(dev, contiguous_blocks):
    B, H, H_kv, d, N, rank, l = 1, 4, 2, 128, 4, 1, 200
    L = N * l
    q, k, v = synth.draw(B, H, H_kv, d, l, L, "bf16", seed=77)
    scale = 1.0 / math.sqrt(d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    Q, K, V = host(q, k, v)
    O_acc = torch.empty((B, H, l, d), dtype=torch.float32, device=dev)
    m = torch.empty((B, H, l), dtype=torch.float32, device=dev)
    lsum = torch.empty_like(m)
    ra.state_init(O_acc, m, lsum)
    for t, j in enumerate(ra.ring_schedule(rank, N)):
        kb, vb = kd[:, :, j * l:(j + 1) * l], vd[:, :, j * l:(j + 1) * l]
        if contiguous_blocks:
            kb, vb = kb.contiguous(), vb.contiguous()
        ra.step(qd, kb, vb, O_acc, m, lsum, scale)
        torch.cuda.synchronize()
        Op, Mp, Zp = oracle.share(Q, K, V, scale, rank, N, steps=t + 1)
        Og = (O_acc / lsum[..., None]).cpu().numpy().reshape(Op.shape)
        check_O(Og, Op, "bf16", f"step {t}")
        bnd = stat_bounds_bf16(Q, K, (B, H, H_kv, d, l, L), scale, np.arange(B * H * l), Mp,
                               n_tiles=(t + 1) * -(-l // 64), n_steps=t + 1)
        check_stats(m.cpu().numpy().ravel(), lsum.cpu().numpy().ravel(), Mp, Zp, "bf16",
                    f"step {t}", bounds=bnd)
    cast = torch.empty((B, H, l, d), dtype=torch.bfloat16, device=dev)
    ra.finalize(O_acc, lsum, O_out=cast)
    torch.cuda.synchronize()
    Or, _, _ = oracle.share(Q, K, V, scale, rank, N)
    check_O(O_acc.cpu().numpy().reshape(Or.shape), Or, "bf16", "finalized")
    assert torch.equal(cast, O_acc.to(torch.bfloat16))


def test_step_resume_is_bitwise(dev):
    """The state (O_acc, m, l) plus the next step index is the whole share state:
    copying it out and continuing gives the same bits as running straight through."""
    B, H, d, N, rank, l = 1, 2, 128, 4, 2, 256
    q, k, v = synth.draw(B, H, H, d, l, N * l, "bf16", seed=78)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    sched = ra.ring_schedule(rank, N)

    def run(stop=None, state=None):
        O_acc = torch.empty((B, H, l, d), dtype=torch.float32, device=dev)
        m = torch.empty((B, H, l), dtype=torch.float32, device=dev)
        s = torch.empty_like(m)
        ra.state_init(O_acc, m, s)
        if state is not None:
            O_acc.copy_(state[0]); m.copy_(state[1]); s.copy_(state[2])
        steps = sched[:stop] if state is None else sched[len(sched) - (N - stop):]
        for j in steps:
            ra.step(qd, kd[:, :, j * l:(j + 1) * l], vd[:, :, j * l:(j + 1) * l], O_acc, m, s, 0.088)
        torch.cuda.synchronize()
        return O_acc, m, s

    full = run(stop=N)
    half = [x.clone() for x in run(stop=2)]
    resumed = run(stop=2, state=half)
    for a, b in zip(full, resumed):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ invariants on the GPU

def test_N_and_rank_independence(dev):
    """Same queries, same sequence: any N and any ring order give the exact answer."""
    B, H, d, L, rows = 1, 2, 128, 1536, 96
    q, k, v = synth.draw(B, H, H, d, rows, L, "bf16", seed=79)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    Q, K, V = host(q, k, v)
    Or, _, _ = oracle.attention_rows(Q, K, V, 1 / math.sqrt(d))
    outs = []
    for N in (1, 2, 3, 4, 6, 8, 12):
        l = L // N
        for rank in sorted({0, N // 2, N - 1}):
            O_acc = torch.empty((B, H, rows, d), dtype=torch.float32, device=dev)
            m = torch.empty((B, H, rows), dtype=torch.float32, device=dev)
            s = torch.empty_like(m)
            ra.state_init(O_acc, m, s)
            for j in ra.ring_schedule(rank, N):
                ra.step(qd, kd[:, :, j * l:(j + 1) * l], vd[:, :, j * l:(j + 1) * l], O_acc, m, s,
                        1 / math.sqrt(d))
            ra.finalize(O_acc, s)
            torch.cuda.synchronize()
            out = O_acc.cpu().numpy().reshape(Or.shape)
            check_O(out, Or, "bf16", f"N={N} rank={rank}")
            outs.append(out)
    spread = max(np.abs(o - outs[0]).max() for o in outs)
    assert spread < 1e-2


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_keys_and_unit_values(dev, dtype):
    B, H, d, L, N = 1, 2, 64, 512, 4
    l = L // N
    q, k, v = synth.draw(B, H, H, d, l, L, dtype, seed=80)
    qd, vd = q.to(dev), v.to(dev)
    O, *_ = run_share(qd, torch.zeros_like(k).to(dev), vd, 1, N, 0.125)
    mean = v.double().mean(dim=2, keepdim=True).expand(B, H, l, d)
    tol = 1e-5 if dtype == "f32" else 2e-2
    assert (O.cpu().double() - mean).abs().max() <= tol
    O1, *_ = run_share(qd, k.to(dev), torch.ones_like(v).to(dev), 2, N, 0.125)
    assert (O1.cpu().double() - 1).abs().max() <= (1e-5 if dtype == "f32" else 1e-2)


def test_gqa_equals_repeated_kv_mha_bitwise(dev):
    B, H, H_kv, d, L, N = 1, 6, 2, 128, 768, 3
    l = L // N
    q, k, v = synth.draw(B, H, H_kv, d, l, L, "bf16", seed=81)
    qd = q.to(dev)
    O1, *_ = run_share(qd, k.to(dev), v.to(dev), 0, N, 0.088)
    kr = k.repeat_interleave(H // H_kv, dim=1).contiguous().to(dev)
    vr = v.repeat_interleave(H // H_kv, dim=1).contiguous().to(dev)
    O2, *_ = run_share(qd, kr, vr, 0, N, 0.088)
    assert torch.equal(O1, O2)


def test_repeated_runs_are_bitwise_equal(dev):
    B, H, d, L, N = 1, 4, 128, 8192, 4
    q, k, v = synth.draw(B, H, H, d, L // N, L, "bf16", seed=82)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    first = run_share(qd, kd, vd, 1, N, 0.088)[0].clone()
    for _ in range(4):
        assert torch.equal(run_share(qd, kd, vd, 1, N, 0.088)[0], first)


def test_empty_inputs_are_noops(dev):
    q = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    O = torch.zeros((1, 2, 0, 128), dtype=torch.float32, device=dev)
    # L = 0: nothing to do; the binding hands the library empty tensors
    ra.share_forward(0, 4, 0, 2, 2, 128, 1, q, k, k, 0.088, O)
    qq, kk, vv = synth.draw(1, 2, 2, 128, 16, 64, "bf16", seed=83)
    qd = qq.to(dev)
    O_acc = torch.empty((1, 2, 16, 128), dtype=torch.float32, device=dev)
    m = torch.empty((1, 2, 16), dtype=torch.float32, device=dev)
    s = torch.empty_like(m)
    ra.state_init(O_acc, m, s)
    ra.step(qd, kk.to(dev), vv.to(dev), O_acc, m, s, 0.088)
    before = [x.clone() for x in (O_acc, m, s)]
    empty = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device=dev)
    ra.step(qd, empty, empty, O_acc, m, s, 0.088)
    torch.cuda.synchronize()
    for a, b in zip(before, (O_acc, m, s)):
        assert torch.equal(a, b)


# ------------------------------------------------------------------ full-size workloads

FULL = ["share_L32K_N8", "share_L128K_N8", "gqa_L128K_N8_28q4kv", "share_L1M_N64_std3"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_sampled_rows(dev, name):
    """The launch the benchmark times, at full size, against the oracle on at least 4096
    rows: in every head the first and last row and both sides of every 256-row query-tile
    boundary, topped up with seeded random rows."""
    w = synth.WORKLOADS[name]
    _say(f"[{name}] drawing inputs")
    q, k, v = synth.draw_workload(w)
    scale = 1.0 / math.sqrt(w.d)
    _say(f"[{name}] running share rank {w.rank} of {w.N}")
    O, m, lo, cast, trace = run_share(q.to(dev), k.to(dev), v.to(dev), w.rank, w.N, scale)
    assert trace.cpu().tolist() == oracle.ring_schedule(w.rank, w.N)
    assert torch.isfinite(O).all()
    rows = synth.boundary_rows(w.B, w.H, w.l, 4096, w.seed)
    Q, K, V = host(q, k, v)
    Og, cg = flat_rows(O, rows).cpu().numpy(), flat_rows(cast, rows).float().cpu().numpy()
    mg, lg = flat_rows(m, rows).cpu().numpy(), flat_rows(lo, rows).cpu().numpy()
    worst = [0.0, 0.0, 0.0]
    for i0 in range(0, len(rows), 1024):
        part = rows[i0:i0 + 1024]
        _say(f"[{name}] oracle on rows {i0}..{i0 + len(part) - 1} of {len(rows)}")
        Or, M, Z = oracle.share(Q, K, V, scale, w.rank, w.N, rows=part)
        sl = slice(i0, i0 + len(part))
        err = check_O(Og[sl], Or, "bf16", name)
        check_O(cg[sl], Or, "bf16", name + " cast")
        bnd = stat_bounds_bf16(Q, K, (w.B, w.H, w.H_kv, w.d, w.l, w.L), scale, part, M)
        wm, wl = check_stats(mg[sl], lg[sl], M, Z, "bf16", name, bounds=bnd)
        worst = [max(worst[0], err), max(worst[1], wm), max(worst[2], wl)]
    _say(f"[{name}] {len(rows)} rows: max abs err {worst[0]:.2e}, m err/bound "
         f"{worst[1]:.3f}, lse err/bound {worst[2]:.3f}")


def test_full_size_step_path_sampled_rows(dev):
    """The per-step path the benchmark also times on the 128K share (N ra_step calls over
    views of the resident K/V in ring order, then ra_finalize), at full size, against the
    oracle on every head's first and last row and both sides of every 256-row query-tile
    boundary (4096 rows)."""
    w = synth.WORKLOADS["share_L128K_N8"]
    _say("[step path 128K] drawing inputs")
    q, k, v = synth.draw_workload(w)
    scale = 1.0 / math.sqrt(w.d)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    O_acc = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.float32, device=dev)
    m = torch.empty((w.B, w.H, w.l), dtype=torch.float32, device=dev)
    lsum = torch.empty_like(m)
    _say(f"[step path 128K] {w.N} steps of rank {w.rank}, then finalize")
    ra.state_init(O_acc, m, lsum)
    for j in ra.ring_schedule(w.rank, w.N):
        ra.step(qd, kd[:, :, j * w.l:(j + 1) * w.l], vd[:, :, j * w.l:(j + 1) * w.l], O_acc, m,
                lsum, scale)
    cast = torch.empty((w.B, w.H, w.l, w.d), dtype=torch.bfloat16, device=dev)
    ra.finalize(O_acc, lsum, O_out=cast)
    torch.cuda.synchronize()
    assert torch.isfinite(O_acc).all()
    assert torch.equal(cast, O_acc.to(torch.bfloat16))
    rows = synth.boundary_rows(w.B, w.H, w.l, 0, w.seed)
    Q, K, V = host(q, k, v)
    Og = flat_rows(O_acc, rows).cpu().numpy()
    mg, lg = flat_rows(m, rows).cpu().numpy(), flat_rows(lsum, rows).cpu().numpy()
    worst = [0.0, 0.0, 0.0]
    for i0 in range(0, len(rows), 1024):
        part = rows[i0:i0 + 1024]
        _say(f"[step path 128K] oracle on rows {i0}..{i0 + len(part) - 1} of {len(rows)}")
        Or, M, Z = oracle.share(Q, K, V, scale, w.rank, w.N, rows=part)
        sl = slice(i0, i0 + len(part))
        err = check_O(Og[sl], Or, "bf16", "step path 128K")
        bnd = stat_bounds_bf16(Q, K, (w.B, w.H, w.H_kv, w.d, w.l, w.L), scale, part, M,
                               n_tiles=w.N * -(-w.l // 64), n_steps=w.N)
        wm, wl = check_stats(mg[sl], lg[sl], M, Z, "bf16", "step path 128K", bounds=bnd)
        worst = [max(worst[0], err), max(worst[1], wm), max(worst[2], wl)]
    _say(f"[step path 128K] {len(rows)} rows: max abs err {worst[0]:.2e}, m err/bound "
         f"{worst[1]:.3f}, lse err/bound {worst[2]:.3f}")


def test_largest_head_range(dev):
    """The largest key range one head may span: 2^23 - 1 keys of d = 128 bf16 are 2^31 - 256
    bytes, the edge of the kernel's 32-bit buffer range (one key more is RA_ENOTSUP, checked
    on the CPU).  N = 47 blocks of 178481 rows, so query tiles and key tiles are both ragged;
    one head, rank 23; sampled rows (tile edges, both ends) against the oracle."""
    B, H, H_kv, d, N, rank = 1, 1, 1, 128, 47, 23
    L = (1 << 23) - 1
    l = L // N
    assert l * N == L and l % 64 != 0 and l % 256 != 0
    _say("[largest head range] drawing inputs")
    q, k, v = synth.draw(B, H, H_kv, d, l, L, "bf16", 1010)
    scale = 1.0 / math.sqrt(d)
    _say(f"[largest head range] running share rank {rank} of {N}, L = {L}")
    O, m, lo, cast, trace = run_share(q.to(dev), k.to(dev), v.to(dev), rank, N, scale)
    assert trace.cpu().tolist() == oracle.ring_schedule(rank, N)
    assert torch.isfinite(O).all()
    rows = sorted({0, 1, 255, 256, 12345, 65535, 65536, l // 2, l - 257, l - 256, l - 2, l - 1})
    Q, K, V = host(q, k, v)
    _say(f"[largest head range] oracle on {len(rows)} rows")
    Or, M, Z = oracle.share(Q, K, V, scale, rank, N, rows=rows)
    err = check_O(flat_rows(O, rows).cpu().numpy(), Or, "bf16", "largest head range")
    check_O(flat_rows(cast, rows).float().cpu().numpy(), Or, "bf16", "largest head range cast")
    bnd = stat_bounds_bf16(Q, K, (B, H, H_kv, d, l, L), scale, rows, M)
    wm, wl = check_stats(flat_rows(m, rows).cpu().numpy(), flat_rows(lo, rows).cpu().numpy(), M,
                         Z, "bf16", "largest head range", bounds=bnd)
    _say(f"[largest head range] max abs err {err:.2e}, m err/bound {wm:.3f}, "
         f"lse err/bound {wl:.3f}")


def test_share_32k_every_row(dev):
    """The 32K share (4096 query rows of each of 32 heads against 32768 keys) against the
    oracle on every row, not a sample: O, its bf16 cast and the row statistics.  The
    oracle runs in chunks of four heads (about 5 s each on 16 host threads)."""
    w = synth.WORKLOADS["share_L32K_N8"]
    _say("[32K every row] drawing inputs")
    q, k, v = synth.draw_workload(w)
    scale = 1.0 / math.sqrt(w.d)
    O, m, lo, cast, trace = run_share(q.to(dev), k.to(dev), v.to(dev), w.rank, w.N, scale)
    assert trace.cpu().tolist() == oracle.ring_schedule(w.rank, w.N)
    assert torch.isfinite(O).all()
    Q, K, V = host(q, k, v)
    Og = O.reshape(-1, w.d).cpu().numpy()
    cg = cast.reshape(-1, w.d).float().cpu().numpy()
    mg, lg = m.reshape(-1).cpu().numpy(), lo.reshape(-1).cpu().numpy()
    n, chunk = w.B * w.H * w.l, 4 * w.l
    worst = 0.0
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk), dtype=np.int64)
        Or, M, Z = oracle.share(Q, K, V, scale, w.rank, w.N, rows=rows)
        err = check_O(Og[rows], Or, "bf16", f"32K rows {r0}+")
        check_O(cg[rows], Or, "bf16", f"32K cast rows {r0}+")
        bnd = stat_bounds_bf16(Q, K, (w.B, w.H, w.H_kv, w.d, w.l, w.L), scale, rows, M)
        check_stats(mg[rows], lg[rows], M, Z, "bf16", f"32K rows {r0}+", bounds=bnd)
        worst = max(worst, err)
        _say(f"[32K every row] rows {r0}..{r0 + len(rows) - 1}: max abs err {err:.2e}")
    _say(f"[32K every row] all {n} rows: max abs err {worst:.2e}")
