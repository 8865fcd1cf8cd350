"""Pins of the CPU oracle to facts fixed by the pages and by mathematics.

None of these re-types the oracle's formula: each compares it with a value printed on
the pages (the N = 4 ring table), an independent simulation of the ring described on
the pages, a closed form, an invariant of exact attention, or torch's own fp64
scaled-dot-product attention (a library routine the oracle does not call).
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from long_context_exact_ra_amd import synth


def _rand(shape, seed, scale=1.0):
    return (np.random.default_rng(seed).standard_normal(shape) * scale).astype(np.float32)


def _sdpa(Q, K, V, scale):
    """torch fp64 SDPA on the CPU, K/V heads repeated for grouped-query attention."""
    H, H_kv = Q.shape[1], K.shape[1]
    q = torch.from_numpy(np.asarray(Q, np.float64))
    k = torch.from_numpy(np.asarray(K, np.float64)).repeat_interleave(H // H_kv, dim=1)
    v = torch.from_numpy(np.asarray(V, np.float64)).repeat_interleave(H // H_kv, dim=1)
    return F.scaled_dot_product_attention(q, k, v, scale=scale).numpy()


# ---------------------------------------------------------------- ring schedule

def _read_golden(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "ring_schedule_n4.txt")) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(tuple(int(x) for x in line.split()))
    return rows


def test_schedule_matches_printed_n4_table(golden_dir):
    rows = _read_golden(golden_dir)
    assert len(rows) == 8
    for step, gpu, block, send_to in rows:
        assert oracle.ring_schedule(gpu, 4)[step] == block
        assert send_to == (gpu + 1) % 4
        # the block passed on at step t is the one the receiver uses at step t+1
        if step + 1 < 4:
            assert oracle.ring_schedule(send_to, 4)[step + 1] == block


@pytest.mark.parametrize("N", [1, 2, 3, 4, 5, 7, 8, 64])
def test_schedule_is_a_ring_rotation(N):
    table = [oracle.ring_schedule(i, N) for i in range(N)]
    for i in range(N):
        assert table[i][0] == i                      # step 0 uses the local block
        assert sorted(table[i]) == list(range(N))    # every block exactly once
        for t in range(N - 1):
            assert table[i][t + 1] == table[(i - 1) % N][t]   # received from i-1
    for t in range(N):
        assert sorted(table[i][t] for i in range(N)) == list(range(N))


@pytest.mark.parametrize("N", [1, 2, 4, 5, 8, 64])
def test_schedule_equals_message_passing_simulation(N):
    """Simulate the ring as the slowleelab page describes it (each GPU starts with its
    own block; after computing it passes the block it holds to GPU i+1) and compare
    the blocks each GPU computes with against the oracle's schedule."""
    holding = list(range(N))
    used = [[] for _ in range(N)]
    sends = [0] * N
    for t in range(N):
        for i in range(N):
            used[i].append(holding[i])
        if t == N - 1:
            break                                     # nothing left to pass on
        new = [None] * N
        for i in range(N):
            new[(i + 1) % N] = holding[i]
            sends[i] += 1
        holding = new
    for i in range(N):
        assert used[i] == oracle.ring_schedule(i, N)
        assert sends[i] == N - 1


def test_kv_head_contiguous_groups():
    # The grouping of grouped-query attention as torch applies it (each K/V head repeated
    # for H / H_kv consecutive query heads, repeat_interleave), for every divisor pair.
    for H in (1, 2, 6, 8, 28, 32, 64):
        for H_kv in (g for g in range(1, H + 1) if H % g == 0):
            want = torch.arange(H_kv).repeat_interleave(H // H_kv).tolist()
            assert [oracle.kv_head(h, H, H_kv) for h in range(H)] == want, (H, H_kv)
    assert [oracle.kv_head(h, 28, 4) for h in range(28)] == [h // 7 for h in range(28)]
    assert [oracle.kv_head(h, 8, 8) for h in range(8)] == list(range(8))
    assert [oracle.kv_head(h, 8, 1) for h in range(8)] == [0] * 8
    with pytest.raises(ValueError):
        oracle.kv_head(0, 6, 4)


# ---------------------------------------------------------------- library routine

@pytest.mark.parametrize("H,H_kv", [(4, 4), (4, 2), (6, 1)])
def test_oracle_equals_torch_sdpa_fp64(H, H_kv):
    B, l_q, L, d = 2, 7, 40, 16
    Q, K, V = _rand((B, H, l_q, d), 1), _rand((B, H_kv, L, d), 2), _rand((B, H_kv, L, d), 3)
    scale = 0.37
    O, _, _ = oracle.attention_rows(Q, K, V, scale)
    ref = _sdpa(Q, K, V, scale)
    np.testing.assert_allclose(O.reshape(ref.shape), ref, rtol=0, atol=1e-13)


def test_default_scale_is_inverse_sqrt_head_dim():
    """SDPA's default scale is 1/sqrt(head dim): the reading of sqrt(d) as the head
    dimension (not the model width) must reproduce it."""
    B, H, l_q, L, d = 1, 2, 5, 33, 64
    Q, K, V = _rand((B, H, l_q, d), 4), _rand((B, H, L, d), 5), _rand((B, H, L, d), 6)
    O, _, _ = oracle.attention_rows(Q, K, V, 1.0 / math.sqrt(d))
    ref = F.scaled_dot_product_attention(*(torch.from_numpy(x).double() for x in (Q, K, V)))
    np.testing.assert_allclose(O.reshape(ref.shape), ref.numpy(), atol=1e-13)


def test_large_logits_match_sdpa():
    """Q and K with std 3 and d = 128 give logits of std ~9 (the million-token
    workload's distribution); without the max shift exp would overflow."""
    B, H, l_q, L, d = 1, 1, 6, 4096, 128
    Q, K, V = _rand((B, H, l_q, d), 7, 3.0), _rand((B, H, L, d), 8, 3.0), _rand((B, H, L, d), 9)
    O, M, Z = oracle.attention_rows(Q, K, V, 1.0 / math.sqrt(d))
    ref = _sdpa(Q, K, V, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(O.reshape(ref.shape), ref, atol=1e-12)
    assert np.all(Z >= 1.0)


# ---------------------------------------------------------------- closed forms

def test_zero_keys_give_mean_of_values():
    B, H, l_q, L, d = 1, 2, 4, 50, 8
    Q, V = _rand((B, H, l_q, d), 10), _rand((B, H, L, d), 11)
    K = np.zeros((B, H, L, d), np.float32)
    O, M, Z = oracle.attention_rows(Q, K, V, 0.5)
    mean = V.astype(np.float64).mean(axis=2)           # [B, H, d]
    np.testing.assert_allclose(O.reshape(B, H, l_q, d), np.repeat(mean[:, :, None], l_q, 2),
                               atol=1e-14)
    assert np.all(M == 0.0) and np.allclose(Z, L)


def test_unit_values_give_ones():
    B, H, l_q, L, d = 1, 2, 5, 64, 16
    Q, K = _rand((B, H, l_q, d), 12, 3.0), _rand((B, H, L, d), 13, 3.0)
    V = np.ones((B, H, L, d), np.float32)
    O, _, _ = oracle.attention_rows(Q, K, V, 0.25)
    np.testing.assert_allclose(O, 1.0, atol=1e-14)


def test_single_key_returns_its_value():
    Q, K, V = _rand((1, 1, 3, 8), 14), _rand((1, 1, 1, 8), 15), _rand((1, 1, 1, 8), 16)
    O, M, Z = oracle.attention_rows(Q, K, V, 0.3)
    np.testing.assert_allclose(O, np.repeat(V[0, 0].astype(np.float64), 3, 0), atol=0)
    s = 0.3 * Q[0, 0].astype(np.float64) @ K[0, 0, 0].astype(np.float64)
    np.testing.assert_allclose(M, s, rtol=1e-15)
    assert np.all(Z == 1.0)


def test_two_keys_scalar_closed_form():
    """d = 1, two keys: weights are the logistic function of the score difference."""
    q, k0, k1, v0, v1, sc = 0.75, -1.25, 2.0, 3.0, -5.0, 0.5
    Q = np.array([[[[q]]]], np.float32)
    K = np.array([[[[k0], [k1]]]], np.float32)
    V = np.array([[[[v0], [v1]]]], np.float32)
    O, M, Z = oracle.attention_rows(Q, K, V, sc)
    s0, s1 = sc * q * k0, sc * q * k1
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    assert O[0, 0] == pytest.approx(w0 * v0 + (1 - w0) * v1, abs=1e-15)
    assert M[0] == pytest.approx(max(s0, s1), abs=1e-16)
    assert Z[0] == pytest.approx(1.0 + math.exp(min(s0, s1) - max(s0, s1)), abs=1e-15)


def test_dominant_key_selects_its_value():
    B, H, l_q, L, d = 1, 1, 1, 30, 16
    Q = _rand((B, H, l_q, d), 17)
    K = _rand((B, H, L, d), 18) * 0.01
    V = _rand((B, H, L, d), 19)
    K[0, 0, 11] = Q[0, 0, 0] * 50.0
    O, _, _ = oracle.attention_rows(Q, K, V, 1.0)
    np.testing.assert_allclose(O[0], V[0, 0, 11], atol=1e-12)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("N", [1, 2, 4, 8, 16, 64, 256])
def test_share_independent_of_N_and_rank(N):
    """Any split into N ring blocks, visited in any rank's ring order, gives the same
    result as attention over all keys (slowleelab page, 4.2: after N steps every Q_i
    has met every block)."""
    B, H, l_q, L, d = 1, 2, 6, 256, 16
    Q, K, V = _rand((B, H, l_q, d), 20), _rand((B, H, L, d), 21), _rand((B, H, L, d), 22)
    ref, Mr, Zr = oracle.attention_rows(Q, K, V, 0.25)
    for rank in sorted({0, N // 2, N - 1}):
        O, M, Z = oracle.share(Q, K, V, 0.25, rank, N)
        np.testing.assert_allclose(O, ref, atol=1e-13)
        np.testing.assert_allclose(M, Mr, atol=0)
        np.testing.assert_allclose(Z, Zr, rtol=1e-13)


def test_key_shift_invariance_and_no_overflow():
    """Adding one vector c to every key adds q.c to every score of a row, which a safe
    softmax cancels exactly; with q.c ~ 1e3 an unshifted exp would overflow."""
    B, H, l_q, L, d = 1, 2, 4, 40, 8
    Q, K, V = _rand((B, H, l_q, d), 23), _rand((B, H, L, d), 24), _rand((B, H, L, d), 25)
    K[..., 0] = np.round(K[..., 0] * 256.0) / 256.0  # so K + c below is exact in fp32
    c = np.zeros(d, np.float32)
    c[0] = 256.0
    Q[..., 0] = np.abs(Q[..., 0]) + 4.0
    ref, _, _ = oracle.attention_rows(Q, K, V, 1.0)
    O, M, _ = oracle.attention_rows(Q, K + c, V, 1.0)
    assert np.all(np.isfinite(O)) and M.max() > 1000.0
    np.testing.assert_allclose(O, ref, atol=1e-10)


def test_affine_equivariance_in_values():
    B, H, l_q, L, d = 1, 1, 5, 32, 4
    Q, K, V = _rand((B, H, l_q, d), 26), _rand((B, H, L, d), 27), _rand((B, H, L, d), 28)
    A = np.array([[1, 0, 0, 2], [0, -1, 0, 0], [0, 0, 0.5, 0], [0, 0, 0, 1]], np.float32)
    b = np.array([0.5, -2.0, 0.25, 1.0], np.float32)
    O, _, _ = oracle.attention_rows(Q, K, V, 0.7)
    O2, _, _ = oracle.attention_rows(Q, K, (V @ A + b).astype(np.float32), 0.7)
    np.testing.assert_allclose(O2, O @ A.astype(np.float64) + b, atol=1e-6)


def test_joint_key_value_permutation():
    B, H, l_q, L, d = 1, 2, 3, 37, 8
    Q, K, V = _rand((B, H, l_q, d), 29), _rand((B, H, L, d), 30), _rand((B, H, L, d), 31)
    perm = np.random.default_rng(32).permutation(L)
    O, _, _ = oracle.attention_rows(Q, K, V, 0.4)
    O2, _, _ = oracle.attention_rows(Q, K[:, :, perm].copy(), V[:, :, perm].copy(), 0.4)
    np.testing.assert_allclose(O2, O, atol=1e-14)
    # permuting only the values must change the answer (pins the K/V pairing)
    O3, _, _ = oracle.attention_rows(Q, K, V[:, :, perm].copy(), 0.4)
    assert np.abs(O3 - O).max() > 1e-3


def test_gqa_equals_repeated_kv_mha():
    B, H, H_kv, l_q, L, d = 2, 6, 2, 4, 24, 8
    Q, K, V = _rand((B, H, l_q, d), 33), _rand((B, H_kv, L, d), 34), _rand((B, H_kv, L, d), 35)
    O, M, Z = oracle.attention_rows(Q, K, V, 0.3)
    Kr = np.repeat(K, H // H_kv, axis=1)
    Vr = np.repeat(V, H // H_kv, axis=1)
    O2, M2, Z2 = oracle.attention_rows(Q, Kr, Vr, 0.3)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(M, M2)


def test_bf16_bits_are_read_exactly():
    B, H, l_q, L, d = 1, 2, 3, 20, 8
    q, k, v = synth.draw(B, H, H, d, l_q, L, "bf16", seed=36)
    as_f32 = [x.float().numpy() for x in (q, k, v)]
    as_bits = [synth.to_oracle_array(x) for x in (q, k, v)]
    O1, M1, Z1 = oracle.attention_rows(*as_f32, 0.35)
    O2, M2, Z2 = oracle.attention_rows(*as_bits, 0.35)
    np.testing.assert_array_equal(O1, O2)
    np.testing.assert_array_equal(M1, M2)


def test_row_selection_matches_full_run():
    B, H, l_q, L, d = 2, 3, 9, 16, 8
    Q, K, V = _rand((B, H, l_q, d), 37), _rand((B, H, L, d), 38), _rand((B, H, L, d), 39)
    O, M, Z = oracle.attention_rows(Q, K, V, 0.5)
    rows = [0, 5, 17, 30, B * H * l_q - 1]
    O2, M2, Z2 = oracle.attention_rows(Q, K, V, 0.5, rows=rows)
    np.testing.assert_array_equal(O2, O[rows])
    np.testing.assert_array_equal(M2, M[rows])


# ---------------------------------------------------------------- the step recursion

@pytest.mark.parametrize("N,rank", [(4, 0), (4, 3), (5, 2), (8, 5)])
def test_online_steps_reach_prefix_definition(N, rank):
    """Running the pages' per-step merge in ring order reproduces, after every step,
    the definition restricted to the blocks seen so far (running max exactly, the
    normalised output and the sum to fp64 rounding)."""
    B, H, l, d = 1, 1, 6, 16
    L = N * l
    Q, K, V = _rand((B, H, l, d), 40, 2.0), _rand((B, H, L, d), 41, 2.0), _rand((B, H, L, d), 42)
    q = Q[0, 0].astype(np.float64)
    k = K[0, 0].astype(np.float64)
    v = V[0, 0].astype(np.float64)
    state = oracle.init_state(l, d)
    for t, j in enumerate(oracle.ring_schedule(rank, N)):
        state = oracle.online_step(state, q, k[j * l:(j + 1) * l], v[j * l:(j + 1) * l], 0.3)
        Op, Mp, Zp = oracle.share(Q, K, V, 0.3, rank, N, steps=t + 1)
        O_acc, m, lsum = state
        np.testing.assert_allclose(m, Mp, rtol=1e-15, atol=1e-15)
        np.testing.assert_allclose(lsum, Zp, rtol=1e-13)
        np.testing.assert_allclose(O_acc / lsum[:, None], Op, atol=1e-13)
    np.testing.assert_allclose(oracle.finalize(state),
                               oracle.attention_rows(Q, K, V, 0.3)[0], atol=1e-13)


def test_chunk_local_attention_is_rejected():
    """Negative control: attention restricted to each query's own block (the
    block-diagonal softmax of the 'RingAttention' module on the intelliparadigm page)
    is not exact attention: it changes with N, so the N-independence check above
    would catch an implementation that behaved like it."""
    B, H, L, d = 1, 1, 64, 8
    Q, K, V = _rand((B, H, L, d), 43), _rand((B, H, L, d), 44), _rand((B, H, L, d), 45)
    exact, _, _ = oracle.attention_rows(Q, K, V, 0.5)

    def chunk_local(N):
        l = L // N
        q, k, v = (x[0, 0].astype(np.float64) for x in (Q, K, V))
        out = np.empty((L, d))
        for j in range(N):
            s = 0.5 * q[j * l:(j + 1) * l] @ k[j * l:(j + 1) * l].T
            p = np.exp(s - s.max(axis=1, keepdims=True))
            out[j * l:(j + 1) * l] = (p / p.sum(axis=1, keepdims=True)) @ v[j * l:(j + 1) * l]
        return out

    assert np.abs(chunk_local(1) - exact).max() < 1e-13
    assert np.abs(chunk_local(4) - chunk_local(8)).max() > 1e-2
    assert np.abs(chunk_local(4) - exact).max() > 1e-2


# ---------------------------------------------------------------- the oracle's inputs

def test_workload_shapes():
    w = synth.WORKLOADS["share_L128K_N8"]
    assert (w.l, w.H, w.d, w.L, w.N) == (16384, 32, 128, 131072, 8)
    assert w.flops() == pytest.approx(3.518e13, rel=1e-3)
    g = synth.WORKLOADS["gqa_L128K_N8_28q4kv"]
    assert g.H // g.H_kv == 7
    m = synth.WORKLOADS["share_L1M_N64_std3"]
    assert m.l == 16384 and m.qk_std == 3.0


def test_draw_is_seeded_and_ordered():
    a = synth.draw(1, 2, 1, 8, 4, 12, "bf16", seed=5)
    b = synth.draw(1, 2, 1, 8, 4, 12, "bf16", seed=5)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    g = torch.Generator().manual_seed(5)
    q = torch.randn((1, 2, 4, 8), generator=g)
    assert torch.equal(a[0], q.to(torch.bfloat16))
