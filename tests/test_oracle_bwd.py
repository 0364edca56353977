"""Pins for the backward-pass functions of the fp64 oracle (no GPU needed).

The gradients of O with respect to Q, K, V for an upstream gradient dO
("Long-Context Attention Explained", section "What FlashAttention does not
change": recomputed from the saved row statistics).  Pinned against: torch
autograd through SDPA in fp64 on the CPU (a library routine), 50-digit
central differences of an independent brute-force forward pass, and the
invariants the definition fixes (key gradients of a row sum to zero, value
gradients sum to the upstream gradients, zero dO gives zero gradients, GQA
equals MHA with repeated K/V and summed gradients).
"""
import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs

from test_oracle import _vals


def _case(B, L, n_q, n_kv, d, seed):
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
    dout = inputs.make_qkv(B, L, n_q, n_kv, d, seed + 500)[0]
    return q, k, v, dout


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal,scale", [
    (2, 37, 6, 2, 16, 1, 0.3), (1, 40, 4, 4, 32, 0, 0.2), (1, 65, 8, 1, 8, 1, 0.9),
    (2, 1, 2, 1, 16, 1, 0.5)])
def test_bwd_matches_torch_autograd_fp64(B, L, n_q, n_kv, d, causal, scale):
    torch = pytest.importorskip("torch")
    q, k, v, do = _case(B, L, n_q, n_kv, d, seed=100 + L)
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, scale, causal)
    t = lambda x: torch.from_numpy(_vals(x)).requires_grad_(True)
    tq, tk, tv = t(q), t(k), t(v)
    g = n_q // n_kv
    sc = float(np.float32(scale))
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(g, 1), tv.repeat_interleave(g, 1), is_causal=bool(causal), scale=sc)
    o.backward(torch.from_numpy(_vals(do)))
    assert np.max(np.abs(dq - tq.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) <= 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) <= 1e-12
    # the row statistics: LSE as the forward oracle, delta = dO . O
    of, lf, _ = oracle.attention_rows(q, k, v, scale, causal)
    assert np.array_equal(lse, lf)
    assert np.max(np.abs(delta - np.sum(_vals(do).reshape(-1, d) * of, axis=1))) <= 1e-13


def _mp_forward_loss(mp, qv, kv_, vv, dov, scale, causal):
    """sum over rows of dO . O in mp arithmetic (an independent forward)."""
    B, n_q, L, d = len(qv), len(qv[0]), len(qv[0][0]), len(qv[0][0][0])
    g = n_q // len(kv_[0])
    total = mp.mpf(0)
    for b in range(B):
        for h in range(n_q):
            for i in range(L):
                keys = range(i + 1) if causal else range(L)
                s = [scale * mp.fsum(qv[b][h][i][t] * kv_[b][h // g][j][t] for t in range(d))
                     for j in keys]
                z = mp.fsum(mp.e ** x for x in s)
                for t in range(d):
                    o = mp.fsum(mp.e ** x * vv[b][h // g][j][t] for x, j in zip(s, keys)) / z
                    total += dov[b][h][i][t] * o
    return total


def test_bwd_central_differences_50_digits():
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    B, L, n_q, n_kv, d, causal, scale = 1, 4, 2, 1, 3, 1, 0.7
    q, k, v, do = _case(B, L, n_q, n_kv, d, seed=7)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, scale, causal)
    sc = mp.mpf(float(np.float32(scale)))
    to_mp = lambda x: [[[[mp.mpf(float(e)) for e in row] for row in hh] for hh in bb]
                       for bb in _vals(x)]
    Q, K, V, DO = to_mp(q), to_mp(k), to_mp(v), to_mp(do)
    eps = mp.mpf(10) ** -20
    for name, T, grad in (("q", Q, dq), ("k", K, dk), ("v", V, dv)):
        for idx in [(0, 0, 0, 0), (0, 0, L - 1, d - 1), (0, 1 if T is Q else 0, 2, 1)]:
            b_, h_, i_, t_ = idx
            x0 = T[b_][h_][i_][t_]
            T[b_][h_][i_][t_] = x0 + eps
            up = _mp_forward_loss(mp, Q, K, V, DO, sc, causal)
            T[b_][h_][i_][t_] = x0 - eps
            dn = _mp_forward_loss(mp, Q, K, V, DO, sc, causal)
            T[b_][h_][i_][t_] = x0
            fd = float((up - dn) / (2 * eps))
            assert abs(grad[idx] - fd) <= 1e-13 * max(1.0, abs(fd)), (name, idx, grad[idx], fd)


@pytest.mark.parametrize("causal", [1, 0])
def test_bwd_invariants(causal):
    B, L, n_q, n_kv, d = 2, 50, 6, 3, 16
    q, k, v, do = _case(B, L, n_q, n_kv, d, seed=9)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, 0.25, causal)
    # sum_j dS_ij = 0 for every row, so the key gradients of a kv head sum to 0
    assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    # sum_j P_ij = 1, so the value gradients sum to the group's upstream gradients
    g = n_q // n_kv
    want = _vals(do).reshape(B, n_kv, g, L, d).sum(axis=(2, 3))
    assert np.max(np.abs(dv.sum(axis=2) - want)) <= 1e-11
    # zero upstream gradient: zero gradients
    z = np.zeros_like(do)
    dq0, dk0, dv0, _, _ = oracle.attention_bwd(q, k, v, z, 0.25, causal)
    assert not np.any(dq0) and not np.any(dk0) and not np.any(dv0)


def test_bwd_gqa_equals_mha_with_repeated_kv():
    B, L, n_q, n_kv, d = 1, 33, 8, 2, 16
    g = n_q // n_kv
    q, k, v, do = _case(B, L, n_q, n_kv, d, seed=10)
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, 0.3, 1)
    kr, vr = (np.ascontiguousarray(np.repeat(x, g, axis=1)) for x in (k, v))
    dqm, dkm, dvm, _, _ = oracle.attention_bwd(q, kr, vr, do, 0.3, 1)
    assert np.array_equal(dq, dqm)
    assert np.max(np.abs(dk - dkm.reshape(B, n_kv, g, L, d).sum(axis=2))) <= 1e-13
    assert np.max(np.abs(dv - dvm.reshape(B, n_kv, g, L, d).sum(axis=2))) <= 1e-13


def test_bwd_selected_rows_match_full():
    B, L, n_q, n_kv, d = 1, 70, 4, 2, 16
    q, k, v, do = _case(B, L, n_q, n_kv, d, seed=11)
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, 0.3, 1)
    rows = np.array([0, 5, 69, 70, 139, 279])
    assert np.array_equal(oracle.attention_bwd_dq(q, k, v, do, 0.3, 1, lse, delta, rows),
                          dq.reshape(-1, d)[rows])
    krows = np.array([0, 1, 69, 70, 139])
    dks, dvs = oracle.attention_bwd_dkdv(q, k, v, do, 0.3, 1, lse, delta, krows)
    assert np.array_equal(dks, dk.reshape(-1, d)[krows])
    assert np.array_equal(dvs, dv.reshape(-1, d)[krows])
    with pytest.raises(ValueError):
        oracle.attention_bwd_dq(q, k, v, do, 0.3, 1, lse, delta, np.array([280]))


def test_bwd_rounding_bound_holds_in_simulation():
    # emulate a kernel that recomputes P in fp32 from an fp32 LSE, takes D
    # from O rounded to bf16, rounds P and dS to bf16 for the products and
    # the gradients to bf16 once; every gradient element must lie within the
    # oracle's bound of the exact value
    B, L, n_q, n_kv, d, causal, scale = 1, 48, 4, 2, 32, 1, 0.2
    g = n_q // n_kv
    q, k, v, do = _case(B, L, n_q, n_kv, d, seed=12)
    lse, delta, absd = oracle.attention_bwd_rowstats(q, k, v, do, scale, causal)
    rows = np.arange(B * n_q * L)
    krows = np.arange(B * n_kv * L)
    dq, bq = oracle.attention_bwd_dq(q, k, v, do, scale, causal, lse, delta, rows, absd)
    dk, dv, bk, bv = oracle.attention_bwd_dkdv(q, k, v, do, scale, causal, lse, delta, krows, absd)
    o, _, _ = oracle.attention_rows(q, k, v, scale, causal)
    rb = lambda x: inputs.bf16_to_f32(inputs.bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)
    qv, kv_, vv, dov = (_vals(x)[0] for x in (q, k, v, do))
    o_b = rb(o).reshape(n_q, L, d)
    sc32 = np.float32(scale)
    log2e = np.float32(1.4426950408889634)
    sim_dq = np.zeros((n_q, L, d))
    sim_dk = np.zeros((n_kv, L, d))
    sim_dv = np.zeros((n_kv, L, d))
    for h in range(n_q):
        kh = h // g
        s32 = (qv[h].astype(np.float32) @ kv_[kh].astype(np.float32).T)  # exact products, fp32 sums
        l32 = np.float32(lse.reshape(n_q, L)[h]) * log2e
        p32 = np.exp2(s32 * (sc32 * log2e) - l32[:, None]).astype(np.float32)
        mask = np.tril(np.ones((L, L), bool)) if causal else np.ones((L, L), bool)
        p32 = np.where(mask, p32, 0).astype(np.float32)
        dp32 = (dov[h].astype(np.float32) @ vv[kh].astype(np.float32).T)
        d32 = np.sum(dov[h].astype(np.float32) * o_b[h].astype(np.float32), axis=1)
        ds32 = p32 * (dp32 - d32[:, None])
        pb, dsb = rb(p32), rb(ds32)
        sim_dv[kh] += pb.T @ dov[h]
        sim_dk[kh] += float(sc32) * (dsb.T @ qv[h])
        sim_dq[h] = float(sc32) * (dsb @ kv_[kh])
    sim_dq, sim_dk, sim_dv = rb(sim_dq), rb(sim_dk), rb(sim_dv)
    for name, sim, ref, bnd in (("dq", sim_dq, dq, bq), ("dk", sim_dk, dk, bk), ("dv", sim_dv, dv, bv)):
        err = np.abs(sim.reshape(-1, d) - ref)
        assert np.all(err <= bnd + 1e-12), (name, float(np.max(err - bnd)))
        assert np.max(err / (bnd + 1e-30)) > 0.05, name   # and the bound is not vacuous
