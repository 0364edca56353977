"""Pins for the rounding bounds of tests/bounds.py (CPU only).

Each bound claims that a kernel with a stated arithmetic lands within it of
the exact (oracle) value.  The pins run that arithmetic on the CPU, in fp32
and with the stated roundings, accumulating every long sum one term at a time
in fp32 (the order that rounds most often), and check that every simulated
element lies within its bound of the oracle's exact value, and that the
bound is not vacuous (some elements use a visible part of it).
"""
import math

import numpy as np
import pytest

import bounds
import oracle
from causal_gqa_prefill_amd import inputs

f32 = np.float32


def _rb(x):
    """Round to bf16 (nearest even), back as fp64."""
    return inputs.bf16_to_f32(inputs.bf16_bits(np.asarray(x, dtype=np.float32))).astype(np.float64)


def _vals(bits):
    return inputs.bf16_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------
# backward pass, at a sequence length where the fp32 sums are long
# ---------------------------------------------------------------------------
def test_bwd_bound_holds_for_fp32_sums_at_length_2048():
    B, L, n_q, n_kv, d, causal = 1, 2048, 2, 1, 64, 1
    g = n_q // n_kv
    scale = float(np.float32(1 / 8))
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, 61)
    do = inputs.make_qkv(B, L, n_q, n_kv, d, 62)[0]
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, scale, causal)
    o, _, _ = oracle.attention_rows(q, k, v, scale, causal)
    qv, kv_, vv, dov = (_vals(x)[0] for x in (q, k, v, do))   # [heads, L, d]
    o = o.reshape(n_q, L, d)
    lse = lse.reshape(n_q, L)
    delta = delta.reshape(n_q, L)

    # -- the kernels' arithmetic, simulated
    c2 = f32(f32(scale) * f32(bounds.LOG2E))
    ob = _rb(o).astype(f32)
    mask = np.tril(np.ones((L, L), bool))
    dsb = np.empty((n_q, L, L), dtype=f32)
    pb = np.empty((n_q, L, L), dtype=f32)
    d_sim = np.empty((n_q, L))
    for h in range(n_q):
        q32, k32 = qv[h].astype(f32), kv_[0].astype(f32)
        v32, do32 = vv[0].astype(f32), dov[h].astype(f32)
        s32 = q32 @ k32.T                                          # fp32 dot products
        lse2 = f32(f32(lse[h]) * f32(bounds.LOG2E))
        x = f32(s32.astype(np.float64) * float(c2) - lse2.astype(np.float64)[:, None])  # one fma
        p32 = np.where(mask, f32(np.exp2(x.astype(np.float64))), f32(0))
        dp32 = do32 @ v32.T
        acc = np.zeros(L, dtype=f32)
        for t in range(d):                                         # D from the bf16 output
            acc = f32(acc + f32(do32[:, t] * ob[h][:, t]))
        d_sim[h] = acc
        ds32 = f32(p32 * f32(dp32 - acc[:, None]))
        pb[h] = _rb(p32)
        dsb[h] = _rb(ds32)
    # dQ: one fp32 rounding per key, keys in order
    sim_dq = np.empty((n_q, L, d))
    k32 = kv_[0].astype(f32)
    for h in range(n_q):
        acc = np.zeros((L, d), dtype=f32)
        for j in range(L):
            acc = f32(acc + f32(dsb[h][:, j:j + 1] * k32[j][None, :]))
        sim_dq[h] = _rb(f32(acc * f32(scale)))
    # dK, dV: one fp32 rounding per query row, over the group's heads
    acck = np.zeros((L, d), dtype=f32)
    accv = np.zeros((L, d), dtype=f32)
    for h in range(n_q):
        q32, do32 = qv[h].astype(f32), dov[h].astype(f32)
        for i in range(L):
            acck = f32(acck + f32(dsb[h][i][:, None] * q32[i][None, :]))
            accv = f32(accv + f32(pb[h][i][:, None] * do32[i][None, :]))
    sim_dk = _rb(f32(acck * f32(scale)))
    sim_dv = _rb(accv)

    # -- against the bounds
    grp = bounds.BwdGroup(qv, kv_[0], vv[0], dov, o, lse, delta, scale, causal)
    heads = np.repeat(np.arange(n_q), L)
    idx = np.tile(np.arange(L), n_q)
    bq = grp.dq_bound(heads, idx, dq.reshape(-1, d))
    bk, bv = grp.dkdv_bound(np.arange(L), dk.reshape(-1, d), dv.reshape(-1, d))
    bd = bounds.bwd_delta_bound(dov.reshape(-1, d), o.reshape(-1, d))
    for name, sim, ref, bnd in (("dq", sim_dq.reshape(-1, d), dq.reshape(-1, d), bq),
                                ("dk", sim_dk, dk.reshape(-1, d), bk),
                                ("dv", sim_dv, dv.reshape(-1, d), bv),
                                ("delta", d_sim.reshape(-1), delta.reshape(-1), bd)):
        err = np.abs(sim - ref)
        assert np.all(err <= bnd), (name, float(np.max(err - bnd)))
        assert np.max(err / (bnd + 1e-300)) > 0.05, name    # not vacuous


@pytest.mark.parametrize("slip", ["lse off by 0.05", "delta omitted"])
def test_bwd_bound_catches_a_planted_slip(slip):
    """Gradients from a slipped arithmetic (a wrong row statistic, or dS
    without the delta term), computed exactly otherwise: some elements must
    leave the bound."""
    B, L, n_q, n_kv, d, causal = 1, 256, 1, 1, 64, 1
    scale = float(np.float32(1 / 8))
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, 63)
    do = inputs.make_qkv(B, L, n_q, n_kv, d, 64)[0]
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, scale, causal)
    o, _, _ = oracle.attention_rows(q, k, v, scale, causal)
    qv, kv_, vv, dov = (_vals(x)[0] for x in (q, k, v, do))
    o = o.reshape(n_q, L, d)
    shift = 0.05 if slip == "lse off by 0.05" else 0.0
    p = np.where(np.tril(np.ones((L, L), bool)),
                 np.exp(scale * (qv[0] @ kv_[0].T) - lse[:, None] - shift), 0)
    ds = p * ((dov[0] @ vv[0].T) - (delta[:, None] if slip != "delta omitted" else 0.0))
    bad_dq = scale * (ds @ kv_[0])
    bad_dv = p.T @ dov[0]
    grp = bounds.BwdGroup(qv, kv_[0], vv[0], dov, o, lse.reshape(1, L), delta.reshape(1, L),
                          scale, causal)
    bq = grp.dq_bound(np.zeros(L, int), np.arange(L), dq.reshape(-1, d))
    _, bv = grp.dkdv_bound(np.arange(L), dk.reshape(-1, d), dv.reshape(-1, d))
    assert (np.any(np.abs(bad_dq - dq.reshape(-1, d)) > bq)
            or np.any(np.abs(bad_dv - dv.reshape(-1, d)) > bv))


# ---------------------------------------------------------------------------
# FP8: the weights rounded to e4m3 against a running reference
# ---------------------------------------------------------------------------
def _fp8_case(B, L_q, L_k, n_q, n_kv, d, seed):
    return inputs.make_fp8_qkv(B, L_q, L_k, n_q, n_kv, d, seed)


def test_fp8_bound_holds_in_simulation():
    # p = 2^(s log2 e - m_ref) for references anywhere within 2^8 below the
    # row max, rounded to e4m3 (nearest even), P V summed one key at a time in
    # fp32, divided by the fp32 sum of the unrounded p, O rounded to bf16:
    # every element within the bound of the exact output
    B, Lq, Lk, q_off, n_q, n_kv, d = 1, 24, 600, 576, 2, 1, 16
    q, k, v, dq, dk, dv = _fp8_case(B, Lq, Lk, n_q, n_kv, d, seed=84)
    scale = 0.6
    o, l, _ = oracle.attention_rows_chunk_fp8(q, k, v, scale, dq, dk, dv, True, q_off)
    tab = oracle.e4m3_table()
    qv, kv_, vv = tab[q] * dq, tab[k] * dk, tab[v] * dv
    rows = np.arange(B * n_q * Lq)
    bnd = bounds.fp8_rows_bound(q, k, v, dq, dk, dv, float(np.float32(scale)), l, rows, True,
                                q_off, tab)
    rng = np.random.default_rng(5)
    worst = 0.0
    for h in range(n_q):
        for i in range(Lq):
            r = h * Lq + i
            n = q_off + i + 1
            s = (kv_[0, 0, :n] @ qv[0, h, i]) * float(np.float32(scale)) * math.log2(math.e)
            for m_ref in (s.max(), s.max() - 8.0, s.max() - rng.uniform(0, 8)):
                p = f32(np.exp2(s - m_ref))
                assert p.max() <= 256.0
                p_hat = tab[inputs.e4m3_bits(p)].astype(f32)
                acc = np.zeros(d, dtype=f32)
                tot = f32(0)
                for j in range(n):
                    acc = f32(acc + f32(p_hat[j] * vv[0, 0, j].astype(f32)))
                    tot = f32(tot + p[j])
                approx = _rb(f32(acc / tot))
                err = np.abs(approx - o[r])
                assert np.all(err <= bnd[r]), (h, i, m_ref)
                worst = max(worst, float(np.max(err / bnd[r])))
    assert worst > 0.05  # the bound is not vacuous on these rows
