"""Pins for the FP8 (OCP e4m3) path of the fp64 oracle (no GPU needed).

FP8 attention: "flops / prefill-attention", section "Workarounds".  The
oracle decodes each e4m3 code exactly, multiplies by the tensor's descale
factor and runs the plain attention.  Pinned here against: torch's
float8_e4m3fn decoder and encoder (a library routine), the format's
closed-form values, the already-pinned bf16 path on inputs both formats hold
exactly, and 50-digit brute force.  (The bound on what rounding the weights
to e4m3 can change lives with the tests, in bounds.py, pinned in
test_bounds.py.)
"""
import math

import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs

from test_oracle import _vals


def test_e4m3_table_matches_torch_and_closed_forms():
    torch = pytest.importorskip("torch")
    t = oracle.e4m3_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    both_nan = np.isnan(t) & np.isnan(ref)
    assert np.all(both_nan | (t == ref))
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF]) and np.sum(np.isnan(t)) == 2
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0           # largest finite
    assert t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9  # subnormals
    assert t[0x08] == 2.0 ** -6                               # smallest normal
    assert t[0x38] == 1.0 and t[0x39] == 1.125 and t[0x40] == 2.0
    assert t[0x00] == 0.0 and math.copysign(1.0, t[0x80]) == -1.0


def test_e4m3_encoder_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 40,
        rng.uniform(-2.0 ** -6, 2.0 ** -6, 20000).astype(np.float32),   # subnormal range
        (inputs._e4m3_positive_values()[:-1] + inputs._e4m3_positive_values()[1:]).astype(np.float32) / 2,  # ties
    ])
    x = np.clip(x, -460, 460)
    mine = inputs.e4m3_bits(x)
    th = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mine, th)


def _fp8_case(B, Lq, Lk, n_q, n_kv, d, seed, pow2_scales=False):
    q, k, v, dq, dk, dv = inputs.make_fp8_qkv(B, Lq, Lk, n_q, n_kv, d, seed)
    if pow2_scales:
        dq, dk, dv = (float(2.0 ** round(math.log2(s))) for s in (dq, dk, dv))
    return q, k, v, dq, dk, dv


@pytest.mark.parametrize("B,Lq,Lk,q_off,n_q,n_kv,d,causal", [
    (1, 37, 37, 0, 4, 2, 16, 1), (2, 9, 40, 31, 6, 3, 8, 1), (1, 12, 30, 0, 2, 1, 32, 0)])
def test_fp8_path_equals_bf16_path_on_shared_values(B, Lq, Lk, q_off, n_q, n_kv, d, causal):
    # with power-of-two descales every decoded value is exact in bf16 as well:
    # the fp8 path must give the bf16 path's (pinned) results bit for bit
    q, k, v, dq, dk, dv = _fp8_case(B, Lq, Lk, n_q, n_kv, d, seed=81 + d, pow2_scales=True)
    tab = oracle.e4m3_table()
    to_bf16 = lambda c, s: inputs.bf16_bits((tab[c] * s).astype(np.float32))
    qb, kb, vb = to_bf16(q, dq), to_bf16(k, dk), to_bf16(v, dv)
    assert np.array_equal(_vals(qb), tab[q] * dq)  # really exact
    o8, l8, f8 = oracle.attention_rows_chunk_fp8(q, k, v, 0.3, dq, dk, dv, causal, q_off)
    ob, lb, fb = oracle.attention_rows_chunk(qb, kb, vb, 0.3, causal, q_offset=q_off)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb) and f8 == fb


def test_fp8_brute_force_50_digits():
    mpmath = pytest.importorskip("mpmath")
    torch = pytest.importorskip("torch")
    mp = mpmath.mp
    mp.dps = 50
    B, Lq, Lk, q_off, n_q, n_kv, d = 1, 3, 7, 4, 4, 2, 8
    q, k, v, dq, dk, dv = _fp8_case(B, Lq, Lk, n_q, n_kv, d, seed=83)
    dec = lambda c: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    qv, kv_, vv = dec(q) * dq, dec(k) * dk, dec(v) * dv
    o, l, _ = oracle.attention_rows_chunk_fp8(q, k, v, 0.45, dq, dk, dv, True, q_off)
    o = o.reshape(n_q, Lq, d)
    l = l.reshape(n_q, Lq)
    sc = mp.mpf(float(np.float32(0.45)))
    for h in range(n_q):
        kh = h // (n_q // n_kv)
        for i in range(Lq):
            keys = range(q_off + i + 1)
            s = [sc * mp.fsum(mp.mpf(qv[0, h, i, t]) * mp.mpf(kv_[0, kh, j, t]) for t in range(d))
                 for j in keys]
            lz = mp.log(mp.fsum(mp.e ** x for x in s))
            assert abs(l[h, i] - float(lz)) <= 1e-14 * max(1.0, abs(float(lz)))
            for t in range(d):
                ot = mp.fsum(mp.e ** (x - lz) * mp.mpf(vv[0, kh, j, t]) for x, j in zip(s, keys))
                assert abs(o[h, i, t] - float(ot)) <= 1e-14


def test_fp8_bad_arguments_rejected():
    q, k, v, dq, dk, dv = _fp8_case(1, 4, 8, 2, 1, 16, seed=85)
    with pytest.raises(ValueError):
        oracle.attention_rows_chunk_fp8(q, k, v, 0.5, float("inf"), dk, dv, True, 0)
    with pytest.raises(ValueError):
        oracle.attention_rows_chunk_fp8(q, k, v, 0.5, dq, dk, dv, True, 5)   # 5 + 4 > 8
    with pytest.raises(ValueError):
        oracle.attention_rows_chunk_fp8(q.astype(np.uint16), k, v, 0.5, dq, dk, dv, True, 0)
