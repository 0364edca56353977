"""Planted mistakes in a copy of the oracle must be caught by its pins.

Each mutant is a one-line edit of attn_oracle.c that a careless author could
plausibly make; it is compiled on the CPU into a temporary library, and at
least one of the pin checks below has to fail on it, while all of them pass on
the real oracle.  This guards the pins themselves.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from causal_gqa_prefill_amd import inputs

from test_oracle import _brute_force, _bits_from_f32, _vals

SRC = open(obuild.SRC).read()

MUTANTS = {
    "no max subtraction": ("w[j] = exp(s[j] - m);", "w[j] = exp(s[j]); (void)0;"),
    "mask excludes self": ("causal ? q_off + i + 1 : Lk", "causal ? q_off + i : Lk"),
    "mask one too wide": ("causal ? q_off + i + 1 : Lk",
                          "causal ? (q_off + i + 2 < Lk ? q_off + i + 2 : Lk) : Lk"),
    "chunk offset ignored": ("causal ? q_off + i + 1 : Lk", "causal ? i + 1 : Lk"),
    "kv heads strided by Lq": ("const int64_t kbase = (b * n_kv + kvh) * Lk * d_h;",
                               "const int64_t kbase = (b * n_kv + kvh) * Lq * d_h;"),
    "e4m3 bias 8": ("x = ldexp(1.0 + m / 8.0, e - 7);", "x = ldexp(1.0 + m / 8.0, e - 8);"),
    "e4m3 subnormals as normals": ("x = ldexp((double)m, -9);", "x = ldexp(1.0 + m / 8.0, -6);"),
    "descale ignored": ("return widen_e4m3(((const uint8_t *)base)[idx]) * mul;",
                        "return widen_e4m3(((const uint8_t *)base)[idx]); (void)mul;"),
    "dS sign in dQ": ("p * (bwd_dp(v, dout, L, n_q, n_kv, d_h, b, h, i, j) - delta[row])",
                      "p * (delta[row] - bwd_dp(v, dout, L, n_q, n_kv, d_h, b, h, i, j))"),
    "delta not subtracted in dK": ("p * (bwd_dp(v, dout, L, n_q, n_kv, d_h, b, h, i, j) - delta[qrow_id])",
                                   "p * bwd_dp(v, dout, L, n_q, n_kv, d_h, b, h, i, j); (void)delta"),
    "dQ without scale": ("out[t] += sc * ds * widen_bf16(krow[t]);",
                         "out[t] += ds * widen_bf16(krow[t]);"),
    "dV from dS": ("ov[t] += p * widen_bf16(drow[t]);", "ov[t] += ds * widen_bf16(drow[t]);"),
    "dK from dO": ("ok[t] += sc * ds * widen_bf16(qrow[t]);",
                   "ok[t] += sc * ds * widen_bf16(drow[t]); (void)qrow;"),
    "delta without O": ("acc += widen_bf16(dout[row * d_h + t]) * o[r * d_h + t];",
                        "acc += widen_bf16(dout[row * d_h + t]);"),
    "kv head h mod n_kv": ("const int64_t kvh = h / g;", "const int64_t kvh = h % n_kv;"),
    "log2 in lse": ("*lse = m + log(total);", "*lse = m + log2(total);"),
    "K read transposed": ("dot += elem(kind, q, qrow + t, dq) * elem(kind, k, krow + t, dk);",
                          "dot += elem(kind, q, qrow + t, dq) * elem(kind, k, kbase + t * L + j, dk);"
                          " (void)krow;"),
    "scale ignored": ("s[j] = scale * dot;", "s[j] = dot / sqrt((double)d_h); (void)scale;"),
    "weights not normalised": ("w[j] = w[j] / total;", "w[j] = w[j];"),
    "V read from K": ("out[t] += p * elem(kind, v, vrow + t, dv);",
                      "out[t] += p * elem(kind, k, vrow + t, dv);"),
    "lse without max": ("*lse = m + log(total);", "*lse = log(total);"),
    "flops halved": ("(uint64_t)(4 * d_h * n_vis)", "(uint64_t)(2 * d_h * n_vis)"),
}


def _check_brute(lib):
    for (B, L, n_q, n_kv, d, causal, scale) in [(2, 9, 4, 2, 8, 1, 0.3),
                                                (1, 7, 6, 2, 5, 0, 0.6)]:
        q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, seed=77 + L)
        ref_o, ref_l = _brute_force(q, k, v, scale, causal)
        o, l, _ = oracle.attention_rows(q, k, v, scale, causal, lib=lib)
        if not (np.max(np.abs(o - ref_o.reshape(-1, d))) <= 1e-14 and
                np.max(np.abs(l - ref_l.reshape(-1))) <= 1e-14):
            return False
    return True


def _check_large_scores(lib):
    q, k, v = inputs.make_qkv(1, 64, 2, 1, 16, seed=5)
    q = _bits_from_f32(inputs.bf16_to_f32(q) * np.float32(300.0))
    o, l, _ = oracle.attention_rows(q, k, v, 1.0, True, lib=lib)
    return bool(np.all(np.isfinite(o)) and np.all(np.isfinite(l)))


def _check_constant_v(lib):
    B, L, n_q, n_kv, d = 1, 20, 4, 2, 8
    q, k, _ = inputs.make_qkv(B, L, n_q, n_kv, d, seed=9)
    c = np.array([[1.5], [-2.5]], dtype=np.float32)[None, :, :, None] * np.ones((1, 2, L, d), np.float32)
    v = _bits_from_f32(c)
    o, _, _ = oracle.attention_rows(q, k, v, 0.2, True, lib=lib)
    o = o.reshape(n_q, L, d)
    want = np.array([1.5, 1.5, -2.5, -2.5])[:, None, None]
    return bool(np.max(np.abs(o - want)) <= 1e-14)


def _check_zero_query(lib):
    L = 30
    _, k, v = inputs.make_qkv(1, L, 1, 1, 8, seed=23)
    q = np.zeros((1, 1, L, 8), dtype=np.uint16)
    o, l, _ = oracle.attention_rows(q, k, v, 0.5, True, lib=lib)
    means = np.cumsum(_vals(v)[0, 0], axis=0) / np.arange(1, L + 1)[:, None]
    return bool(np.max(np.abs(o - means)) <= 1e-14 and
                np.max(np.abs(l - np.log(np.arange(1, L + 1)))) <= 1e-14)


def _check_flops(lib):
    B, L, n_q, n_kv, d = 1, 37, 4, 2, 8
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, seed=51)
    _, _, fc = oracle.attention_rows(q, k, v, 0.3, True, lib=lib)
    return fc == 2 * B * n_q * d * L * (L + 1)


def _check_chunk_brute(lib):
    # a causal chunk at an offset, GQA with two kv heads and two sequences,
    # fewer queries than keys
    B, Lq, Lk, q_off, n_q, n_kv, d = 2, 3, 8, 4, 4, 2, 4
    q, _, _ = inputs.make_qkv(B, Lq, n_q, n_kv, d, seed=81)
    _, k, v = inputs.make_qkv(B, Lk, n_q, n_kv, d, seed=82)
    ref_o, ref_l = _brute_force(q, k, v, 0.5, 1, q_off=q_off)
    o, l, _ = oracle.attention_rows_chunk(q, k, v, 0.5, True, q_offset=q_off, lib=lib)
    return bool(np.max(np.abs(o - ref_o.reshape(-1, d))) <= 1e-14 and
                np.max(np.abs(l - ref_l.reshape(-1))) <= 1e-14)


def _check_fp8(lib):
    # the e4m3 decoder against torch and the fp8 path against the bf16 path on
    # values both hold exactly (power-of-two descales)
    torch = pytest.importorskip("torch")
    tab = oracle.e4m3_table(lib=lib)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    if not np.all((np.isnan(tab) & np.isnan(ref)) | (tab == ref)):
        return False
    q, k, v, *_ = inputs.make_fp8_qkv(1, 6, 20, 2, 1, 8, 86)
    dq, dk, dv = 0.25, 0.5, 2.0
    to_b = lambda c, s_: inputs.bf16_bits((ref[c] * s_).astype(np.float32))
    o8, l8, _ = oracle.attention_rows_chunk_fp8(q, k, v, 0.7, dq, dk, dv, True, 14, lib=lib)
    ob, lb, _ = oracle.attention_rows_chunk(to_b(q, dq), to_b(k, dk), to_b(v, dv), 0.7, True,
                                            q_offset=14, lib=lib)
    return bool(np.max(np.abs(o8 - ob)) <= 1e-15 and np.max(np.abs(l8 - lb)) <= 1e-15)


def _check_bwd(lib):
    # the gradients against torch autograd through SDPA in fp64 (GQA, both
    # masks)
    torch = pytest.importorskip("torch")
    B, L, n_q, n_kv, d = 1, 19, 4, 2, 8
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, 87)
    do = inputs.make_qkv(B, L, n_q, n_kv, d, 88)[0]
    for causal in (1, 0):
        dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, 0.4, causal, lib=lib)
        t = lambda x: torch.from_numpy(_vals(x)).requires_grad_(True)
        tq, tk, tv = t(q), t(k), t(v)
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(2, 1), tv.repeat_interleave(2, 1), is_causal=bool(causal),
            scale=float(np.float32(0.4)))
        o.backward(torch.from_numpy(_vals(do)))
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            if not np.max(np.abs(mine - ref.numpy())) <= 1e-12:
                return False
    return True


CHECKS = [_check_brute, _check_large_scores, _check_constant_v,
          _check_zero_query, _check_flops, _check_chunk_brute, _check_fp8, _check_bwd]


def _build_variant(tmp_path, name, src):
    c = tmp_path / (name.replace(" ", "_") + ".c")
    c.write_text(src)
    so = str(tmp_path / (name.replace(" ", "_") + ".so"))
    obuild.compile_to(str(c), so)
    return oracle.load_library(so)


def test_real_oracle_passes_every_check(tmp_path):
    lib = _build_variant(tmp_path, "real", SRC)
    for chk in CHECKS:
        assert chk(lib), chk.__name__


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation site for {name!r} not found"
    lib = _build_variant(tmp_path, name, SRC.replace(old, new))
    with np.errstate(all="ignore"):
        results = {chk.__name__: chk(lib) for chk in CHECKS}
    assert not all(results.values()), f"mutant {name!r} passed every check"
