"""Planted mistakes in a copy of the oracle must be caught by its pins.

Each mutant is a one-line edit of attn_oracle.c that a careless author could
plausibly make; it is compiled on the CPU into a temporary library, and at
least one of the pin checks below has to fail on it, while all of them pass on
the real oracle.  This guards the pins themselves.
"""
import math
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
    "kv heads strided by Lq": ("const uint16_t *kbase = k + (b * n_kv + kvh) * Lk * d_h;",
                               "const uint16_t *kbase = k + (b * n_kv + kvh) * Lq * d_h;"),
    "kv head h mod n_kv": ("const int64_t kvh = h / g;", "const int64_t kvh = h % n_kv;"),
    "log2 in lse": ("*lse = m + log(total);", "*lse = m + log2(total);"),
    "K read transposed": ("dot += widen_bf16(qrow[t]) * widen_bf16(krow[t]);",
                          "dot += widen_bf16(qrow[t]) * widen_bf16(kbase[t * L + j]); (void)krow;"),
    "scale ignored": ("s[j] = scale * dot;", "s[j] = dot / sqrt((double)d_h); (void)scale;"),
    "weights not normalised": ("w[j] = w[j] / total;", "w[j] = w[j];"),
    "V read from K": ("const uint16_t *vbase = v +", "const uint16_t *vbase = k +"),
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


CHECKS = [_check_brute, _check_large_scores, _check_constant_v,
          _check_zero_query, _check_flops, _check_chunk_brute]


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
