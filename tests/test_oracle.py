"""Pins for the fp64 CPU oracle (no GPU needed).

Each test checks the oracle against something other than itself: 50-digit
brute force, closed forms, invariants, a library routine (torch SDPA on the
CPU in fp64), an independent tiled online-softmax written here from the
pages' five steps, and numbers the pages print.  Together they are chosen so
that a plausible slip in the oracle (a dropped max subtraction, a wrong mask
boundary, a wrong key/value head, a wrong log base, a transposed operand, a
mis-applied scale) fails at least one of them; test_oracle_mutants.py checks
exactly that.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")


def _bits_from_f32(x):
    return inputs.bf16_bits(np.asarray(x, dtype=np.float32))


def _vals(bits):
    return inputs.bf16_to_f32(bits).astype(np.float64)


def _random_case(B, L, n_q, n_kv, d, seed, mult=1.0):
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
    if mult != 1.0:
        q = _bits_from_f32(inputs.bf16_to_f32(q) * np.float32(mult))
    return q, k, v


# ----------------------------------------------------------------------------
# 50-digit brute force on tiny inputs ("Why Attention Scaling Breaks",
# section "The O(n^2) problem": softmax(Q K^T / sqrt d) V; causal: each token
# sees itself and earlier tokens; GQA: head h reads kv-head h // g)
# ----------------------------------------------------------------------------
def _brute_force(q, k, v, scale, causal, q_off=0):
    """50-digit attention; query row i sits at key position q_off + i."""
    mpmath = pytest.importorskip("mpmath")
    mp = mpmath.mp
    mp.dps = 50
    B, n_q, L, d = q.shape
    n_kv, Lk = k.shape[1], k.shape[2]
    g = n_q // n_kv
    qv, kv_, vv = _vals(q), _vals(k), _vals(v)
    sc = mp.mpf(float(np.float32(scale)))
    out = np.zeros((B, n_q, L, d))
    lse = np.zeros((B, n_q, L))
    for b in range(B):
        for h in range(n_q):
            kh = h // g
            for i in range(L):
                keys = range(q_off + i + 1) if causal else range(Lk)
                s = []
                for j in keys:
                    acc = mp.mpf(0)
                    for t in range(d):
                        acc += mp.mpf(qv[b, h, i, t]) * mp.mpf(kv_[b, kh, j, t])
                    s.append(sc * acc)
                # direct log-sum-exp: no max subtraction needed at 50 digits
                z = mp.fsum([mp.e ** x for x in s])
                lz = mp.log(z)
                lse[b, h, i] = float(lz)
                for t in range(d):
                    o = mp.fsum([mp.e ** (x - lz) * mp.mpf(vv[b, kh, j, t])
                                 for x, j in zip(s, keys)])
                    out[b, h, i, t] = float(o)
    return out, lse


TINY = [
    # B, L, n_q, n_kv, d, causal, scale
    (1, 1, 1, 1, 1, 1, 0.5),
    (1, 5, 2, 1, 3, 1, 0.37),
    (2, 9, 4, 2, 8, 1, 1.0 / math.sqrt(8)),
    (1, 9, 3, 1, 8, 0, 0.9),
    (2, 7, 6, 2, 5, 0, 0.25),
    (1, 8, 6, 3, 4, 1, 1.7),
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal,scale", TINY)
def test_brute_force_50_digits(B, L, n_q, n_kv, d, causal, scale):
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=11 + L * d + n_q)
    ref_o, ref_l = _brute_force(q, k, v, scale, causal)
    o, l, _ = oracle.attention_rows(q, k, v, scale, causal)
    assert np.max(np.abs(o - ref_o.reshape(-1, d))) <= 1e-14
    assert np.max(np.abs(l - ref_l.reshape(-1))) <= 1e-14


def test_brute_force_large_scores():
    # scores of several hundred: exp would overflow fp64 without the max
    # subtraction ("Long-Context Attention Explained", safe-softmax remark)
    B, L, n_q, n_kv, d = 1, 6, 2, 1, 4
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=5)
    q = _bits_from_f32(inputs.bf16_to_f32(q) * np.float32(300.0))
    k = _bits_from_f32(inputs.bf16_to_f32(k) * np.float32(3.0))
    ref_o, ref_l = _brute_force(q, k, v, 1.0, 1)
    o, l, _ = oracle.attention_rows(q, k, v, 1.0, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    assert np.max(np.abs(l)) > 710  # exp(lse) itself overflows fp64
    assert np.max(np.abs(o - ref_o.reshape(-1, d))) <= 1e-14
    assert np.max(np.abs(l - ref_l.reshape(-1)) / np.abs(ref_l.reshape(-1))) <= 1e-15


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [1, 0])
def test_rows_sum_to_one_identity_v(causal):
    # V = identity makes O equal the materialised weights P: rows sum to 1,
    # masked weights are exactly 0 and visible ones are positive
    L = d = 16
    q, k, _ = _random_case(1, L, 2, 1, d, seed=3)
    v = _bits_from_f32(np.eye(L, dtype=np.float32)[None, None])
    o, _, _ = oracle.attention_rows(q, k, v, 0.3, causal)
    o = o.reshape(2, L, L)
    assert np.max(np.abs(o.sum(axis=-1) - 1.0)) <= 1e-13
    for i in range(L):
        vis = i + 1 if causal else L
        assert np.all(o[:, i, :vis] > 0)
        assert np.all(o[:, i, vis:] == 0.0)


def test_constant_v_returns_v():
    B, L, n_q, n_kv, d = 2, 33, 6, 3, 8
    q, k, _ = _random_case(B, L, n_q, n_kv, d, seed=9)
    c = np.zeros((B, n_kv, 1, d), dtype=np.float32)
    for b in range(B):
        for kv in range(n_kv):
            c[b, kv, 0] = (kv + 1.5) * (-1.0) ** np.arange(d) + 0.25 * b
    v = _bits_from_f32(np.broadcast_to(c, (B, n_kv, L, d)))
    for causal in (1, 0):
        o, _, _ = oracle.attention_rows(q, k, v, 0.2, causal)
        o = o.reshape(B, n_q, L, d)
        for h in range(n_q):
            want = _vals(v)[:, h // (n_q // n_kv), 0, :]
            assert np.max(np.abs(o[:, h] - want[:, None, :])) <= 1e-14


def test_length_one_returns_v0():
    B, n_q, n_kv, d = 2, 4, 2, 16
    q, k, v = _random_case(B, 1, n_q, n_kv, d, seed=21)
    scale = 0.125
    for causal in (1, 0):
        o, l, _ = oracle.attention_rows(q, k, v, scale, causal)
        o = o.reshape(B, n_q, d)
        l = l.reshape(B, n_q)
        for b in range(B):
            for h in range(n_q):
                kv = h // 2
                assert np.array_equal(o[b, h], _vals(v)[b, kv, 0])
                want = float(np.float32(scale)) * float(
                    np.dot(_vals(q)[b, h, 0], _vals(k)[b, kv, 0]))
                assert abs(l[b, h] - want) <= 1e-14 * max(1.0, abs(want))


def test_first_causal_row_returns_v0():
    B, L, n_q, n_kv, d = 1, 40, 4, 4, 32
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=22)
    o, l, _ = oracle.attention_rows(q, k, v, 0.177, True)
    o = o.reshape(B, n_q, L, d)
    l = l.reshape(B, n_q, L)
    for h in range(n_q):
        assert np.array_equal(o[0, h, 0], _vals(v)[0, h, 0])
        want = float(np.float32(0.177)) * float(np.dot(_vals(q)[0, h, 0], _vals(k)[0, h, 0]))
        assert abs(l[0, h, 0] - want) <= 1e-14 * max(1.0, abs(want))


def test_zero_query_gives_running_mean():
    # all scores equal: causal row i is the mean of V[0..i], LSE = ln(i + 1)
    B, L, n_q, n_kv, d = 1, 50, 2, 1, 8
    _, k, v = _random_case(B, L, n_q, n_kv, d, seed=23)
    q = np.zeros((B, n_q, L, d), dtype=np.uint16)
    vv = _vals(v)[0, 0]
    o, l, _ = oracle.attention_rows(q, k, v, 0.5, True)
    o = o.reshape(n_q, L, d)
    l = l.reshape(n_q, L)
    means = np.cumsum(vv, axis=0) / np.arange(1, L + 1)[:, None]
    for h in range(n_q):
        assert np.max(np.abs(o[h] - means)) <= 1e-14
        assert np.max(np.abs(l[h] - np.log(np.arange(1, L + 1)))) <= 1e-14
    o, l, _ = oracle.attention_rows(q, k, v, 0.5, False)
    assert np.max(np.abs(o - vv.mean(axis=0))) <= 1e-14
    assert np.max(np.abs(l - math.log(L))) <= 1e-14


def test_causal_rows_are_noncausal_prefixes():
    B, L, n_q, n_kv, d = 1, 24, 2, 1, 8
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=24)
    oc, lc, _ = oracle.attention_rows(q, k, v, 0.3, True)
    oc = oc.reshape(n_q, L, d)
    lc = lc.reshape(n_q, L)
    onc, lnc, _ = oracle.attention_rows(q, k, v, 0.3, False)
    onc = onc.reshape(n_q, L, d)
    lnc = lnc.reshape(n_q, L)
    assert np.max(np.abs(oc[:, L - 1] - onc[:, L - 1])) <= 1e-15
    assert np.max(np.abs(lc[:, L - 1] - lnc[:, L - 1])) <= 1e-15
    assert np.max(np.abs(oc[:, :L - 1] - onc[:, :L - 1])) > 1e-3  # the mask matters
    for i in (0, 1, 7, 15, 22):
        op, lp, _ = oracle.attention_rows(
            np.ascontiguousarray(q[:, :, :i + 1]), np.ascontiguousarray(k[:, :, :i + 1]),
            np.ascontiguousarray(v[:, :, :i + 1]), 0.3, False)
        op = op.reshape(n_q, i + 1, d)
        lp = lp.reshape(n_q, i + 1)
        assert np.max(np.abs(op[:, i] - oc[:, i])) <= 1e-15
        assert np.max(np.abs(lp[:, i] - lc[:, i])) <= 1e-15


def test_gqa_equals_mha_with_repeated_kv():
    B, L, n_q, n_kv, d = 2, 31, 8, 2, 16
    g = n_q // n_kv
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=25)
    og, lg, _ = oracle.attention_rows(q, k, v, 0.25, True)
    kr = np.ascontiguousarray(np.repeat(k, g, axis=1))
    vr = np.ascontiguousarray(np.repeat(v, g, axis=1))
    om, lm, _ = oracle.attention_rows(q, kr, vr, 0.25, True)
    assert np.array_equal(og, om) and np.array_equal(lg, lm)
    # the other grouping (head h -> kv-head h mod n_kv) is a different model
    kt = np.ascontiguousarray(np.tile(k, (1, g, 1, 1)))
    vt = np.ascontiguousarray(np.tile(v, (1, g, 1, 1)))
    ot, _, _ = oracle.attention_rows(q, kt, vt, 0.25, True)
    assert np.max(np.abs(ot - og)) > 1e-3


def test_batch_independence():
    B, L, n_q, n_kv, d = 2, 17, 4, 2, 8
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=26)
    o, l, _ = oracle.attention_rows(q, k, v, 0.4, True)
    o = o.reshape(B, -1)
    l = l.reshape(B, -1)
    for b in range(B):
        ob, lb, _ = oracle.attention_rows(q[b:b + 1], k[b:b + 1], v[b:b + 1], 0.4, True)
        assert np.array_equal(ob.reshape(-1), o[b]) and np.array_equal(lb, l[b])


def test_selected_rows_match_full_run():
    B, L, n_q, n_kv, d = 1, 64, 6, 2, 16
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=27)
    o, l, f = oracle.attention_rows(q, k, v, 0.25, True)
    rows = inputs.sample_rows(B, n_q, L, 50, seed=3, block_rows=32)
    os_, ls, fs = oracle.attention_rows(q, k, v, 0.25, True, rows=rows)
    assert np.array_equal(os_, o[rows]) and np.array_equal(ls, l[rows])
    i = rows % L
    assert fs == int(np.sum(4 * d * (i + 1)))


# ----------------------------------------------------------------------------
# library special case: torch SDPA on the CPU in fp64 ("Long-Context
# Attention Explained": SDPA on a CPU matched the plain version to 4.4e-16,
# 8.9e-16 with is_causal=True)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("causal", [1, 0])
def test_torch_sdpa_fp64(causal):
    torch = pytest.importorskip("torch")
    B, L, n_q, n_kv, d = 2, 129, 8, 2, 64
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=31)
    scale = float(np.float32(1 / math.sqrt(d)))
    o, l, _ = oracle.attention_rows(q, k, v, scale, causal)
    tq, tk, tv = (torch.from_numpy(_vals(x)) for x in (q, k, v))
    g = n_q // n_kv
    tk_r = tk.repeat_interleave(g, dim=1)
    tv_r = tv.repeat_interleave(g, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        tq, tk_r, tv_r, is_causal=bool(causal), scale=scale)
    assert np.max(np.abs(o - ref.reshape(-1, d).numpy())) <= 1e-12
    s = torch.matmul(tq, tk_r.transpose(-1, -2).contiguous()) * scale
    if causal:
        mask = torch.ones(L, L, dtype=torch.bool).tril()
        s = s.masked_fill(~mask, float("-inf"))
    ref_lse = torch.logsumexp(s, dim=-1).reshape(-1).numpy()
    assert np.max(np.abs(l - ref_lse)) <= 1e-12


# ----------------------------------------------------------------------------
# exactness of the tiled algorithm: an independent fp64 tiled softmax with
# queries in the outer loop that folds per-tile partial results by their
# log-sum-exp ("Long-Context Attention Explained", sections "Tiling" and
# "Online softmax": partial statistics combine by rescaling), at the check
# ledger's block sizes, non-divisors of L included
# ----------------------------------------------------------------------------
def _tiled_online_softmax(qv, kv, vv, scale, causal, block):
    """One head, fp64, queries in the outer loop.  Each key tile yields a
    finished partial result for the block's rows (its own log-sum-exp and
    its normalised weighted sum of V), and the partials fold into a running
    pair (lse_run, o_run) by log-sum-exp: the new normaliser is
    logaddexp(lse_run, lse_tile) and each side's output is weighted by
    exp(its lse - the new one).  A row that sees no key of a tile contributes
    nothing from it."""
    L, d = qv.shape
    out = np.empty((L, d))
    lse = np.empty(L)
    for i0 in range(0, L, block):
        i1 = min(L, i0 + block)
        rows = np.arange(i0, i1)
        lse_run = np.full(i1 - i0, -np.inf)
        o_run = np.zeros((i1 - i0, d))
        key_end = i1 if causal else L       # keys past the block's last query stay unseen
        for j0 in range(0, key_end, block):
            j1 = min(L, j0 + block)
            logits = scale * (qv[i0:i1] @ kv[j0:j1].T)
            if causal:
                logits[np.arange(j0, j1)[None, :] > rows[:, None]] = -np.inf
            seen = np.any(np.isfinite(logits), axis=1)
            top = np.where(seen, logits.max(axis=1), 0.0)[:, None]
            mass = np.exp(logits - top).sum(axis=1)
            lse_tile = np.where(seen, top[:, 0] + np.log(np.where(seen, mass, 1.0)), -np.inf)
            o_tile = (np.exp(logits - top) @ vv[j0:j1]) / np.where(seen, mass, 1.0)[:, None]
            lse_new = np.logaddexp(lse_run, lse_tile)
            o_run = (np.exp(lse_run - lse_new)[:, None] * o_run
                     + np.exp(lse_tile - lse_new)[:, None] * o_tile)
            lse_run = lse_new
        out[i0:i1] = o_run
        lse[i0:i1] = lse_run
    return out, lse


def test_tiled_online_softmax_matches_oracle_ledger_bound():
    ledger = json.load(open(GOLDEN))["check_ledger"]["block_sizes_fp64"]
    L, d = ledger["N"], 64
    q, k, v = _random_case(1, L, 1, 1, d, seed=41)
    o, l, _ = oracle.attention_rows(q, k, v, 1 / math.sqrt(d), False)
    sc = float(np.float32(1 / math.sqrt(d)))
    for block in ledger["blocks"]:
        to, tl = _tiled_online_softmax(_vals(q)[0, 0], _vals(k)[0, 0], _vals(v)[0, 0],
                                       sc, False, block)
        # the ledger's bound holds for up to 32 partials per row; each further
        # fold rescales the running output once more, so the rounding error
        # may grow linearly with the number of folds (block 1: 1000 folds)
        folds = -(-L // block)
        bound = ledger["bound"] * max(1.0, folds / 32)
        assert np.max(np.abs(to - o)) <= bound, block
        assert np.max(np.abs(tl - l)) <= 1e-13


@pytest.mark.parametrize("block", [1, 7, 32, 64, 128, 200])
def test_tiled_online_softmax_causal(block):
    L, d = 200, 64
    q, k, v = _random_case(1, L, 1, 1, d, seed=42)
    sc = float(np.float32(0.125))
    o, l, _ = oracle.attention_rows(q, k, v, sc, True)
    to, tl = _tiled_online_softmax(_vals(q)[0, 0], _vals(k)[0, 0], _vals(v)[0, 0],
                                   sc, True, block)
    assert np.max(np.abs(to - o)) <= 1e-13
    assert np.max(np.abs(tl - l)) <= 1e-13


def test_ledger_example_magnitude():
    # the teaching run: N = 1024, d = 64, block 64, tiled vs plain differ by
    # rounding only (the page printed 3.9e-16 on its own inputs)
    ledger = json.load(open(GOLDEN))["check_ledger"]["tiled_vs_naive_fp64"]
    L, d = ledger["N"], ledger["d"]
    q, k, v = _random_case(1, L, 1, 1, d, seed=0)
    sc = float(np.float32(1 / math.sqrt(d)))
    o, _, _ = oracle.attention_rows(q, k, v, sc, False)
    to, _ = _tiled_online_softmax(_vals(q)[0, 0], _vals(k)[0, 0], _vals(v)[0, 0],
                                  sc, False, ledger["block"])
    assert np.max(np.abs(to - o)) <= 10 * ledger["max_abs"]


# ----------------------------------------------------------------------------
# flop count ("flops / prefill-attention": 2 * n_q * d_h * L^2 causal; the
# exact visible-pair count is L(L+1)/2 per head)
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("B,L,n_q,n_kv,d", [(1, 37, 4, 2, 8), (2, 64, 6, 3, 16)])
def test_flop_count(B, L, n_q, n_kv, d):
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=51)
    _, _, fc = oracle.attention_rows(q, k, v, 0.3, True)
    assert fc == 2 * B * n_q * d * L * (L + 1)
    page_f = 2 * n_q * d * L * L * B
    assert fc == page_f + page_f // L  # F * (1 + 1/L)
    _, _, fn = oracle.attention_rows(q, k, v, 0.3, False)
    assert fn == 4 * B * n_q * d * L * L


def test_large_scores_stay_finite():
    # Q x 20 pushes scores past 150 ("Long-Context Attention Explained",
    # check ledger: scores of 162 made an unsafe softmax produce NaN)
    B, L, n_q, n_kv, d = 1, 256, 2, 1, 64
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=61, mult=20.0)
    o, l, _ = oracle.attention_rows(q, k, v, 0.25, True)
    qv, kv = _vals(q)[0, 0], _vals(k)[0, 0]
    assert np.max(np.abs(qv @ kv.T * 0.25)) > 150
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))
    assert np.max(np.abs(o)) <= np.max(np.abs(_vals(v))) + 1e-12


def test_bad_arguments_rejected():
    q, k, v = _random_case(1, 4, 3, 2, 4, seed=1)  # 3 % 2 != 0
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, 0.5, True)
    q, k, v = _random_case(1, 4, 2, 1, 4, seed=1)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, float("nan"), True)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, k, v, 0.5, True, rows=np.array([8], dtype=np.int64))


# ----------------------------------------------------------------------------
# chunked prefill ("flops / prefill-attention", section "Workarounds": a long
# prompt processed in pieces; a piece's query i is token q_off + i of the
# sequence and, causally, sees every earlier token of the whole sequence)
# ----------------------------------------------------------------------------
def _random_chunk(B, Lq, Lk, n_q, n_kv, d, seed):
    q, _, _ = inputs.make_qkv(B, Lq, n_q, n_kv, d, seed)
    _, k, v = inputs.make_qkv(B, Lk, n_q, n_kv, d, seed + 1000)
    return q, k, v


CHUNK_TINY = [
    # B, Lq, Lk, q_off, n_q, n_kv, d, causal, scale
    (1, 3, 9, 6, 2, 1, 4, 1, 0.4),
    (2, 4, 7, 2, 4, 2, 3, 1, 0.8),
    (1, 1, 6, 5, 3, 1, 5, 1, 0.3),
    (1, 5, 5, 0, 2, 2, 4, 1, 0.6),
    (1, 4, 3, 0, 4, 2, 4, 0, 0.5),   # non-causal, fewer keys than queries
    (2, 3, 8, 0, 2, 1, 6, 0, 1.1),
]


@pytest.mark.parametrize("B,Lq,Lk,q_off,n_q,n_kv,d,causal,scale", CHUNK_TINY)
def test_chunk_brute_force_50_digits(B, Lq, Lk, q_off, n_q, n_kv, d, causal, scale):
    q, k, v = _random_chunk(B, Lq, Lk, n_q, n_kv, d, seed=300 + Lq * Lk + q_off)
    ref_o, ref_l = _brute_force(q, k, v, scale, causal, q_off=q_off)
    o, l, f = oracle.attention_rows_chunk(q, k, v, scale, causal, q_offset=q_off)
    assert np.max(np.abs(o - ref_o.reshape(-1, d))) <= 1e-14
    assert np.max(np.abs(l - ref_l.reshape(-1))) <= 1e-14
    vis = (q_off + np.arange(Lq) + 1) if causal else np.full(Lq, Lk)
    assert f == 4 * d * B * n_q * int(vis.sum())


def test_chunk_rows_are_rows_of_the_whole_sequence():
    # the last Lq queries of a causal sequence of length L, run as a chunk at
    # q_off = L - Lq over all L keys, are exactly those rows of the whole run
    B, L, n_q, n_kv, d = 2, 70, 4, 2, 16
    q, k, v = _random_case(B, L, n_q, n_kv, d, seed=71)
    o, l, _ = oracle.attention_rows(q, k, v, 0.3, True)
    o = o.reshape(B, n_q, L, d)
    l = l.reshape(B, n_q, L)
    for q_off in (0, 1, 31, 32, 69):
        qc = np.ascontiguousarray(q[:, :, q_off:])
        oc, lc, _ = oracle.attention_rows_chunk(qc, k, v, 0.3, True, q_offset=q_off)
        assert np.array_equal(oc.reshape(B, n_q, L - q_off, d), o[:, :, q_off:])
        assert np.array_equal(lc.reshape(B, n_q, L - q_off), l[:, :, q_off:])
    # keys past the chunk's last query are invisible: a causal middle chunk
    # reads only the prefix k[:, :, :q_off + Lq]
    q_off, Lq = 20, 17
    qc = np.ascontiguousarray(q[:, :, q_off:q_off + Lq])
    oc, lc, _ = oracle.attention_rows_chunk(qc, k, v, 0.3, True, q_offset=q_off)
    assert np.array_equal(oc.reshape(B, n_q, Lq, d), o[:, :, q_off:q_off + Lq])
    kp = np.ascontiguousarray(k[:, :, :q_off + Lq])
    vp = np.ascontiguousarray(v[:, :, :q_off + Lq])
    op, lp, _ = oracle.attention_rows_chunk(qc, kp, vp, 0.3, True, q_offset=q_off)
    assert np.array_equal(op, oc) and np.array_equal(lp, lc)


def test_chunk_zero_query_running_mean():
    # equal scores: row i of a causal chunk is the mean of V[0 .. q_off + i]
    Lq, Lk, q_off, d = 6, 40, 30, 8
    _, k, v = _random_chunk(1, Lq, Lk, 1, 1, d, seed=72)
    q = np.zeros((1, 1, Lq, d), dtype=np.uint16)
    o, l, _ = oracle.attention_rows_chunk(q, k, v, 0.5, True, q_offset=q_off)
    n = q_off + np.arange(Lq) + 1
    means = np.cumsum(_vals(v)[0, 0], axis=0)[q_off:q_off + Lq] / n[:, None]
    assert np.max(np.abs(o - means)) <= 1e-14
    assert np.max(np.abs(l - np.log(n))) <= 1e-14


def test_chunk_bad_arguments_rejected():
    q, k, v = _random_chunk(1, 4, 8, 2, 1, 4, seed=73)
    with pytest.raises(ValueError):
        oracle.attention_rows_chunk(q, k, v, 0.5, True, q_offset=5)   # 5 + 4 > 8
    with pytest.raises(ValueError):
        oracle.attention_rows_chunk(q, k, v, 0.5, True, q_offset=-1)
    with pytest.raises(ValueError):
        oracle.attention_rows_chunk(q, k, v, 0.5, False, q_offset=-1)
    oracle.attention_rows_chunk(q, k, v, 0.5, False, q_offset=100)  # unused when not causal


# ----------------------------------------------------------------------------
# merging partial results ("Long-Context Attention Explained", section
# "Online softmax": statistics of two key sets combine by rescaling both to
# the larger maximum; the LSE carries max and sum in one number)
# ----------------------------------------------------------------------------
def test_merge_prefix_and_chunk_equals_whole_row():
    # a chunk's causal attention over all keys = merge of (non-causal over the
    # keys before the chunk) and (causal over the chunk's own keys)
    B, Lq, q_off, n_q, n_kv, d = 2, 19, 45, 6, 2, 16
    Lk = q_off + Lq
    q, k, v = _random_chunk(B, Lq, Lk, n_q, n_kv, d, seed=74)
    o, l, _ = oracle.attention_rows_chunk(q, k, v, 0.2, True, q_offset=q_off)
    kp, vp = (np.ascontiguousarray(x[:, :, :q_off]) for x in (k, v))
    ks, vs = (np.ascontiguousarray(x[:, :, q_off:]) for x in (k, v))
    oa, la, _ = oracle.attention_rows_chunk(q, kp, vp, 0.2, False)
    ob, lb, _ = oracle.attention_rows_chunk(q, ks, vs, 0.2, True, q_offset=0)
    om, lm = oracle.merge_partials(oa, la, ob, lb)
    assert np.max(np.abs(om - o)) <= 1e-14
    assert np.max(np.abs(lm - l)) <= 1e-13
    # the merge is symmetric
    om2, lm2 = oracle.merge_partials(ob, lb, oa, la)
    assert np.max(np.abs(om2 - om)) <= 1e-15 and np.array_equal(lm2, lm)


def test_merge_closed_forms():
    rng = np.random.default_rng(75)
    o = rng.standard_normal((5, 8))
    l = rng.standard_normal(5) * 10
    # two copies of one partial: same output, LSE + ln 2
    om, lm = oracle.merge_partials(o, l, o, l)
    assert np.max(np.abs(om - o)) <= 1e-15
    assert np.max(np.abs(lm - (l + math.log(2)))) <= 1e-14
    # an empty side (LSE -inf) leaves the other exactly
    ninf = np.full(5, -np.inf)
    om, lm = oracle.merge_partials(o, l, np.full_like(o, np.nan), ninf)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    om, lm = oracle.merge_partials(np.zeros_like(o), ninf, o, l)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    # both empty: out 0, LSE -inf
    om, lm = oracle.merge_partials(o, ninf, o, ninf)
    assert np.array_equal(om, np.zeros_like(o)) and np.all(np.isneginf(lm))
    # LSEs far apart (beyond exp's range) still weigh correctly
    la = np.array([1000.0]); lb = np.array([0.0])
    om, lm = oracle.merge_partials(o[:1], la, o[1:2], lb)
    assert np.array_equal(om, o[:1]) and lm[0] == 1000.0
    # weights e^1 : e^0 against a hand-worked value
    om, lm = oracle.merge_partials(np.array([[1.0]]), np.array([1.0]),
                                   np.array([[0.0]]), np.array([0.0]))
    assert abs(om[0, 0] - math.e / (math.e + 1)) <= 1e-15
    assert abs(lm[0] - math.log(math.e + 1)) <= 1e-15


# ----------------------------------------------------------------------------
# decode ("Memory-bound vs compute-bound", sections "Prefill against decode"
# and "Attention itself": one new query against the whole cache): the query is
# token Lk - 1, so the chunk oracle with one query at q_offset = Lk - 1 is the
# decode; it sees every cached key, i.e. it is the non-causal single row
# ----------------------------------------------------------------------------
def test_decode_reading_of_the_chunk_oracle():
    B, Lk, n_q, n_kv, d = 2, 77, 6, 2, 16
    q, k, v = _random_chunk(B, 1, Lk, n_q, n_kv, d, seed=76)
    oc, lc, fc = oracle.attention_rows_chunk(q, k, v, 0.3, True, q_offset=Lk - 1)
    on, ln_, fn = oracle.attention_rows_chunk(q, k, v, 0.3, False)
    assert np.array_equal(oc, on) and np.array_equal(lc, ln_) and fc == fn == 4 * d * Lk * B * n_q
    # and it is the last row of a whole-sequence prefill whose last query is q
    qs = np.concatenate([np.zeros((B, n_q, Lk - 1, d), np.uint16), q], axis=2)
    ow, lw, _ = oracle.attention_rows(np.ascontiguousarray(qs), k, v, 0.3, True)
    ow = ow.reshape(B, n_q, Lk, d)[:, :, -1].reshape(-1, d)
    lw = lw.reshape(B, n_q, Lk)[:, :, -1].reshape(-1)
    assert np.array_equal(ow, oc) and np.array_equal(lw, lc)
