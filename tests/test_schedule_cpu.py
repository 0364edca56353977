"""The forward kernels' work list and static schedule, through the library's
host diagnostic attn_prefill_schedule (the same list code the kernels run),
on the CPU: every work item computed exactly once, whether the rounds run all
static (as under graph capture) or hand the list's end to the dynamic tail;
balanced pairs of equal causal length; runs of one to three (batch, kv-head)
streams per XCD; the tail heavy first.  The work and its balance follow
"Long-Context Attention Explained" (causal work per query block, and its
balance over thread blocks); the list itself is this library's."""
import numpy as np
import pytest

from causal_gqa_prefill_amd import binding
from causal_gqa_prefill_amd.configs import config


def _check(B, Lq, Lk, q_offset, n_q, n_kv, d_h, causal, n_cu):
    info, lst, rounds = binding.schedule(B, Lq, Lk, q_offset, n_q, n_kv, d_h, causal, n_cu)
    n_items, grid, n_qblk = info["n_items"], info["grid"], info["n_qblk"]
    ipq, sg, pair_t, r_static = info["items_per_qblk"], info["sg"], info["pair_t"], info["r_static"]
    g = n_q // n_kv
    hwg = 8 if g % 8 == 0 else 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    ngroups = g // hwg
    assert n_qblk == -(-Lq // (256 // hwg)) and ipq == B * n_kv * ngroups
    assert n_items == ipq * n_qblk and grid == min(n_items, n_cu)
    # the list is a bijection onto (q-block, head group, stream)
    key = (lst[:, 0].astype(np.int64) * ngroups + lst[:, 1]) * (B * n_kv) + lst[:, 2]
    assert lst[:, 0].min() >= 0 and lst[:, 0].max() < n_qblk
    assert lst[:, 1].min() >= 0 and lst[:, 1].max() < ngroups
    assert lst[:, 2].min() >= 0 and lst[:, 2].max() < B * n_kv
    assert np.unique(key).size == n_items
    # all rounds static: every list entry exactly once
    flat = rounds.ravel()
    got = flat[flat >= 0]
    assert got.size == n_items and np.array_equal(np.sort(got), np.arange(n_items))
    # with the dynamic tail: the static rounds hold entries 0 .. r_static grid - 1
    # exactly (the tail draws the rest in list order)
    stat = rounds[:r_static].ravel()
    if r_static * grid < n_items:
        assert (stat >= 0).all()   # a tail follows: the static rounds are full
    stat = stat[stat >= 0]
    assert np.array_equal(np.sort(stat), np.arange(min(r_static * grid, n_items)))
    if pair_t > 0:
        assert causal == 1 and sg > 0
        pr = info["pair_rounds"]
        assert pr == r_static and pr % 2 == 0 and pr * grid < n_items
        qb = lst[:, 0]
        heavy, light = qb[rounds[0:pr:2]], qb[rounds[1:pr:2]]
        # each workgroup's two members: one pair, equal causal sums
        assert (heavy + light == n_qblk - 1 + pair_t).all()
        assert (lst[rounds[0:pr:2], 2] == lst[rounds[1:pr:2], 2]).all()
        assert (lst[rounds[0:pr:2], 1] == lst[rounds[1:pr:2], 1]).all()
        assert (light >= pair_t).all() and (heavy >= light).all()
        # the tail: q-blocks below pair_t, heavy first
        tail = qb[pr * grid:]
        assert (tail < pair_t).all() and (np.diff(tail) <= 0).all()
        assert tail.size == pair_t * ipq
    if sg > 0 and grid % 8 == 0 and (pair_t > 0 or sg < n_qblk) and B * n_kv > 1:
        # a run of G / 8 consecutive entries per XCD and round: one or two
        # streams, up to four where a short last super-group cuts the runs
        counts = [np.unique(lst[rounds[r, x::8], 2]).size for r in range(r_static) for x in range(8)]
        assert max(counts) <= 4 and np.mean(counts) <= 2.2, (max(counts), np.mean(counts))
    return info


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5, 6])
def test_config_schedules(idx):
    c = config(idx)
    info = _check(c.B, c.L, c.L, 0, c.n_q, c.n_kv, c.d_h, 1, 256)
    # the list forms the launches use on a 256-CU MI355X
    expect = {2: (8, 0), 4: (32, 320), 5: (10, 256)}
    if idx in expect:
        assert (info["sg"], info["pair_t"]) == expect[idx]
    if idx == 5:
        assert info["pair_rounds"] == 54 and info["n_items"] == 18432


@pytest.mark.parametrize("n_cu", [256, 304, 80, 64, 8, 7, 1])
def test_grid_sizes(n_cu):
    _check(1, 32768, 32768, 0, 64, 8, 128, 1, n_cu)
    _check(2, 9000, 9000, 0, 24, 4, 64, 1, n_cu)


def test_chunk_and_noncausal():
    _check(1, 16384, 49152, 32768, 64, 8, 128, 1, 256)   # a late chunk, balanced pairs
    _check(1, 5000, 20000, 15000, 36, 6, 128, 1, 256)
    _check(2, 16384, 16384, 0, 32, 8, 128, 0, 256)       # non-causal: no pairs
    info = _check(1, 65536, 65536, 0, 32, 8, 128, 0, 256)
    assert info["pair_t"] == 0


def test_random_shapes():
    rng = np.random.default_rng(11)
    n_pairs = 0
    for _ in range(120):
        hwg_g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        n_kv = int(rng.choice([1, 2, 4, 6, 8]))
        B = int(rng.choice([1, 1, 2, 3]))
        Lq = int(rng.integers(1, 40000))
        causal = int(rng.integers(0, 2))
        q_off = int(rng.integers(0, 3000)) if causal else 0
        info = _check(B, Lq, Lq + q_off, q_off, n_kv * hwg_g, n_kv, int(rng.choice([64, 128])), causal,
                      int(rng.choice([256, 256, 248, 80])))
        n_pairs += info["pair_t"] > 0
    assert n_pairs >= 10


def test_schedule_errors():
    with pytest.raises(binding.AttnPrefillError):
        binding.schedule(1, 100, 100, 0, 6, 4, 128, 1, 256)      # n_q % n_kv
    with pytest.raises(binding.AttnPrefillError):
        binding.schedule(1, 100, 100, 0, 8, 4, 96, 1, 256)       # d_h
    with pytest.raises(binding.AttnPrefillError):
        binding.schedule(1, 100, 100, 1, 8, 4, 128, 1, 256)      # q_offset + Lq > Lk
    with pytest.raises(binding.AttnPrefillError):
        binding.schedule(1, 100, 100, 0, 8, 4, 128, 1, 0)        # n_cu
