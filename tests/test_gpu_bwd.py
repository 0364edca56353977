"""Backward pass on the HIP path vs the fp64 oracle, element by element,
through the C ABI ("Long-Context Attention Explained", section "What
FlashAttention does not change": gradients recomputed from the saved LSE).

The kernels receive the oracle's output rounded to bf16 and its LSE rounded
to fp32 for every query row the checked gradients depend on, so the
comparison isolates the backward arithmetic.  Contract: every checked element
of dQ, dK and dV within the per-element rounding bound of tests/bounds.py (P
recomputed in fp32, delta from the bf16 output, P and dS rounded to bf16,
fp32 sums charged one rounding per term over their true lengths, one bf16
rounding of the result; pinned on the CPU by a simulation that accumulates
in fp32), delta within its own bound.
"""
import numpy as np
import pytest

import bounds
import oracle
from causal_gqa_prefill_amd import inputs
from causal_gqa_prefill_amd.configs import config

from gpu_util import from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _check(name, got, ref, bound):
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite"
    ratio = np.max(err / (bound + 1e-30))
    say(f"  {name}: n={ref.size} max|d|={err.max():.3e} mean|d|={err.mean():.3e} "
        f"max|ref|={np.abs(ref).max():.3e} max err/bound={ratio:.3f}")
    assert np.all(err <= bound + 1e-7), f"{name}: {np.sum(err > bound + 1e-7)} past the bound"


def _run_case(B, L, n_q, n_kv, d, causal, seed, q_rows=None, k_rows=None, label="",
              groups=None):
    """Oracle statistics of the query rows the checked gradients depend on,
    GPU backward fed the oracle's O (bf16) and LSE (fp32) for those rows (the
    other rows hold O = 0, LSE = 0: finite, never read by a checked
    gradient), then dQ on q_rows and dK, dV on k_rows (flat ids; None: every
    row of the checked groups) against the oracle within the bounds.
    groups: (b, kv-head) pairs to check (None: all)."""
    import torch
    from causal_gqa_prefill_amd import attn_prefill_backward
    scale = float(np.float32(d ** -0.5))
    g = n_q // n_kv
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
    do = inputs.make_qkv(B, L, n_q, n_kv, d, seed + 500)[0]
    name = label or f"bwd B={B} L={L} n_q={n_q} n_kv={n_kv} causal={causal}"
    say(f"case {name}")
    if groups is None:
        groups = [(b, h) for b in range(B) for h in range(n_kv)]
    if q_rows is None:
        q_rows = np.concatenate([((b * n_q + kvh * g + hh) * L + np.arange(L))
                                 for b, kvh in groups for hh in range(g)])
    if k_rows is None:
        k_rows = np.concatenate([((b * n_kv + kvh) * L + np.arange(L)) for b, kvh in groups])
    q_rows, k_rows = np.asarray(q_rows), np.asarray(k_rows)
    # query rows the checked gradients read: the dQ rows, and every row of
    # the group that sees a checked key
    parts = [q_rows]
    kb, kh, kj = k_rows // (n_kv * L), (k_rows // L) % n_kv, k_rows % L
    for b, kvh in {(int(x), int(y)) for x, y in zip(kb, kh)}:
        i0 = int(kj[(kb == b) & (kh == kvh)].min()) if causal else 0
        for hh in range(g):
            parts.append((b * n_q + kvh * g + hh) * L + np.arange(i0, L))
    need = np.unique(np.concatenate(parts)).astype(np.int64)
    say(f"  oracle statistics for {need.size} query rows")
    o_rows, lse_rows, delta_rows = oracle.attention_bwd_rowstats(q, k, v, do, scale, causal,
                                                                 rows=need)
    n_all = B * n_q * L
    o_full = np.zeros((n_all, d))
    lse_full = np.full(n_all, np.nan)
    delta_full = np.full(n_all, np.nan)
    o_full[need], lse_full[need], delta_full[need] = o_rows, lse_rows, delta_rows
    o_bits = inputs.bf16_bits(o_full.astype(np.float32)).reshape(q.shape)
    lse_dev = np.where(np.isnan(lse_full), 0.0, lse_full).astype(np.float32).reshape(B, n_q, L)
    tq, tk, tv, tdo, to = (to_dev(x) for x in (q, k, v, do, o_bits))
    tl = torch.from_numpy(lse_dev).cuda()
    dq, dk, dv, dl = attn_prefill_backward(tq, tk, tv, to, tl, tdo, scale=scale, causal=causal)
    torch.cuda.synchronize()
    dq = from_dev_bf16(dq).reshape(-1, d)
    dk = from_dev_bf16(dk).reshape(-1, d)
    dv = from_dev_bf16(dv).reshape(-1, d)
    dl = dl.cpu().numpy().astype(np.float64).reshape(-1)
    rq = oracle.attention_bwd_dq(q, k, v, do, scale, causal, lse_full, delta_full, q_rows)
    rk, rv = oracle.attention_bwd_dkdv(q, k, v, do, scale, causal, lse_full, delta_full, k_rows)
    # the bounds, group by group
    qv, kv_, vv, dov = (inputs.bf16_to_f32(x).astype(np.float64) for x in (q, k, v, do))
    ov = o_full.reshape(B, n_q, L, d)
    bq = np.empty_like(rq)
    bk = np.empty_like(rk)
    bv = np.empty_like(rv)
    for b, kvh in groups:
        hs = slice(kvh * g, kvh * g + g)
        grp = bounds.BwdGroup(qv[b, hs], kv_[b, kvh], vv[b, kvh], dov[b, hs], ov[b, hs],
                              lse_full.reshape(B, n_q, L)[b, hs],
                              delta_full.reshape(B, n_q, L)[b, hs], scale, causal)
        sel = np.nonzero((q_rows // (n_q * L) == b) & ((q_rows // L) % n_q // g == kvh))[0]
        if sel.size:
            bq[sel] = grp.dq_bound((q_rows[sel] // L) % n_q - kvh * g, q_rows[sel] % L, rq[sel])
        sel = np.nonzero((k_rows // (n_kv * L) == b) & ((k_rows // L) % n_kv == kvh))[0]
        if sel.size:
            bk[sel], bv[sel] = grp.dkdv_bound(k_rows[sel] % L, rk[sel], rv[sel])
    _check(name + " dQ", dq[q_rows], rq, bq)
    _check(name + " dK", dk[k_rows], rk, bk)
    _check(name + " dV", dv[k_rows], rv, bv)
    # delta from the bf16 output, on the rows fed the oracle's output
    d_bound = bounds.bwd_delta_bound(dov.reshape(-1, d)[need], o_rows) + 1e-6
    _check(name + " delta", dl[need], delta_rows, d_bound)


SHAPES = [
    # B, L, n_q, n_kv, d, causal
    (1, 1, 4, 4, 128, 1),
    (1, 31, 4, 2, 128, 1),
    (1, 64, 8, 2, 128, 1),
    (2, 129, 6, 3, 128, 1),
    (1, 130, 4, 4, 128, 0),
    (1, 257, 8, 1, 128, 1),
    (1, 300, 16, 2, 128, 0),
    (1, 1000, 4, 2, 128, 1),
    (1, 1, 2, 1, 64, 1),
    (1, 128, 4, 4, 64, 1),      # the tiny causal MHA workload's shape
    (2, 200, 6, 2, 64, 1),
    (1, 333, 8, 8, 64, 0),
    # grids of more key blocks than three rounds of the CUs: the dK/dV kernel
    # with one group of waves per workgroup (smaller grids use two)
    (200, 256, 2, 2, 64, 1),    # 800 key blocks
    (150, 384, 4, 2, 128, 1),   # 900 key blocks
    (150, 256, 2, 2, 128, 0),   # 600 non-causal key blocks
    (100, 384, 4, 2, 64, 1),    # 600 causal key blocks: two groups per block, several rounds
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", SHAPES)
def test_bwd_parity(B, L, n_q, n_kv, d, causal):
    _run_case(B, L, n_q, n_kv, d, causal, seed=200 + L + n_q + d)


@pytest.mark.parametrize("index", [2, 3, 4, 5])
def test_bwd_workload_group_parity(index):
    # one key/value group of the workload at full length (groups are
    # independent): 512 sampled query rows and 256 sampled key rows.  For the
    # 128K-token GQA-6 layer the key rows come from the last 2048 positions,
    # so that the oracle needs the statistics of 6 x 2048 query rows instead
    # of the whole layer's; its dQ rows are anywhere (each needs only its own
    # statistics), so the full-length key sums of dQ are checked there, and the
    # full-length query sums of dK and dV at the 32K-token GQA-8 layer.
    cfg = config(index)
    g = cfg.n_q // cfg.n_kv
    L = cfg.L
    rng = np.random.default_rng(cfg.seed + 9)
    q_rows = np.sort(rng.choice(g * L, 512, replace=False))
    q_rows = np.union1d(q_rows, [0, L - 1, g * L - 1])
    if index == 5:
        k_rows = np.sort(rng.choice(np.arange(L - 2048, L), 256, replace=False))
        k_rows = np.union1d(k_rows, [L - 2048, L - 1])
    else:
        k_rows = np.sort(rng.choice(L, 256, replace=False))
        k_rows = np.union1d(k_rows, [0, 127, 128, L - 1])
    _run_case(1, L, g, 1, cfg.d_h, cfg.causal, cfg.seed, q_rows, k_rows,
              label=f"bwd config{index} one group (L={L}, g={g})")


def test_bwd_pipeline_and_errors():
    # forward then backward on the GPU: every gradient element within the
    # rounding bound of the oracle's backward at the forward's own O and LSE
    # (and within 2% of the largest exact gradient); deterministic; errors raise
    import torch
    from causal_gqa_prefill_amd import AttnPrefillError, attn_prefill, attn_prefill_backward
    say("case bwd pipeline")
    B, L, n_q, n_kv, d = 1, 777, 8, 2, 128
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, 301)
    do = inputs.make_qkv(B, L, n_q, n_kv, d, 302)[0]
    tq, tk, tv, tdo = (to_dev(x) for x in (q, k, v, do))
    out, lse = attn_prefill(tq, tk, tv)
    g1 = attn_prefill_backward(tq, tk, tv, out, lse, tdo)
    g2 = attn_prefill_backward(tq, tk, tv, out, lse, tdo)
    torch.cuda.synchronize()
    for a, b_ in zip(g1, g2):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_)
    scale = float(np.float32(d ** -0.5))
    ref = oracle.attention_bwd(q, k, v, do, scale, 1)
    for name, gpu, exact in (("dQ", g1[0], ref[0]), ("dK", g1[1], ref[1]), ("dV", g1[2], ref[2])):
        got = from_dev_bf16(gpu)
        rel = np.max(np.abs(got - exact)) / np.max(np.abs(exact))
        say(f"  pipeline {name}: max|d| / max|ref| = {rel:.3e}")
        assert rel <= 2e-2
    # element by element: the oracle's gradients at the forward's own output
    # and LSE (P from that LSE, delta = dO . O from that bf16 output) are what
    # the backward kernels compute up to their rounding, so the per-element
    # bound applies to the whole forward -> backward chain
    o_fwd = from_dev_bf16(out).reshape(B, n_q, L, d)
    lse_fwd = lse.cpu().numpy().astype(np.float64).reshape(B, n_q, L)
    dov = inputs.bf16_to_f32(do).astype(np.float64)
    delta_fwd = np.sum(dov * o_fwd, axis=-1)
    rows_q = np.arange(B * n_q * L, dtype=np.int64)
    rows_k = np.arange(B * n_kv * L, dtype=np.int64)
    rq = oracle.attention_bwd_dq(q, k, v, do, scale, 1, lse_fwd.reshape(-1), delta_fwd.reshape(-1),
                                 rows_q)
    rk, rv = oracle.attention_bwd_dkdv(q, k, v, do, scale, 1, lse_fwd.reshape(-1),
                                       delta_fwd.reshape(-1), rows_k)
    qv, kv_, vv = (inputs.bf16_to_f32(x).astype(np.float64) for x in (q, k, v))
    g = n_q // n_kv
    bq = np.empty_like(rq)
    bk = np.empty_like(rk)
    bv = np.empty_like(rv)
    for kvh in range(n_kv):
        hs = slice(kvh * g, kvh * g + g)
        grp = bounds.BwdGroup(qv[0, hs], kv_[0, kvh], vv[0, kvh], dov[0, hs], o_fwd[0, hs],
                              lse_fwd[0, hs], delta_fwd[0, hs], scale, 1)
        sel = np.arange(kvh * g * L, (kvh + 1) * g * L)
        bq[sel] = grp.dq_bound(sel // L - kvh * g, sel % L, rq[sel])
        sel = np.arange(kvh * L, (kvh + 1) * L)
        bk[sel], bv[sel] = grp.dkdv_bound(sel % L, rk[sel], rv[sel])
    _check("pipeline dQ", from_dev_bf16(g1[0]).reshape(-1, d), rq, bq)
    _check("pipeline dK", from_dev_bf16(g1[1]).reshape(-1, d), rk, bk)
    _check("pipeline dV", from_dev_bf16(g1[2]).reshape(-1, d), rv, bv)
    with pytest.raises(AttnPrefillError):
        attn_prefill_backward(tq, tk, tv, out, lse, tdo, scale=float("nan"))
    with pytest.raises(ValueError):
        attn_prefill_backward(tq, tk, tv, out, lse[:, :4].contiguous(), tdo)
