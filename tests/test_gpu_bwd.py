"""Backward pass on the HIP path vs the fp64 oracle, element by element,
through the C ABI ("Long-Context Attention Explained", section "What
FlashAttention does not change": gradients recomputed from the saved LSE).

The kernels receive the oracle's output rounded to bf16 and its LSE rounded
to fp32, so the comparison isolates the backward arithmetic.  Contract: every
element of dQ, dK and dV within the oracle's per-element rounding bound (P
recomputed in fp32, delta from the bf16 output, P and dS rounded to bf16,
fp32 accumulation, one bf16 rounding of the result; pinned on the CPU by a
simulation), delta within its own bound.
"""
import numpy as np
import pytest

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


def _run_case(B, L, n_q, n_kv, d, causal, seed, q_rows=None, k_rows=None, label=""):
    """Oracle stats and outputs for (all or sampled) rows, GPU backward with the
    oracle's O (bf16) and LSE (fp32), compare."""
    import torch
    from causal_gqa_prefill_amd import attn_prefill_backward
    scale = float(np.float32(d ** -0.5))
    q, k, v = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
    do = inputs.make_qkv(B, L, n_q, n_kv, d, seed + 500)[0]
    name = label or f"bwd B={B} L={L} n_q={n_q} n_kv={n_kv} causal={causal}"
    say(f"case {name}")
    o, lse_o, _ = oracle.attention_rows(q, k, v, scale, causal)
    lse, delta, absd = oracle.attention_bwd_rowstats(q, k, v, do, scale, causal)
    o_bits = inputs.bf16_bits(o.astype(np.float32)).reshape(q.shape)
    tq, tk, tv, tdo, to = (to_dev(x) for x in (q, k, v, do, o_bits))
    tl = torch.from_numpy(lse_o.astype(np.float32).reshape(B, n_q, L)).cuda()
    dq, dk, dv, dl = attn_prefill_backward(tq, tk, tv, to, tl, tdo, scale=scale, causal=causal)
    torch.cuda.synchronize()
    dq = from_dev_bf16(dq).reshape(-1, d)
    dk = from_dev_bf16(dk).reshape(-1, d)
    dv = from_dev_bf16(dv).reshape(-1, d)
    dl = dl.cpu().numpy().astype(np.float64).reshape(-1)
    if q_rows is None:
        q_rows = np.arange(B * n_q * L)
    if k_rows is None:
        k_rows = np.arange(B * n_kv * L)
    rq, bq = oracle.attention_bwd_dq(q, k, v, do, scale, causal, lse, delta, q_rows, absd)
    rk, rv, bk, bv = oracle.attention_bwd_dkdv(q, k, v, do, scale, causal, lse, delta, k_rows,
                                               absd)
    _check(name + " dQ", dq[q_rows], rq, bq)
    _check(name + " dK", dk[k_rows], rk, bk)
    _check(name + " dV", dv[k_rows], rv, bv)
    # delta from the bf16 output: within (2^-8 + 2^-16) sum |dO O| of the exact one
    d_bound = (2.0 ** -8 + 2.0 ** -16) * absd + 1e-6
    _check(name + " delta", dl, delta, d_bound)


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


@pytest.mark.parametrize("index", [2, 3])
def test_bwd_workload_group_parity(index):
    # one key/value group of the workload at full length (groups are
    # independent), sampled rows: 512 query rows and 256 key rows
    cfg = config(index)
    g = cfg.n_q // cfg.n_kv
    rng = np.random.default_rng(cfg.seed + 9)
    q_rows = np.sort(rng.choice(g * cfg.L, 512, replace=False))
    k_rows = np.sort(rng.choice(cfg.L, 256, replace=False))
    q_rows = np.union1d(q_rows, [0, cfg.L - 1, g * cfg.L - 1])
    k_rows = np.union1d(k_rows, [0, 127, 128, cfg.L - 1])
    _run_case(1, cfg.L, g, 1, cfg.d_h, cfg.causal, cfg.seed, q_rows, k_rows,
              label=f"bwd config{index} one group (L={cfg.L}, g={g})")


def test_bwd_pipeline_and_errors():
    # forward then backward on the GPU: gradients close to the isolated run;
    # deterministic; errors raise
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
    ref = oracle.attention_bwd(q, k, v, do, float(np.float32(d ** -0.5)), 1)
    for name, gpu, exact in (("dQ", g1[0], ref[0]), ("dK", g1[1], ref[1]), ("dV", g1[2], ref[2])):
        got = from_dev_bf16(gpu)
        rel = np.max(np.abs(got - exact)) / np.max(np.abs(exact))
        say(f"  pipeline {name}: max|d| / max|ref| = {rel:.3e}")
        assert rel <= 2e-2
    with pytest.raises(AttnPrefillError):
        attn_prefill_backward(tq, tk, tv, out, lse, tdo, scale=float("nan"))
    with pytest.raises(ValueError):
        attn_prefill_backward(tq, tk, tv, out, lse[:, :4].contiguous(), tdo)
