"""FP8 (OCP e4m3) prefill on the HIP path vs the fp64 oracle, element by
element, through the C ABI ("flops / prefill-attention", section
"Workarounds", FP8 attention).

Contract: the oracle runs the plain attention on the exactly decoded inputs
(times their descale factors), so the rounding the kernel adds beyond the
bf16 path's is P rounded to e4m3 before P V.  Each output element must lie
within the per-element bound of tests/bounds.py for the kernel's arithmetic
(2^-4 sum_j P_j |v_j| + 2^-10 max_j P_j sum_j |v_j| for the e4m3 weights,
the fp32 sums charged one rounding per term over their true lengths, one
bf16 rounding of O); LSE (from unrounded weights) within 1e-3 absolute, the
bf16 path's bar.
"""
import numpy as np
import pytest

import bounds
import oracle
from causal_gqa_prefill_amd import inputs
from causal_gqa_prefill_amd.configs import CONFIGS, CHUNK_CONFIGS

from gpu_util import LSE_MAX_ABS, from_dev_bf16, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _dev8(codes):
    import torch
    return torch.from_numpy(np.ascontiguousarray(codes)).to("cuda")


def _run_fp8(q8, k8, v8, dq, dk, dv, scale, causal, q_offset=0):
    import torch
    from causal_gqa_prefill_amd import attn_prefill_fp8_into
    q, k, v = _dev8(q8), _dev8(k8), _dev8(v8)
    B, n_q, Lq, d = q.shape
    out = torch.empty((B, n_q, Lq, d), dtype=torch.bfloat16, device="cuda").fill_(float("nan"))
    lse = torch.empty((B, n_q, Lq), dtype=torch.float32, device="cuda").fill_(float("nan"))
    attn_prefill_fp8_into(q, k, v, out, lse, dq, dk, dv, q_offset=q_offset, scale=scale,
                          causal=causal)
    torch.cuda.synchronize()
    return from_dev_bf16(out), lse.cpu().numpy().astype(np.float64)


def fp8_reference(q8, k8, v8, scale, dq, dk, dv, causal, q_off, rows=None):
    """The oracle's rows and the test-side rounding bound of each element."""
    ref_o, ref_l, _ = oracle.attention_rows_chunk_fp8(q8, k8, v8, scale, dq, dk, dv, causal,
                                                      q_off, rows=rows)
    if rows is None:
        rows = np.arange(q8.shape[0] * q8.shape[1] * q8.shape[2])
    bound = bounds.fp8_rows_bound(q8, k8, v8, dq, dk, dv, float(np.float32(scale)), ref_l,
                                  rows, causal, q_off, oracle.e4m3_table())
    return ref_o, ref_l, bound


def compare_fp8(name, o, l, ref_o, ref_l, bound):
    assert np.all(np.isfinite(o)), f"{name}: non-finite output"
    assert np.all(np.isfinite(l)), f"{name}: non-finite lse"
    err = np.abs(o - ref_o)
    allowed = bound + 1e-6
    lerr = np.abs(l - ref_l)
    say(f"  {name}: rows={len(ref_l)} max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
        f"max err/allowed={np.max(err / allowed):.3f} max|dLSE|={lerr.max():.3e}")
    assert np.all(err <= allowed), f"{name}: {np.sum(err > allowed)} elements past the bound"
    assert lerr.max() <= LSE_MAX_ABS, f"{name}: lse abs {lerr.max()}"
    return err


SHAPES = [
    # B, Lq, Lk, q_offset, n_q, n_kv, causal
    (1, 1, 1, 0, 4, 4, 1),
    (1, 63, 63, 0, 8, 2, 1),
    (1, 64, 64, 0, 4, 1, 1),
    (1, 65, 65, 0, 16, 2, 1),
    (2, 129, 129, 0, 6, 3, 1),
    (1, 130, 130, 0, 8, 8, 0),
    (1, 257, 257, 0, 12, 2, 1),
    (1, 1000, 1000, 0, 8, 1, 1),
    (1, 1, 300, 299, 8, 2, 1),
    (2, 100, 357, 200, 4, 2, 1),
    (1, 65, 1000, 33, 4, 2, 1),
    (1, 31, 7, 0, 4, 2, 0),
    (1, 4097, 4097, 0, 4, 4, 1),
    (2, 300, 1000, 700, 12, 2, 1),      # g = 6 (two heads per workgroup), B = 2
    (1, 129, 2000, 0, 8, 2, 0),         # non-causal chunk
    (1, 2048, 8192, 6144, 16, 2, 1),    # a long chunk at an offset
    (160, 260, 260, 0, 8, 1, 1),        # 1440 work items: several per persistent workgroup
    (300, 40, 90, 50, 2, 2, 1),         # 600 chunk items of one or two tiles (MHA)
    (4, 2048, 2048, 0, 16, 16, 1),      # whole heads per XCD and round: 4 heads, 2 rounds
    (8, 1024, 1024, 0, 32, 8, 1),       # whole heads per XCD and round: 2 heads, 4 rounds
]


@pytest.mark.parametrize("B,Lq,Lk,q_off,n_q,n_kv,causal", SHAPES)
def test_fp8_parity(B, Lq, Lk, q_off, n_q, n_kv, causal):
    d = 128
    name = f"fp8 B={B} Lq={Lq} Lk={Lk} q_off={q_off} n_q={n_q} n_kv={n_kv} causal={causal}"
    say(f"case {name}")
    scale = float(np.float32(d ** -0.5))
    q8, k8, v8, dq, dk, dv = inputs.make_fp8_qkv(B, Lq, Lk, n_q, n_kv, d, seed=Lq + 3 * Lk + q_off)
    o, l = _run_fp8(q8, k8, v8, dq, dk, dv, scale, causal, q_off)
    rows = None
    if B * n_q * Lq * Lk > 500_000_000:   # else every row (the oracle takes seconds at most)
        rows = inputs.sample_rows(B, n_q, Lq, 4096, seed=Lq)
    ref_o, ref_l, bound = fp8_reference(q8, k8, v8, scale, dq, dk, dv, causal, q_off, rows)
    o = o.reshape(-1, d)
    l = l.reshape(-1)
    if rows is not None:
        o, l = o[rows], l[rows]
    compare_fp8(name, o, l, ref_o, ref_l, bound)


# the d_h = 128 workloads, the 128K-token GQA-6 layer included
FP8_CONFIGS = [c for c in CONFIGS if c.d_h == 128]


@pytest.mark.parametrize("cfg", FP8_CONFIGS, ids=[f"config{c.index}" for c in FP8_CONFIGS])
def test_fp8_config_parity(cfg):
    say(f"fp8 config {cfg.index}: {cfg.describe()}")
    q8, k8, v8, dq, dk, dv = inputs.make_fp8_qkv(cfg.B, cfg.L, cfg.L, cfg.n_q, cfg.n_kv,
                                                 cfg.d_h, cfg.seed)
    o, l = _run_fp8(q8, k8, v8, dq, dk, dv, cfg.scale, cfg.causal)
    rows = inputs.sample_rows(cfg.B, cfg.n_q, cfg.L, 4096, cfg.seed)
    ref_o, ref_l, bound = fp8_reference(q8, k8, v8, cfg.scale, dq, dk, dv, cfg.causal, 0, rows)
    compare_fp8(f"fp8 config{cfg.index} sampled", o.reshape(-1, cfg.d_h)[rows],
                l.reshape(-1)[rows], ref_o, ref_l, bound)
    # every element written (outputs start as NaN): configs 4 and 5 hand the
    # last rounds of their schedule out dynamically, and an item the counter
    # skipped would leave NaN behind
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "an output row was not written"


def test_fp8_chunk_workload_parity():
    cfg = CHUNK_CONFIGS[0]
    say(f"fp8 chunk workload: {cfg.describe()}")
    q8, k8, v8, dq, dk, dv = inputs.make_fp8_qkv(cfg.B, cfg.Lq, cfg.Lk, cfg.n_q, cfg.n_kv,
                                                 cfg.d_h, cfg.seed)
    o, l = _run_fp8(q8, k8, v8, dq, dk, dv, cfg.scale, cfg.causal, cfg.q_offset)
    rows = inputs.sample_rows(cfg.B, cfg.n_q, cfg.Lq, 2048, cfg.seed)
    ref_o, ref_l, bound = fp8_reference(q8, k8, v8, cfg.scale, dq, dk, dv, cfg.causal,
                                        cfg.q_offset, rows)
    compare_fp8("fp8 chunk1 sampled", o.reshape(-1, cfg.d_h)[rows], l.reshape(-1)[rows],
                ref_o, ref_l, bound)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "an output row was not written"


def test_fp8_chunk_with_dynamic_tail():
    """The FP8 kernel on a causal chunk long enough for the schedule's
    dynamic tail (GQA-8, 16384 queries at offset 16384 of 32768 keys: 16
    rounds on 256 CUs): every output element written, 4096 sampled rows
    within the rounding bound."""
    B, Lq, Lk, q_off, n_q, n_kv, d = 1, 16384, 32768, 16384, 64, 8, 128
    say(f"case fp8 chunk with dynamic tail Lq={Lq} Lk={Lk} q_off={q_off}")
    scale = float(np.float32(d ** -0.5))
    q8, k8, v8, dq, dk, dv = inputs.make_fp8_qkv(B, Lq, Lk, n_q, n_kv, d, seed=7400)
    o, l = _run_fp8(q8, k8, v8, dq, dk, dv, scale, 1, q_off)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "an output row was not written"
    rows = inputs.sample_rows(B, n_q, Lq, 4096, seed=7400)
    ref_o, ref_l, bound = fp8_reference(q8, k8, v8, scale, dq, dk, dv, 1, q_off, rows)
    compare_fp8("fp8 chunk with dynamic tail", o.reshape(-1, d)[rows], l.reshape(-1)[rows],
                ref_o, ref_l, bound)


def test_fp8_deterministic_and_errors():
    import torch
    from causal_gqa_prefill_amd import AttnPrefillError, attn_prefill_fp8
    say("case fp8 determinism and errors")
    q8, k8, v8, dq, dk, dv = inputs.make_fp8_qkv(1, 777, 777, 8, 2, 128, seed=97)
    q, k, v = _dev8(q8), _dev8(k8), _dev8(v8)
    o1, l1 = attn_prefill_fp8(q, k, v, dq, dk, dv)
    o2, l2 = attn_prefill_fp8(q, k, v, dq, dk, dv)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    with pytest.raises(AttnPrefillError):
        attn_prefill_fp8(q[..., :64].contiguous(), k[..., :64].contiguous(),
                         v[..., :64].contiguous(), dq, dk, dv)          # d_h 64 unsupported
    with pytest.raises(AttnPrefillError):
        attn_prefill_fp8(q, k, v, dq, dk, dv, q_offset=1)               # 1 + 777 > 777
    with pytest.raises(TypeError):
        attn_prefill_fp8(q.to(torch.int16), k, v, dq, dk, dv)
