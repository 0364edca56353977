"""Decode (one new query per sequence against its whole K/V cache) on the HIP
path vs the fp64 oracle, element by element, through the C ABI.

The decode query is token Lk - 1 of its sequence, so the oracle is the chunk
oracle with one query at q_offset = Lk - 1 over the cache's first Lk rows
("Memory-bound vs compute-bound", sections "Prefill against decode" and
"Attention itself": one query vector against the whole cache).
"""
import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs
from causal_gqa_prefill_amd.configs import DECODE_CONFIGS

from gpu_util import compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _oracle_decode(qb, kb, vb, Lk, scale, rows=None):
    B, n_q, d = qb.shape
    q4 = np.ascontiguousarray(qb[:, :, None, :])
    k = np.ascontiguousarray(kb[:, :, :Lk])
    v = np.ascontiguousarray(vb[:, :, :Lk])
    return oracle.attention_rows_chunk(q4, k, v, scale, True, q_offset=Lk - 1, rows=rows)


def _run_decode(qb, kb, vb, Lk, scale, workspace=None, stream=None):
    import torch
    from causal_gqa_prefill_amd import attn_decode_into
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out = torch.empty_like(q).fill_(float("nan"))
    lse = torch.empty(tuple(q.shape[:2]), dtype=torch.float32, device=q.device).fill_(float("nan"))
    attn_decode_into(q, k, v, out, lse, Lk=Lk, scale=scale, workspace=workspace, stream=stream)
    torch.cuda.synchronize()
    return from_dev_bf16(out), lse.cpu().numpy().astype(np.float64)


DECODES = [
    # B, Lk, capacity, n_q, n_kv, d
    (1, 1, 1, 4, 4, 64),
    (1, 5, 9, 8, 2, 128),
    (2, 63, 64, 6, 3, 128),
    (1, 64, 100, 4, 1, 64),
    (1, 65, 65, 2, 2, 128),
    (3, 257, 300, 8, 8, 128),
    (1, 1000, 1000, 32, 1, 128),     # 32 query heads on one key/value head
    (2, 4097, 4200, 16, 2, 128),
    (1, 12345, 12345, 12, 2, 64),
    (5, 3000, 3001, 5, 5, 64),
    (1, 70000, 70000, 8, 1, 128),
    (300, 100, 100, 4, 1, 64),      # many short sequences
    (3, 4095, 5000, 24, 3, 128),    # g = 8, Lk one short of a tile multiple
    (2, 33, 40, 12, 12, 128),       # MHA decode, Lk just past one tile
    (1, 257, 257, 6, 2, 64),
    (1, 40000, 40000, 8, 1, 64),    # d_h = 64 with 313 key ranges: two combine chunks
]


@pytest.mark.parametrize("B,Lk,cap,n_q,n_kv,d", DECODES)
def test_decode_parity(B, Lk, cap, n_q, n_kv, d):
    name = f"decode B={B} Lk={Lk} cap={cap} n_q={n_q} n_kv={n_kv} d={d}"
    say(f"case {name}")
    scale = float(np.float32(1.0 / np.sqrt(d)))
    qb, kb, vb = inputs.make_decode_qkv(B, Lk, n_q, n_kv, d, seed=Lk + 13 * cap + d,
                                        capacity=cap)
    o, l = _run_decode(qb, kb, vb, Lk, scale)
    ref_o, ref_l, _ = _oracle_decode(qb, kb, vb, Lk, scale)
    compare(name, o.reshape(-1, d), l.reshape(-1), ref_o, ref_l)


@pytest.mark.parametrize("cfg", DECODE_CONFIGS, ids=[f"decode{c.index}" for c in DECODE_CONFIGS])
def test_decode_workload_parity(cfg):
    say(f"decode workload {cfg.index}: {cfg.describe()}")
    qb, kb, vb = inputs.make_decode_qkv(cfg.B, cfg.Lk, cfg.n_q, cfg.n_kv, cfg.d_h, cfg.seed)
    o, l = _run_decode(qb, kb, vb, cfg.Lk, cfg.scale)
    o = o.reshape(-1, cfg.d_h)
    l = l.reshape(-1)
    rows = None
    if cfg.sampled_rows:
        rows = np.sort(np.random.default_rng(cfg.seed + 7).choice(
            cfg.B * cfg.n_q, size=cfg.sampled_rows, replace=False)).astype(np.int64)
    ref_o, ref_l, _ = _oracle_decode(qb, kb, vb, cfg.Lk, cfg.scale, rows=rows)
    if rows is not None:
        compare(f"decode{cfg.index} sampled", o[rows], l[rows], ref_o, ref_l)
    else:
        compare(f"decode{cfg.index}", o, l, ref_o, ref_l)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_decode_matches_last_row_of_prefill():
    # the decode of token L-1 and the last row of a causal prefill of L tokens
    # compute the same thing by different kernels: both within tolerance of
    # the oracle, and close to each other
    import torch
    from causal_gqa_prefill_amd import attn_decode, attn_prefill
    B, L, n_q, n_kv, d = 2, 1500, 8, 2, 128
    say(f"case decode vs prefill last row, L={L}")
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=95)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    op, lp = attn_prefill(q, k, v)
    od, ld = attn_decode(q[:, :, L - 1].contiguous(), k, v)
    torch.cuda.synchronize()
    diff = (op[:, :, L - 1].float() - od.float()).abs().max().item()
    ldiff = (lp[:, :, L - 1] - ld).abs().max().item()
    say(f"  prefill vs decode: max|dO|={diff:.3e} max|dLSE|={ldiff:.3e}")
    assert diff <= 2e-2 and ldiff <= 1e-3


def test_decode_shared_workspace_two_calls_and_stream():
    # one workspace for two calls in a row (the second smaller), on a
    # non-default stream; each result must match the oracle
    import torch
    from causal_gqa_prefill_amd import binding
    say("case shared workspace, two calls, side stream")
    d = 128
    big = (2, 9000, 16, 4, d)
    small = (1, 700, 8, 2, d)
    need = max(binding.decode_workspace_bytes(*big), binding.decode_workspace_bytes(*small))
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    scale = float(np.float32(d ** -0.5))
    for (B, Lk, n_q, n_kv, _) in (big, small):
        qb, kb, vb = inputs.make_decode_qkv(B, Lk, n_q, n_kv, d, seed=96 + Lk)
        with torch.cuda.stream(side):
            o, l = _run_decode(qb, kb, vb, Lk, scale, workspace=ws, stream=side)
        ref_o, ref_l, _ = _oracle_decode(qb, kb, vb, Lk, scale)
        compare(f"shared workspace B={B} Lk={Lk}", o.reshape(-1, d), l.reshape(-1), ref_o, ref_l)


def test_decode_binding_errors():
    import torch
    from causal_gqa_prefill_amd import AttnPrefillError, attn_decode, binding
    say("case decode binding errors")
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnPrefillError):
        attn_decode(q, k, k.clone(), Lk=65)                   # capacity 64 < Lk
    with pytest.raises(AttnPrefillError):
        attn_decode(q, k, k.clone(), workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    q66 = torch.zeros((1, 66, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnPrefillError):
        attn_decode(q66, k, k.clone())                        # 33 heads per kv head
    with pytest.raises(ValueError):
        attn_decode(q[:, :, :64].contiguous(), k, k.clone())  # head size mismatch
    assert binding.decode_workspace_bytes(1, 64, 8, 2, 128) > 0
