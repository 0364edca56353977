"""Both tile configurations of the forward kernel against the oracle and
against each other, and guard canaries after every output buffer.

The forward kernel is built for two MFMA shapes: v_mfma_f32_32x32x16_bf16
(the default) and v_mfma_f32_16x16x32_bf16 (selected with the environment
variable ATTN_PREFILL_MFMA=16, read at each launch).  They lay scores and
accumulators out differently and sum in different orders, so their outputs
differ by rounding only: each must meet the oracle tolerances on its own.

Canaries: every output is the head of a larger buffer whose tail holds a
known bit pattern; after the call the tail must be unchanged (no kernel may
write past its output)."""
import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs

from gpu_util import compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu

CANARY = 4096          # elements of guard after each output
PATTERN = 0x5A5A       # bf16 bits of the guard (a finite value no kernel writes by chance)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _guarded(shape, dtype):
    """(tensor of `shape` at the head of a larger buffer, the buffer, guard
    slice).  The tensor is NaN-poisoned, the guard filled with PATTERN."""
    import torch
    n = int(np.prod(shape))
    buf = torch.empty(n + CANARY, dtype=dtype, device="cuda")
    if dtype == torch.bfloat16:
        buf.view(torch.int16).fill_(PATTERN)
    else:
        buf.view(torch.int32).fill_(PATTERN | (PATTERN << 16))
    head = buf[:n].view(shape)
    head.fill_(float("nan"))
    return head, buf, slice(n, n + CANARY)


def _guard_intact(buf, sl):
    import torch
    tail = buf[sl]
    if tail.dtype == torch.bfloat16:
        return bool(torch.all(tail.view(torch.int16) == PATTERN))
    return bool(torch.all(tail.view(torch.int32) == (PATTERN | (PATTERN << 16))))


def _fwd(qb, kb, vb, scale, causal, mfma, monkeypatch):
    """One forward call with the given MFMA shape into guarded outputs."""
    import torch
    from causal_gqa_prefill_amd import attn_prefill_into
    monkeypatch.setenv("ATTN_PREFILL_MFMA", str(mfma))
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    B, n_q, L, d = q.shape
    out, obuf, osl = _guarded((B, n_q, L, d), torch.bfloat16)
    lse, lbuf, lsl = _guarded((B, n_q, L), torch.float32)
    attn_prefill_into(q, k, v, out, lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert _guard_intact(obuf, osl), f"mfma {mfma}: write past the output"
    assert _guard_intact(lbuf, lsl), f"mfma {mfma}: write past the lse"
    return from_dev_bf16(out).reshape(-1, d), lse.cpu().numpy().astype(np.float64).reshape(-1)


CASES = [
    # B, L, n_q, n_kv, d, causal
    (1, 128, 4, 4, 64, 1),       # the tiny causal MHA workload
    (1, 1, 4, 4, 128, 1),
    (1, 65, 16, 2, 128, 1),
    (2, 257, 3, 1, 128, 1),
    (1, 1000, 8, 1, 128, 1),
    (1, 4097, 6, 6, 64, 1),
    (2, 300, 4, 4, 128, 0),
    (1, 777, 16, 4, 128, 0),
    (160, 260, 8, 1, 128, 1),    # many items per persistent workgroup
    (64, 700, 2, 1, 64, 1),
    (4, 2048, 32, 32, 128, 1),   # the Llama-2-7B-shaped layer
]


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", CASES)
def test_both_mfma_shapes_against_oracle_and_each_other(B, L, n_q, n_kv, d, causal, monkeypatch):
    scale = float(np.float32(1.0 / np.sqrt(d)))
    say(f"case tile configs B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal}")
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=6000 + L + n_q)
    o32, l32 = _fwd(qb, kb, vb, scale, causal, 32, monkeypatch)
    o16, l16 = _fwd(qb, kb, vb, scale, causal, 16, monkeypatch)
    total = B * n_q * L
    rows = None if total <= 70000 else inputs.sample_rows(B, n_q, L, 4096, seed=L)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, scale, causal, rows=rows)
    sel = slice(None) if rows is None else rows
    compare("32x32x16", o32[sel], l32[sel], ref_o, ref_l)
    compare("16x16x32", o16[sel], l16[sel], ref_o, ref_l)
    say(f"  32x32 vs 16x16: max|dO|={np.max(np.abs(o32 - o16)):.3e} "
        f"max|dLSE|={np.max(np.abs(l32 - l16)):.3e}")


def test_both_mfma_shapes_on_the_gqa6_128k_layer(monkeypatch):
    """The 128K-token GQA-6 layer with the 16x16 shape (the default shape
    is checked at this size by the workload parity tests), 4096 seeded rows."""
    from causal_gqa_prefill_amd.configs import config
    cfg = config(5)
    say(f"16x16 on {cfg.describe()}")
    qb, kb, vb = inputs.make_config_qkv(cfg)
    o16, l16 = _fwd(qb, kb, vb, cfg.scale, cfg.causal, 16, monkeypatch)
    rows = inputs.sample_rows(cfg.B, cfg.n_q, cfg.L, cfg.sampled_rows, cfg.seed)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, cfg.scale, cfg.causal, rows=rows)
    compare("16x16x32 config5 sampled", o16[rows], l16[rows], ref_o, ref_l)


def test_guards_after_chunk_merge_decode_fp8_bwd_outputs(monkeypatch):
    """Every other entry point writes exactly its outputs."""
    import torch
    from causal_gqa_prefill_amd import (attn_decode_into, attn_prefill_backward,
                                        attn_prefill_chunk_into, attn_prefill_fp8_into,
                                        merge_partials)
    monkeypatch.delenv("ATTN_PREFILL_MFMA", raising=False)
    say("case guards after chunk / merge / decode / fp8 / backward outputs")
    # chunk
    qb, kb, vb = inputs.make_chunk_qkv(1, 300, 1000, 8, 2, 128, seed=71)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out, ob, osl = _guarded(tuple(q.shape), torch.bfloat16)
    lse, lb, lsl = _guarded(tuple(q.shape[:3]), torch.float32)
    attn_prefill_chunk_into(q, k, v, out, lse, 700)
    torch.cuda.synchronize()
    assert _guard_intact(ob, osl) and _guard_intact(lb, lsl), "chunk"
    assert bool(torch.all(torch.isfinite(out.float()))) and bool(torch.all(torch.isfinite(lse)))
    # merge
    oa, la, obb, lbb = inputs.make_partials(5000, 64, seed=72, empty_every=7)
    oa_t, ob_t = to_dev(oa), to_dev(obb)
    la_t, lb_t = torch.from_numpy(la).cuda(), torch.from_numpy(lbb).cuda()
    mo, mb, msl = _guarded((5000, 64), torch.bfloat16)
    ml, mlb, mlsl = _guarded((5000,), torch.float32)
    merge_partials(oa_t, la_t, ob_t, lb_t, out=mo, lse_out=ml)
    torch.cuda.synchronize()
    assert _guard_intact(mb, msl) and _guard_intact(mlb, mlsl), "merge"
    # decode
    qd, kd, vd = inputs.make_decode_qkv(3, 5000, 16, 2, 128, seed=73, capacity=5100)
    qd_t, kd_t, vd_t = to_dev(qd), to_dev(kd), to_dev(vd)
    do_, dob, dosl = _guarded(tuple(qd_t.shape), torch.bfloat16)
    dl, dlb, dlsl = _guarded((3, 16), torch.float32)
    attn_decode_into(qd_t, kd_t, vd_t, do_, dl, Lk=5000)
    torch.cuda.synchronize()
    assert _guard_intact(dob, dosl) and _guard_intact(dlb, dlsl), "decode"
    # fp8
    q8, k8, v8, s_q, s_k, s_v = inputs.make_fp8_qkv(1, 500, 500, 8, 2, 128, seed=74)
    q8t, k8t, v8t = (torch.from_numpy(x).cuda() for x in (q8, k8, v8))
    fo, fob, fosl = _guarded((1, 8, 500, 128), torch.bfloat16)
    fl, flb, flsl = _guarded((1, 8, 500), torch.float32)
    attn_prefill_fp8_into(q8t, k8t, v8t, fo, fl, s_q, s_k, s_v)
    torch.cuda.synchronize()
    assert _guard_intact(fob, fosl) and _guard_intact(flb, flsl), "fp8"
    # backward
    qb2, kb2, vb2 = inputs.make_qkv(1, 400, 8, 2, 128, seed=75)
    dob2 = inputs.make_qkv(1, 400, 8, 2, 128, seed=76)[0]
    q2, k2, v2, do2 = (to_dev(x) for x in (qb2, kb2, vb2, dob2))
    from causal_gqa_prefill_amd import attn_prefill
    o2, l2 = attn_prefill(q2, k2, v2)
    gq, gqb, gqsl = _guarded(tuple(q2.shape), torch.bfloat16)
    gk, gkb, gksl = _guarded(tuple(k2.shape), torch.bfloat16)
    gv, gvb, gvsl = _guarded(tuple(v2.shape), torch.bfloat16)
    gd, gdb, gdsl = _guarded(tuple(q2.shape[:3]), torch.float32)
    attn_prefill_backward(q2, k2, v2, o2, l2, do2, grads=(gq, gk, gv, gd))
    torch.cuda.synchronize()
    for name, b_, s_ in (("dq", gqb, gqsl), ("dk", gkb, gksl), ("dv", gvb, gvsl),
                         ("delta", gdb, gdsl)):
        assert _guard_intact(b_, s_), f"backward {name}"
