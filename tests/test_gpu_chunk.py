"""Chunked prefill and the partial-result merge on the HIP path vs the fp64
oracle, element by element, through the C ABI.

Chunked prefill: "flops / prefill-attention", section "Workarounds" (a long
prompt prefilled in pieces, each piece attending to every earlier token).
Merge: "Long-Context Attention Explained", section "Online softmax" (two sets
of row statistics combine by rescaling to the larger maximum).
"""
import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs
from causal_gqa_prefill_amd.configs import CHUNK_CONFIGS

from gpu_util import compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _run_chunk(qb, kb, vb, q_offset, scale, causal):
    import torch
    from causal_gqa_prefill_amd import attn_prefill_chunk_into
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    B, n_q, Lq, _ = q.shape
    out = torch.empty_like(q).fill_(float("nan"))
    lse = torch.empty((B, n_q, Lq), dtype=torch.float32, device=q.device).fill_(float("nan"))
    attn_prefill_chunk_into(q, k, v, out, lse, q_offset, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return from_dev_bf16(out), lse.cpu().numpy().astype(np.float64)


CHUNKS = [
    # B, Lq, Lk, q_offset, n_q, n_kv, d, causal
    (1, 1, 300, 299, 8, 2, 128, 1),      # one query at the end of the cache
    (1, 1, 300, 17, 4, 4, 64, 1),        # one query, many keys after it unused
    (1, 64, 1000, 936, 8, 1, 128, 1),
    (2, 100, 357, 200, 4, 2, 64, 1),     # middle chunk: keys past it are ignored
    (1, 257, 2048, 1791, 16, 2, 128, 1),
    (1, 129, 129, 0, 6, 3, 128, 1),      # the whole sequence as one chunk
    (1, 65, 1000, 33, 4, 2, 128, 1),     # offset not a multiple of any tile
    (1, 31, 7, 0, 4, 2, 128, 0),         # non-causal, fewer keys than queries
    (1, 200, 1500, 0, 6, 3, 128, 0),
    (1, 3, 5000, 0, 2, 1, 64, 0),
    (1, 1000, 5000, 3000, 8, 2, 128, 1),
    (3, 77, 500, 400, 6, 2, 64, 1),     # B = 3, d_h = 64, ragged chunk
    (2, 130, 400, 50, 12, 2, 128, 0),   # non-causal: the offset is unused
    (1, 256, 256, 0, 8, 4, 128, 0),
    (200, 100, 333, 200, 8, 2, 128, 1),  # 800 items: several chunk items per workgroup
    (300, 40, 90, 50, 2, 2, 64, 1),      # 600 items of 2 tiles each (MHA, d_h = 64)
]


@pytest.mark.parametrize("B,Lq,Lk,q_off,n_q,n_kv,d,causal", CHUNKS)
def test_chunk_parity(B, Lq, Lk, q_off, n_q, n_kv, d, causal):
    name = f"chunk B={B} Lq={Lq} Lk={Lk} q_off={q_off} n_q={n_q} n_kv={n_kv} d={d} causal={causal}"
    say(f"case {name}")
    scale = float(np.float32(1.0 / np.sqrt(d)))
    qb, kb, vb = inputs.make_chunk_qkv(B, Lq, Lk, n_q, n_kv, d, seed=Lq * 7 + Lk + q_off)
    o, l = _run_chunk(qb, kb, vb, q_off, scale, causal)
    ref_o, ref_l, _ = oracle.attention_rows_chunk(qb, kb, vb, scale, causal, q_offset=q_off)
    compare(name, o.reshape(-1, d), l.reshape(-1), ref_o, ref_l)


@pytest.mark.parametrize("cfg", CHUNK_CONFIGS, ids=[f"chunk{c.index}" for c in CHUNK_CONFIGS])
def test_chunk_workload_parity(cfg):
    say(f"chunk workload {cfg.index}: {cfg.describe()}")
    qb, kb, vb = inputs.make_chunk_qkv(cfg.B, cfg.Lq, cfg.Lk, cfg.n_q, cfg.n_kv, cfg.d_h,
                                       cfg.seed)
    o, l = _run_chunk(qb, kb, vb, cfg.q_offset, cfg.scale, cfg.causal)
    rows = inputs.sample_rows(cfg.B, cfg.n_q, cfg.Lq, cfg.sampled_rows, cfg.seed)
    ref_o, ref_l, _ = oracle.attention_rows_chunk(qb, kb, vb, cfg.scale, cfg.causal,
                                                  q_offset=cfg.q_offset, rows=rows)
    compare(f"chunk{cfg.index} sampled", o.reshape(-1, cfg.d_h)[rows], l.reshape(-1)[rows],
            ref_o, ref_l)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_chunk_with_dynamic_tail():
    """A causal chunk long enough for the schedule's dynamic tail (GQA-8,
    16384 queries at offset 16384 of 32768 keys: 4096 items, 16 rounds on
    256 CUs): every output element written (outputs start as NaN), 4096
    sampled rows against the oracle."""
    B, Lq, Lk, q_off, n_q, n_kv, d = 1, 16384, 32768, 16384, 64, 8, 128
    say(f"case chunk with dynamic tail Lq={Lq} Lk={Lk} q_off={q_off} n_q={n_q} n_kv={n_kv}")
    scale = float(np.float32(1.0 / np.sqrt(d)))
    qb, kb, vb = inputs.make_chunk_qkv(B, Lq, Lk, n_q, n_kv, d, seed=7300)
    o, l = _run_chunk(qb, kb, vb, q_off, scale, True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l)), "an output row was not written"
    rows = inputs.sample_rows(B, n_q, Lq, 4096, seed=7300)
    ref_o, ref_l, _ = oracle.attention_rows_chunk(qb, kb, vb, scale, True, q_offset=q_off, rows=rows)
    compare("chunk with dynamic tail", o.reshape(-1, d)[rows], l.reshape(-1)[rows], ref_o, ref_l)


def test_whole_sequence_chunk_is_bitwise_the_full_entry_point():
    import torch
    from causal_gqa_prefill_amd import attn_prefill, attn_prefill_chunk
    B, L, n_q, n_kv, d = 2, 777, 8, 2, 128
    say(f"case chunk(q_offset=0, Lq=Lk={L}) vs attn_prefill_fwd")
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=91)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    for causal in (True, False):
        o1, l1 = attn_prefill(q, k, v, causal=causal)
        o2, l2 = attn_prefill_chunk(q, k, v, 0, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)


def test_prompt_prefilled_in_chunks_matches_whole_prompt():
    # a 3000-token prompt in chunks of 1024: chunk c sees K/V[0 : end of c]
    import torch
    from causal_gqa_prefill_amd import attn_prefill_chunk
    B, L, n_q, n_kv, d, step = 1, 3000, 8, 2, 128, 1024
    say(f"case prompt L={L} in chunks of {step}")
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed=92)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    outs, lses = [], []
    for s0 in range(0, L, step):
        s1 = min(L, s0 + step)
        o, l = attn_prefill_chunk(q[:, :, s0:s1].contiguous(), k[:, :, :s1].contiguous(),
                                  v[:, :, :s1].contiguous(), s0)
        outs.append(o)
        lses.append(l)
    o = from_dev_bf16(torch.cat(outs, dim=2))
    l = torch.cat(lses, dim=2).cpu().numpy().astype(np.float64)
    rows = inputs.sample_rows(B, n_q, L, 3000, seed=92)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, float(np.float32(d ** -0.5)), True,
                                            rows=rows)
    compare("chunked prompt", o.reshape(-1, d)[rows], l.reshape(-1)[rows], ref_o, ref_l)


@pytest.mark.parametrize("B,Lq,q_off,n_q,n_kv,d", [(1, 500, 2000, 8, 2, 128),
                                                    (2, 70, 130, 4, 4, 64),
                                                    (1, 1, 4095, 6, 1, 128)])
def test_prefix_and_own_keys_merged_on_gpu(B, Lq, q_off, n_q, n_kv, d):
    # cached prefix (non-causal over keys [0, q_off)) and the chunk's own keys
    # (causal, offset 0) run separately, merged on the GPU = the chunk over all
    import torch
    from causal_gqa_prefill_amd import attn_prefill_chunk, merge_partials
    name = f"merge prefix={q_off} chunk={Lq} B={B} n_q={n_q} n_kv={n_kv} d={d}"
    say(f"case {name}")
    Lk = q_off + Lq
    qb, kb, vb = inputs.make_chunk_qkv(B, Lq, Lk, n_q, n_kv, d, seed=93 + Lq)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    oa, la = attn_prefill_chunk(q, k[:, :, :q_off].contiguous(), v[:, :, :q_off].contiguous(),
                                0, causal=False)
    ob, lb = attn_prefill_chunk(q, k[:, :, q_off:].contiguous(), v[:, :, q_off:].contiguous(),
                                0, causal=True)
    om, lm = merge_partials(oa, la, ob, lb)
    torch.cuda.synchronize()
    scale = float(np.float32(d ** -0.5))
    # each partial against the oracle first, then the merge
    kp, vp = (np.ascontiguousarray(x[:, :, :q_off]) for x in (kb, vb))
    ks, vs = (np.ascontiguousarray(x[:, :, q_off:]) for x in (kb, vb))
    ra_o, ra_l, _ = oracle.attention_rows_chunk(qb, kp, vp, scale, False)
    rb_o, rb_l, _ = oracle.attention_rows_chunk(qb, ks, vs, scale, True)
    compare(name + " prefix part", from_dev_bf16(oa).reshape(-1, d),
            la.cpu().numpy().astype(np.float64).reshape(-1), ra_o, ra_l)
    compare(name + " own part", from_dev_bf16(ob).reshape(-1, d),
            lb.cpu().numpy().astype(np.float64).reshape(-1), rb_o, rb_l)
    ref_o, ref_l, _ = oracle.attention_rows_chunk(qb, kb, vb, scale, True, q_offset=q_off)
    compare(name, from_dev_bf16(om).reshape(-1, d),
            lm.cpu().numpy().astype(np.float64).reshape(-1), ref_o, ref_l)


@pytest.mark.parametrize("rows,d,empty_every", [(1, 64, 0), (1000, 128, 0), (4099, 64, 7),
                                                (65536, 128, 5)])
def test_merge_kernel_vs_oracle(rows, d, empty_every):
    # bf16 partials merged in fp32 and rounded once to bf16: within one bf16
    # rounding (2^-8 relative) of the fp64 merge of the same bits, plus 1e-4 for
    # the fp32 weights (exp of an argument up to ~50 carries ~2e-6 relative
    # error, times |o_a - o_b| <= ~10)
    import torch
    from causal_gqa_prefill_amd import merge_partials
    say(f"case merge rows={rows} d={d} empty_every={empty_every}")
    oa_b, la, ob_b, lb = inputs.make_partials(rows, d, seed=rows + d, empty_every=empty_every)
    oa, ob = to_dev(oa_b), to_dev(ob_b)
    la_t = torch.from_numpy(la).cuda()
    lb_t = torch.from_numpy(lb).cuda()
    out = torch.empty_like(oa).fill_(float("nan"))
    lo = torch.empty_like(la_t).fill_(float("nan"))
    merge_partials(oa, la_t, ob, lb_t, out=out, lse_out=lo)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge_partials(inputs.bf16_to_f32(oa_b), la, inputs.bf16_to_f32(ob_b), lb)
    got_o = from_dev_bf16(out)
    got_l = lo.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(got_o))
    assert np.array_equal(np.isneginf(got_l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.all(np.isfinite(got_l[fin]))
    lerr = np.abs(got_l[fin] - ref_l[fin]) / np.maximum(1.0, np.abs(ref_l[fin]))
    oerr = np.abs(got_o - ref_o) - 2.0 ** -8 * np.abs(ref_o)
    say(f"  merge: max rel dLSE={lerr.max() if lerr.size else 0:.3e} "
        f"max |dO| beyond one bf16 rounding={oerr.max():.3e}")
    assert lerr.size == 0 or lerr.max() <= 1e-5
    assert oerr.max() <= 1e-4
    assert np.all(got_o[~fin] == 0.0)


def test_chunk_binding_errors():
    import torch
    from causal_gqa_prefill_amd import AttnPrefillError, attn_prefill_chunk, merge_partials
    say("case binding errors")
    q = torch.zeros((1, 4, 8, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(AttnPrefillError):
        attn_prefill_chunk(q, k, k.clone(), 9)            # 9 + 8 > 16
    with pytest.raises(AttnPrefillError):
        attn_prefill_chunk(q, k, k.clone(), -1)
    with pytest.raises(ValueError):
        attn_prefill_chunk(q, k, k[:, :, :8].contiguous(), 0)  # k and v differ
    o = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    l = torch.zeros((10,), dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError):
        merge_partials(o, l, o[:5].contiguous(), l[:5].contiguous())
    with pytest.raises(TypeError):
        merge_partials(o.float(), l, o, l)
