"""attn_decode_fwd_noalloc (the decode on the library's static device scratch,
for callers that cannot allocate) against attn_decode_fwd with a caller
workspace, through the C ABI: the same kernels run on the same inputs, so the
outputs must agree bit for bit.  Two calls in a row, the second smaller than
the first (the scratch keeps the first call's partials, which must not leak
into the second); each output is also checked against the fp64 oracle at the
decode tolerances."""
import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs

from gpu_util import compare, from_dev_bf16, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _oracle_decode(qb, kb, vb, Lk, scale):
    q4 = np.ascontiguousarray(qb[:, :, None, :])
    k = np.ascontiguousarray(kb[:, :, :Lk])
    v = np.ascontiguousarray(vb[:, :, :Lk])
    return oracle.attention_rows_chunk(q4, k, v, scale, True, q_offset=Lk - 1)


def _both(B, Lk, cap, n_q, n_kv, d, seed):
    """(noalloc out, lse), (workspace out, lse) as raw bits / fp32, on one stream."""
    import torch
    from causal_gqa_prefill_amd import binding
    qb, kb, vb = inputs.make_decode_qkv(B, Lk, n_q, n_kv, d, seed, capacity=cap)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    scale = float(np.float32(1.0 / np.sqrt(d)))
    stream = torch.cuda.current_stream()
    outs = []
    for use_scratch in (True, False):
        out = torch.empty_like(q).fill_(float("nan"))
        lse = torch.empty((B, n_q), dtype=torch.float32, device=q.device).fill_(float("nan"))
        if use_scratch:
            st = binding.decode_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                            out.data_ptr(), lse.data_ptr(), B, Lk, cap, n_q,
                                            n_kv, d, scale, stream.cuda_stream)
        else:
            need = binding.decode_workspace_bytes(B, Lk, n_q, n_kv, d)
            ws = torch.empty(need, dtype=torch.uint8, device=q.device)
            st = binding.decode_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                    lse.data_ptr(), B, Lk, cap, n_q, n_kv, d, scale,
                                    ws.data_ptr(), need, stream.cuda_stream)
        assert st == 0, binding.strerror(st)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy().copy(), lse.cpu().numpy().copy()))
    return outs, (qb, kb, vb, Lk, scale)


def _check_pair(B, Lk, cap, n_q, n_kv, d, seed):
    from causal_gqa_prefill_amd import binding
    need = binding.decode_workspace_bytes(B, Lk, n_q, n_kv, d)
    say(f"noalloc decode: B={B} Lk={Lk} cap={cap} n_q={n_q} n_kv={n_kv} d={d}, workspace "
        f"{need} B of the {binding.decode_scratch_bytes()} B scratch")
    assert 0 < need <= binding.decode_scratch_bytes()
    (scr, ws), (qb, kb, vb, Lk, scale) = _both(B, Lk, cap, n_q, n_kv, d, seed)
    (o_s, l_s), (o_w, l_w) = scr, ws
    assert np.array_equal(o_s, o_w), "outputs differ from the workspace entry point"
    assert np.array_equal(l_s.view(np.uint32), l_w.view(np.uint32)), "LSEs differ"
    ref_o, ref_l, _ = _oracle_decode(qb, kb, vb, Lk, scale)
    o = inputs.bf16_to_f32(o_s.view(np.uint16)).astype(np.float64).reshape(-1, d)
    compare(f"noalloc B={B} Lk={Lk} n_q={n_q} n_kv={n_kv} d={d}", o,
            l_s.reshape(-1).astype(np.float64), ref_o, ref_l)


def test_noalloc_two_calls_second_smaller():
    # a batch at 8K context (about 0.25 MB of partials), then a smaller call
    _check_pair(8, 8192, 8192, 32, 8, 128, seed=4200)
    _check_pair(2, 300, 320, 8, 2, 64, seed=4201)


def test_noalloc_rejects_sizes_past_the_scratch():
    """Too large for the scratch: an error, nothing enqueued (the pointers are
    real, small tensors; validation fails before any of them is used)."""
    import torch
    from causal_gqa_prefill_amd import binding
    B, Lk, n_q, n_kv, d = 2048, 4096, 64, 8, 128
    assert binding.decode_workspace_bytes(B, Lk, n_q, n_kv, d) > binding.decode_scratch_bytes()
    far = 1 << 40   # sizes far larger than these buffers: never dereferenced
    base = torch.empty(64, dtype=torch.uint8, device="cuda:0")
    p = base.data_ptr()
    st = binding.decode_noalloc_raw(p, p + far, p + 2 * far, p + 3 * far, p + 4 * far, B, Lk, Lk,
                                    n_q, n_kv, d, 0.088, torch.cuda.current_stream().cuda_stream)
    assert st == 14, binding.strerror(st)
