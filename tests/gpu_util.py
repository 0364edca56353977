"""Helpers for GPU parity tests: upload bf16 bits, run the HIP path through
the C ABI binding, compare with the fp64 oracle at the stated tolerances."""
import sys

import numpy as np

from causal_gqa_prefill_amd import inputs

# O: max abs <= 2e-2 and mean abs <= 1e-3 (bf16 output); LSE: abs <= 1e-3
O_MAX_ABS = 2e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits, device="cuda:0"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).to(device)


def from_dev_bf16(t):
    import torch
    return inputs.bf16_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def run_gpu(qb, kb, vb, scale, causal, poison=True, stream=None):
    """HIP path on bf16 bits; returns (out f64 [B,n_q,L,d], lse f64 [B,n_q,L])."""
    import torch
    from causal_gqa_prefill_amd import attn_prefill_into
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    B, n_q, L, d = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, n_q, L), dtype=torch.float32, device=q.device)
    if poison:  # every element must be overwritten
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    attn_prefill_into(q, k, v, out, lse, scale=scale, causal=causal, stream=stream)
    torch.cuda.synchronize()
    return from_dev_bf16(out), lse.cpu().numpy().astype(np.float64)


def compare(name, o_gpu_rows, l_gpu_rows, o_ref, l_ref):
    """Element-wise comparison of selected rows against the oracle."""
    assert np.all(np.isfinite(o_gpu_rows)), f"{name}: non-finite output"
    assert np.all(np.isfinite(l_gpu_rows)), f"{name}: non-finite lse"
    err = np.abs(o_gpu_rows - o_ref)
    lerr = np.abs(l_gpu_rows - l_ref)
    say(f"  {name}: rows={len(l_ref)} max|dO|={err.max():.3e} mean|dO|={err.mean():.3e} "
        f"max|dLSE|={lerr.max():.3e}")
    assert err.max() <= O_MAX_ABS, f"{name}: max abs {err.max()}"
    assert err.mean() <= O_MEAN_ABS, f"{name}: mean abs {err.mean()}"
    assert lerr.max() <= LSE_MAX_ABS, f"{name}: lse abs {lerr.max()}"
    return err.max(), err.mean(), lerr.max()
