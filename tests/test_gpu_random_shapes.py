"""Seeded random shapes through the C ABI against the oracle: the bf16
forward (whole sequences and chunks), the FP8 forward and the backward.

The hand-picked shapes of test_gpu_parity.py cover the edges one by one;
this sweep draws batch, sequence length, head counts, group size, head size
and mask at random (seeded) so that combinations nobody thought of are
checked too, among them shapes whose persistent schedule takes stream
blocks (whole heads per XCD and round) and shapes with partial last rounds.
For the bf16 forward one seeded row of every 32-row block of every head is
compared, so every work item of the launch is, within the forward's stated
tolerances; the FP8 and backward cases compare every element within the
rounding bounds of tests/bounds.py."""
import numpy as np
import pytest

import oracle
from causal_gqa_prefill_amd import inputs

from gpu_util import compare, from_dev_bf16, run_gpu, say, to_dev

pytestmark = pytest.mark.gpu

N_CU = 256   # MI355X; only used to pick shapes that take stream blocks


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from causal_gqa_prefill_amd import binding
    binding.library()  # raises if the HIP library is missing: no fallback


def _stream_blocks(B, L, n_q, n_kv):
    """Whether a launch of this shape on N_CU CUs takes whole heads per XCD and
    round (the selection the library's launch code makes for short
    sequences), for labelling and picking cases only."""
    g = n_q // n_kv
    hwg = 8 if g % 8 == 0 else 4 if g % 4 == 0 else 2 if g % 2 == 0 else 1
    n_qblk = -(-L // (256 // hwg))
    per_qblk = B * n_kv * (g // hwg)
    n_items = per_qblk * n_qblk
    grid = min(n_items, N_CU)
    if grid % 8:
        return False
    slots = grid // 8
    return (slots % n_qblk == 0 and per_qblk % (8 * (slots // n_qblk)) == 0
            and (n_items // grid) % 2 == 0)


def _draw(rng):
    d = int(rng.choice([64, 128]))
    g = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
    n_kv = int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.choice([1, 2, 3, 4, 8, 16]))
    L = int(rng.choice([1, 31, 64, 100, 257, 512, 777, 1024, 2048, 3000, 4096]))
    causal = int(rng.random() < 0.8)
    return B, L, g * n_kv, n_kv, d, causal


def _cases(n_random, n_blocks, seed):
    """n_random shapes as drawn, then n_blocks more drawn until they take
    stream blocks; the work of each bounded so the oracle takes seconds."""
    rng = np.random.default_rng(seed)
    out, blocks = [], []
    while len(out) < n_random or len(blocks) < n_blocks:
        B, L, n_q, n_kv, d, causal = _draw(rng)
        if B * n_q * L * L > 3e9:
            continue
        if len(out) < n_random:
            out.append((B, L, n_q, n_kv, d, causal))
        elif _stream_blocks(B, L, n_q, n_kv):
            blocks.append((B, L, n_q, n_kv, d, causal))
    return out + blocks


CASES = _cases(20, 8, seed=9100)


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", CASES)
def test_random_shape(B, L, n_q, n_kv, d, causal):
    scale = float(np.float32(1.0 / np.sqrt(d)))
    seed = 9200 + B * 7 + L * 3 + n_q + d + causal
    label = (f"random B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal}"
             f"{' (stream blocks)' if _stream_blocks(B, L, n_q, n_kv) else ''}")
    say(f"case {label}")
    qb, kb, vb = inputs.make_qkv(B, L, n_q, n_kv, d, seed)
    o, l = run_gpu(qb, kb, vb, scale, causal)
    rng = np.random.default_rng(seed + 1)
    blocks = np.arange(0, B * n_q * L, 32, dtype=np.int64)
    span = np.minimum(32, B * n_q * L - blocks)
    rows = blocks + (rng.random(blocks.size) * span).astype(np.int64)
    ref_o, ref_l, _ = oracle.attention_rows(qb, kb, vb, scale, causal, rows=rows)
    compare(label, o.reshape(-1, d)[rows], l.reshape(-1)[rows], ref_o, ref_l)


def _chunk_cases(n, seed):
    """Random chunks: Lq queries at offset q_offset into Lk keys (causal: the
    chunk ends at or before the last key; non-causal: any Lk)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, _, n_q, n_kv, d, causal = _draw(rng)
        Lk = int(rng.choice([1, 63, 300, 1000, 2048, 5000]))
        Lq = int(rng.integers(1, Lk + 1)) if causal else int(rng.choice([1, 17, 200, 1000]))
        q_off = int(rng.integers(0, Lk - Lq + 1)) if causal else 0
        if B * n_q * Lq * Lk > 3e9:
            continue
        out.append((B, Lq, Lk, q_off, n_q, n_kv, d, causal))
    return out


CHUNK_CASES = _chunk_cases(12, seed=9300)


@pytest.mark.parametrize("B,Lq,Lk,q_off,n_q,n_kv,d,causal", CHUNK_CASES)
def test_random_chunk(B, Lq, Lk, q_off, n_q, n_kv, d, causal):
    import torch
    from causal_gqa_prefill_amd import attn_prefill_chunk_into
    scale = float(np.float32(1.0 / np.sqrt(d)))
    seed = 9400 + B + Lq * 3 + Lk + q_off + n_q + d
    label = f"random chunk B={B} Lq={Lq} Lk={Lk} q_off={q_off} n_q={n_q} n_kv={n_kv} d={d} causal={causal}"
    say(f"case {label}")
    qb, kb, vb = inputs.make_chunk_qkv(B, Lq, Lk, n_q, n_kv, d, seed)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out = torch.empty_like(q).fill_(float("nan"))
    lse = torch.empty((B, n_q, Lq), dtype=torch.float32, device=q.device).fill_(float("nan"))
    attn_prefill_chunk_into(q, k, v, out, lse, q_off, scale=scale, causal=causal)
    torch.cuda.synchronize()
    o = from_dev_bf16(out).reshape(-1, d)
    l = lse.cpu().numpy().astype(np.float64).reshape(-1)
    rng = np.random.default_rng(seed + 1)
    blocks = np.arange(0, B * n_q * Lq, 32, dtype=np.int64)
    span = np.minimum(32, B * n_q * Lq - blocks)
    rows = blocks + (rng.random(blocks.size) * span).astype(np.int64)
    ref_o, ref_l, _ = oracle.attention_rows_chunk(qb, kb, vb, scale, causal, q_offset=q_off,
                                                  rows=rows)
    compare(label, o[rows], l[rows], ref_o, ref_l)


# ---------------------------------------------------------------------------
# FP8 (e4m3, d_h = 128) and the backward pass on random shapes, each checked
# element by element against the oracle within the rounding bounds of
# tests/bounds.py (the helpers of test_gpu_fp8.py and test_gpu_bwd.py)
# ---------------------------------------------------------------------------
def _fp8_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, _, n_q, n_kv, _, causal = _draw(rng)
        Lk = int(rng.choice([1, 65, 300, 1000, 2048]))
        Lq = int(rng.integers(1, Lk + 1)) if causal else int(rng.choice([1, 31, 200]))
        q_off = int(rng.integers(0, Lk - Lq + 1)) if causal else 0
        if B * n_q * Lq * Lk > 1.5e8:
            continue
        out.append((B, Lq, Lk, q_off, n_q, n_kv, causal))
    return out


FP8_CASES = _fp8_cases(10, seed=9500)


@pytest.mark.parametrize("B,Lq,Lk,q_off,n_q,n_kv,causal", FP8_CASES)
def test_random_fp8(B, Lq, Lk, q_off, n_q, n_kv, causal):
    from test_gpu_fp8 import _run_fp8, compare_fp8, fp8_reference
    d = 128
    label = f"random fp8 B={B} Lq={Lq} Lk={Lk} q_off={q_off} n_q={n_q} n_kv={n_kv} causal={causal}"
    say(f"case {label}")
    scale = float(np.float32(d ** -0.5))
    q8, k8, v8, dq, dk, dv = inputs.make_fp8_qkv(B, Lq, Lk, n_q, n_kv, d,
                                                 seed=9600 + B + Lq + 3 * Lk + q_off)
    o, l = _run_fp8(q8, k8, v8, dq, dk, dv, scale, causal, q_off)
    ref_o, ref_l, bound = fp8_reference(q8, k8, v8, scale, dq, dk, dv, causal, q_off)
    compare_fp8(label, o.reshape(-1, d), l.reshape(-1), ref_o, ref_l, bound)


def _bwd_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        B, L, n_q, n_kv, d, causal = _draw(rng)
        if B * n_q * L * L > 4e7 or L > 2048:
            continue
        out.append((B, L, n_q, n_kv, d, causal))
    return out


BWD_CASES = _bwd_cases(8, seed=9700)


@pytest.mark.parametrize("B,L,n_q,n_kv,d,causal", BWD_CASES)
def test_random_backward(B, L, n_q, n_kv, d, causal):
    from test_gpu_bwd import _run_case
    _run_case(B, L, n_q, n_kv, d, causal, seed=9800 + B + L + n_q + d,
              label=f"random bwd B={B} L={L} n_q={n_q} n_kv={n_kv} d={d} causal={causal}")
