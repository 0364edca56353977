"""The C-ABI library loads without a GPU, exports every symbol its header
declares, and rejects bad arguments on the host before any HIP call."""
import os
import re

import pytest

from causal_gqa_prefill_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_prefill.h")

ALIGNED = 0x100000  # never dereferenced: validation fails first


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_\w+)\s*\(", text)))


def test_library_exports_header_symbols():
    lib = binding.library()
    names = _declared_functions()
    assert names == ["attn_decode_fwd", "attn_decode_fwd_noalloc", "attn_decode_scratch_bytes",
                     "attn_decode_workspace_bytes", "attn_merge_partials",
                     "attn_prefill_bwd", "attn_prefill_fwd", "attn_prefill_fwd_chunk",
                     "attn_prefill_fwd_fp8", "attn_prefill_schedule", "attn_prefill_strerror",
                     "attn_prefill_version"]
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    assert binding.library().attn_prefill_version() >= 400
    for code in range(0, 15):
        assert binding.strerror(code) not in ("", "unknown status")
    assert binding.strerror(99) == "unknown status"


def _call(**kw):
    args = dict(q=ALIGNED, k=ALIGNED + 0x10000000, v=ALIGNED + 0x20000000,
                out=ALIGNED + 0x30000000, lse=ALIGNED + 0x40000000,
                B=1, L=128, n_q=4, n_kv=4, d_h=64, scale=0.125, causal=1, stream=0)
    args.update(kw)
    return binding.fwd_raw(args["q"], args["k"], args["v"], args["out"], args["lse"],
                           args["B"], args["L"], args["n_q"], args["n_kv"], args["d_h"],
                           args["scale"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(out=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(L=0), 2), (dict(n_q=-1), 2), (dict(n_kv=0), 2),
    (dict(n_q=6, n_kv=4), 3),
    (dict(d_h=96), 4), (dict(d_h=256), 4), (dict(d_h=0), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5),
    (dict(causal=2), 6), (dict(causal=-1), 6),
    (dict(q=ALIGNED + 8), 7), (dict(out=ALIGNED + 0x30000002), 7), (dict(lse=ALIGNED + 0x40000002), 7),
    (dict(B=1 << 30, n_q=1 << 30, n_kv=1 << 30, L=1 << 30), 8),
    (dict(out=ALIGNED), 9), (dict(lse=ALIGNED + 0x10000010), 9), (dict(lse=ALIGNED + 0x30000100), 9),
])
def test_bad_arguments_rejected_on_host(kw, code):
    assert _call(**kw) == code


def _call_chunk(**kw):
    args = dict(q=ALIGNED, k=ALIGNED + 0x10000000, v=ALIGNED + 0x20000000,
                out=ALIGNED + 0x30000000, lse=ALIGNED + 0x40000000,
                B=1, Lq=64, Lk=128, q_offset=64, n_q=4, n_kv=4, d_h=64, scale=0.125, causal=1,
                stream=0)
    args.update(kw)
    return binding.fwd_chunk_raw(args["q"], args["k"], args["v"], args["out"], args["lse"],
                                 args["B"], args["Lq"], args["Lk"], args["q_offset"], args["n_q"],
                                 args["n_kv"], args["d_h"], args["scale"], args["causal"],
                                 args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(lse=0), 1),
    (dict(Lq=0), 2), (dict(Lk=0), 2), (dict(B=0), 2),
    (dict(n_q=6, n_kv=4), 3), (dict(d_h=32), 4), (dict(scale=float("-inf")), 5),
    (dict(causal=3), 6),
    (dict(q_offset=-1), 11), (dict(q_offset=65), 11), (dict(Lq=129, q_offset=0), 11),
    (dict(q_offset=-1, causal=0), 11),
    (dict(k=ALIGNED + 0x10000004), 7),
    (dict(out=ALIGNED + 0x10000000 + 4096), 9),
])
def test_chunk_bad_arguments_rejected_on_host(kw, code):
    assert _call_chunk(**kw) == code


def _call_merge(**kw):
    args = dict(oa=ALIGNED, la=ALIGNED + 0x10000000, ob=ALIGNED + 0x20000000,
                lb=ALIGNED + 0x30000000, out=ALIGNED + 0x40000000, lo=ALIGNED + 0x50000000,
                rows=1000, d_h=128, stream=0)
    args.update(kw)
    return binding.merge_raw(args["oa"], args["la"], args["ob"], args["lb"], args["out"],
                             args["lo"], args["rows"], args["d_h"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(oa=0), 1), (dict(lo=0), 1),
    (dict(rows=0), 2), (dict(rows=-5), 2),
    (dict(d_h=96), 4),
    (dict(ob=ALIGNED + 0x20000008), 7), (dict(la=ALIGNED + 0x10000002), 7),
    (dict(rows=1 << 60), 8),
    (dict(out=ALIGNED), 9), (dict(lo=ALIGNED + 0x40000000 + 100), 9),
])
def test_merge_bad_arguments_rejected_on_host(kw, code):
    assert _call_merge(**kw) == code


def test_merge_inputs_may_overlap_each_other():
    # o_a == o_b and lse_a == lse_b is a valid (if pointless) call; it fails only
    # at the launch, which needs a GPU, so check it passes validation by making
    # the aliasing check the last gate: a misaligned out still reports 7 first
    assert _call_merge(ob=ALIGNED, lb=ALIGNED + 0x10000000, out=ALIGNED + 0x40000002) == 7


def _ws_splits(B, Lk, n_q, n_kv, d):
    n = binding.decode_workspace_bytes(B, Lk, n_q, n_kv, d)
    per_split = 4 * (d + 1) * B * n_q
    assert n > 0 and n % per_split == 0
    return n // per_split


@pytest.mark.parametrize("B,Lk,n_q,n_kv,d", [(1, 1, 4, 4, 64), (1, 255, 8, 2, 128),
                                             (1, 257, 8, 2, 128), (1, 32768, 32, 8, 128),
                                             (1, 131072, 36, 6, 128), (32, 8192, 32, 8, 128),
                                             (300, 100, 4, 1, 64), (1, 1 << 28, 8, 1, 128)])
def test_decode_workspace_splits(B, Lk, n_q, n_kv, d):
    # key ranges of 128-key multiples: at least one, every one non-empty, at
    # most 4096 per row
    n = _ws_splits(B, Lk, n_q, n_kv, d)
    assert 1 <= n <= min(4096, (Lk + 127) // 128)
    per = -(-Lk // n)
    per = -(-per // 128) * 128
    assert (n - 1) * per < Lk <= n * per


@pytest.mark.parametrize("args", [(0, 10, 4, 4, 64), (1, 0, 4, 4, 64), (1, 10, 6, 4, 64),
                                  (1, 10, 4, 4, 96), (1, 10, 66, 2, 64), (1, (1 << 31) - 1, 4, 4, 64)])
def test_decode_workspace_rejects(args):
    assert binding.decode_workspace_bytes(*args) == 0


def _call_decode(**kw):
    ws = binding.decode_workspace_bytes(2, 100, 8, 2, 128)
    args = dict(q=ALIGNED, k=ALIGNED + 0x10000000, v=ALIGNED + 0x20000000,
                out=ALIGNED + 0x30000000, lse=ALIGNED + 0x40000000, B=2, Lk=100, cap=128,
                n_q=8, n_kv=2, d_h=128, scale=0.125, ws=ALIGNED + 0x50000000, ws_bytes=ws,
                stream=0)
    args.update(kw)
    return binding.decode_raw(args["q"], args["k"], args["v"], args["out"], args["lse"],
                              args["B"], args["Lk"], args["cap"], args["n_q"], args["n_kv"],
                              args["d_h"], args["scale"], args["ws"], args["ws_bytes"],
                              args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(ws=0), 1),
    (dict(B=0), 2), (dict(Lk=0), 2),
    (dict(n_q=7), 3), (dict(n_q=66), 12), (dict(d_h=80), 4), (dict(scale=float("nan")), 5),
    (dict(cap=99), 11),
    (dict(ws=ALIGNED + 0x50000008), 7), (dict(lse=ALIGNED + 0x40000002), 7),
    (dict(ws_bytes=16), 13),
    (dict(out=ALIGNED + 0x10000000 + 512), 9), (dict(ws=ALIGNED + 0x20000000 + 4096), 9),
    (dict(lse=ALIGNED + 0x50000000 + 64), 9),
])
def test_decode_bad_arguments_rejected_on_host(kw, code):
    assert _call_decode(**kw) == code


def _call_decode_noalloc(**kw):
    args = dict(q=ALIGNED, k=ALIGNED + 0x10000000, v=ALIGNED + 0x20000000,
                out=ALIGNED + 0x30000000, lse=ALIGNED + 0x40000000, B=2, Lk=100, cap=128,
                n_q=8, n_kv=2, d_h=128, scale=0.125, stream=0)
    args.update(kw)
    return binding.decode_noalloc_raw(args["q"], args["k"], args["v"], args["out"], args["lse"],
                                      args["B"], args["Lk"], args["cap"], args["n_q"],
                                      args["n_kv"], args["d_h"], args["scale"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(lse=0), 1),
    (dict(B=0), 2), (dict(Lk=0), 2),
    (dict(n_q=7), 3), (dict(n_q=66), 12), (dict(d_h=80), 4), (dict(scale=float("nan")), 5),
    (dict(cap=99), 11), (dict(lse=ALIGNED + 0x40000002), 7),
    (dict(out=ALIGNED + 0x10000000 + 512), 9),
])
def test_decode_noalloc_bad_arguments_rejected_on_host(kw, code):
    assert _call_decode_noalloc(**kw) == code


def test_decode_noalloc_scratch_limit():
    """Sizes whose workspace exceeds the static scratch are refused before any
    HIP call (the buffers sit far apart so that nothing else fails first)."""
    limit = binding.decode_scratch_bytes()
    assert limit == 16 << 20
    big = (2048, 4096, 64, 8, 128)
    assert binding.decode_workspace_bytes(*big) > limit
    B, Lk, n_q, n_kv, d = big
    far = 1 << 40
    assert _call_decode_noalloc(q=ALIGNED, k=ALIGNED + far, v=ALIGNED + 2 * far,
                                out=ALIGNED + 3 * far, lse=ALIGNED + 4 * far, B=B, Lk=Lk, cap=Lk,
                                n_q=n_q, n_kv=n_kv, d_h=d) == 14
    # the largest decode workloads fit
    for sizes in ((32, 8192, 32, 8, 128), (1, 131072, 36, 6, 128), (8, 32768, 64, 8, 128)):
        assert 0 < binding.decode_workspace_bytes(*sizes) <= limit


def _call_fp8(**kw):
    args = dict(q=ALIGNED, k=ALIGNED + 0x10000000, v=ALIGNED + 0x20000000,
                out=ALIGNED + 0x30000000, lse=ALIGNED + 0x40000000,
                B=1, Lq=64, Lk=128, q_offset=64, n_q=4, n_kv=2, d_h=128, scale=0.088,
                dq=0.01, dk=0.01, dv=0.01, causal=1, stream=0)
    args.update(kw)
    return binding.fwd_fp8_raw(args["q"], args["k"], args["v"], args["out"], args["lse"],
                               args["B"], args["Lq"], args["Lk"], args["q_offset"], args["n_q"],
                               args["n_kv"], args["d_h"], args["scale"], args["dq"], args["dk"],
                               args["dv"], args["causal"], args["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(v=0), 1), (dict(B=0), 2), (dict(Lk=0), 2), (dict(n_q=3), 3),
    (dict(d_h=64), 4), (dict(dq=float("nan")), 5), (dict(dv=float("inf")), 5),
    (dict(scale=1e30, dq=1e30, dk=1e30), 5), (dict(causal=2), 6),
    (dict(q_offset=65), 11), (dict(q_offset=-3, causal=0), 11),
    (dict(k=ALIGNED + 0x10000008), 7),
    (dict(out=ALIGNED + 0x10000000 + 4096), 9), (dict(lse=ALIGNED), 9),
])
def test_fp8_bad_arguments_rejected_on_host(kw, code):
    assert _call_fp8(**kw) == code


def _call_bwd(**kw):
    M = 0x10000000
    args = dict(q=ALIGNED, k=ALIGNED + M, v=ALIGNED + 2 * M, out=ALIGNED + 3 * M,
                lse=ALIGNED + 4 * M, dout=ALIGNED + 5 * M, dq=ALIGNED + 6 * M, dk=ALIGNED + 7 * M,
                dv=ALIGNED + 8 * M, delta=ALIGNED + 9 * M, B=1, L=256, n_q=8, n_kv=2, d_h=128,
                scale=0.088, causal=1, stream=0)
    args.update(kw)
    return binding.bwd_raw(*(args[n] for n in ("q", "k", "v", "out", "lse", "dout", "dq", "dk",
                                               "dv", "delta", "B", "L", "n_q", "n_kv", "d_h",
                                               "scale", "causal", "stream")))


@pytest.mark.parametrize("kw,code", [
    (dict(dout=0), 1), (dict(delta=0), 1), (dict(L=0), 2), (dict(n_q=3), 3), (dict(d_h=96), 4),
    (dict(scale=float("inf")), 5), (dict(causal=-1), 6),
    (dict(dq=ALIGNED + 6 * 0x10000000 + 8), 7), (dict(delta=ALIGNED + 9 * 0x10000000 + 2), 7),
    (dict(dk=ALIGNED + 0x10000000 + 256), 9), (dict(dv=ALIGNED + 7 * 0x10000000 + 4096), 9),
    (dict(delta=ALIGNED + 4 * 0x10000000), 9),
])
def test_bwd_bad_arguments_rejected_on_host(kw, code):
    assert _call_bwd(**kw) == code
