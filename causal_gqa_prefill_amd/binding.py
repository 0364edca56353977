"""ctypes binding for libattn_prefill.so (argument marshalling only).

Every step of the attention runs in the HIP kernels of the library; this
module checks tensor properties, allocates outputs with torch (the caller owns
them) and passes raw device pointers plus the current HIP stream across the
C ABI declared in include/attn_prefill.h.  There is no CPU fallback: if the
library is missing or fails to load, the first call raises.
"""
import ctypes
import math
import os

from . import _build

ATTN_PREFILL_OK = 0

_lib = None


class AttnPrefillError(RuntimeError):
    """A nonzero status from attn_prefill_fwd (text from attn_prefill_strerror)."""

    def __init__(self, status, text):
        super().__init__(f"attn_prefill_fwd failed ({status}): {text}")
        self.status = status


def library():
    """Load libattn_prefill.so once and declare the exported signatures."""
    global _lib
    if _lib is None:
        path = os.environ.get("ATTN_PREFILL_LIB", _build.LIB)
        if not os.path.exists(path):
            raise ImportError(
                f"{path} is missing: build it first (python -c "
                "'import __graft_entry__ as g; g.build()' or python "
                "causal_gqa_prefill_amd/_build.py); there is no fallback")
        lib = ctypes.CDLL(path)
        vp = ctypes.c_void_p
        ci = ctypes.c_int
        lib.attn_prefill_fwd.restype = ci
        lib.attn_prefill_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci,
                                         ctypes.c_float, ci, vp]
        lib.attn_prefill_fwd_chunk.restype = ci
        lib.attn_prefill_fwd_chunk.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci,
                                               ctypes.c_float, ci, vp]
        lib.attn_merge_partials.restype = ci
        lib.attn_merge_partials.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_longlong, ci, vp]
        lib.attn_prefill_fwd_fp8.restype = ci
        lib.attn_prefill_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci,
                                             ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                             ctypes.c_float, ci, vp]
        lib.attn_prefill_bwd.restype = ci
        lib.attn_prefill_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ci, ci, ci, ci,
                                         ci, ctypes.c_float, ci, vp]
        lib.attn_decode_fwd.restype = ci
        lib.attn_decode_fwd.argtypes = [vp, vp, vp, vp, vp, ci, ci, ctypes.c_longlong, ci, ci, ci,
                                        ctypes.c_float, vp, ctypes.c_size_t, vp]
        lib.attn_decode_workspace_bytes.restype = ctypes.c_size_t
        lib.attn_decode_workspace_bytes.argtypes = [ci, ci, ci, ci, ci]
        lib.attn_decode_fwd_noalloc.restype = ci
        lib.attn_decode_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, ci, ci, ctypes.c_longlong,
                                                ci, ci, ci, ctypes.c_float, vp]
        lib.attn_decode_scratch_bytes.restype = ctypes.c_size_t
        lib.attn_decode_scratch_bytes.argtypes = []
        lib.attn_prefill_schedule.restype = ci
        lib.attn_prefill_schedule.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci, ci, vp, vp, vp]
        lib.attn_prefill_strerror.restype = ctypes.c_char_p
        lib.attn_prefill_strerror.argtypes = [ci]
        lib.attn_prefill_version.restype = ci
        lib.attn_prefill_version.argtypes = []
        _lib = lib
    return _lib


def strerror(status: int) -> str:
    return library().attn_prefill_strerror(int(status)).decode()


def fwd_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, L, n_q, n_kv, d_h,
            scale, causal, stream_ptr):
    """Direct call of attn_prefill_fwd with integer pointers; returns status."""
    return library().attn_prefill_fwd(
        ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
        ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr),
        int(B), int(L), int(n_q), int(n_kv), int(d_h), float(scale), int(causal),
        ctypes.c_void_p(stream_ptr))


def fwd_chunk_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, Lq, Lk, q_offset, n_q, n_kv, d_h,
                  scale, causal, stream_ptr):
    """Direct call of attn_prefill_fwd_chunk with integer pointers; returns status."""
    return library().attn_prefill_fwd_chunk(
        ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
        ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr),
        int(B), int(Lq), int(Lk), int(q_offset), int(n_q), int(n_kv), int(d_h), float(scale),
        int(causal), ctypes.c_void_p(stream_ptr))


SCHEDULE_PLAN_KEYS = ("grid", "n_items", "n_qblk", "items_per_qblk", "sg", "pair_t", "pair_rounds",
                      "r_static")


def schedule(B, Lq, Lk, q_offset, n_q, n_kv, d_h, causal, n_cu):
    """attn_prefill_schedule: the forward launch's work list and static rounds
    on n_cu compute units (host only).  Returns (plan dict, list [n_items, 3]
    of (q-block, head group, stream), rounds [R, grid] of list entries, -1
    past the list)."""
    import numpy as np
    lib = library()
    plan = (ctypes.c_longlong * 8)()
    args = [int(B), int(Lq), int(Lk), int(q_offset), int(n_q), int(n_kv), int(d_h), int(causal),
            int(n_cu)]
    st = lib.attn_prefill_schedule(*args, ctypes.cast(plan, ctypes.c_void_p), None, None)
    if st != ATTN_PREFILL_OK:
        raise AttnPrefillError(st, strerror(st))
    info = dict(zip(SCHEDULE_PLAN_KEYS, (int(x) for x in plan)))
    n_items, grid = info["n_items"], info["grid"]
    n_rounds = -(-n_items // grid)
    lst = np.zeros((n_items, 3), dtype=np.int32)
    rounds = np.zeros((n_rounds, grid), dtype=np.int32)
    st = lib.attn_prefill_schedule(*args, ctypes.cast(plan, ctypes.c_void_p),
                                   lst.ctypes.data_as(ctypes.c_void_p),
                                   rounds.ctypes.data_as(ctypes.c_void_p))
    if st != ATTN_PREFILL_OK:
        raise AttnPrefillError(st, strerror(st))
    return info, lst, rounds


def merge_raw(oa_ptr, la_ptr, ob_ptr, lb_ptr, out_ptr, lo_ptr, rows, d_h, stream_ptr):
    """Direct call of attn_merge_partials with integer pointers; returns status."""
    return library().attn_merge_partials(
        ctypes.c_void_p(oa_ptr), ctypes.c_void_p(la_ptr), ctypes.c_void_p(ob_ptr),
        ctypes.c_void_p(lb_ptr), ctypes.c_void_p(out_ptr), ctypes.c_void_p(lo_ptr),
        int(rows), int(d_h), ctypes.c_void_p(stream_ptr))


def fwd_fp8_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, Lq, Lk, q_offset, n_q, n_kv, d_h,
                scale, descale_q, descale_k, descale_v, causal, stream_ptr):
    """Direct call of attn_prefill_fwd_fp8 with integer pointers; returns status."""
    return library().attn_prefill_fwd_fp8(
        ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
        ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr), int(B), int(Lq), int(Lk),
        int(q_offset), int(n_q), int(n_kv), int(d_h), float(scale), float(descale_q),
        float(descale_k), float(descale_v), int(causal), ctypes.c_void_p(stream_ptr))


def bwd_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, dout_ptr, dq_ptr, dk_ptr, dv_ptr, delta_ptr,
            B, L, n_q, n_kv, d_h, scale, causal, stream_ptr):
    """Direct call of attn_prefill_bwd with integer pointers; returns status."""
    vp = ctypes.c_void_p
    return library().attn_prefill_bwd(
        vp(q_ptr), vp(k_ptr), vp(v_ptr), vp(out_ptr), vp(lse_ptr), vp(dout_ptr), vp(dq_ptr),
        vp(dk_ptr), vp(dv_ptr), vp(delta_ptr), int(B), int(L), int(n_q), int(n_kv), int(d_h),
        float(scale), int(causal), vp(stream_ptr))


def decode_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, Lk, kv_capacity, n_q, n_kv, d_h, scale,
               ws_ptr, ws_bytes, stream_ptr):
    """Direct call of attn_decode_fwd with integer pointers; returns status."""
    return library().attn_decode_fwd(
        ctypes.c_void_p(q_ptr), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
        ctypes.c_void_p(out_ptr), ctypes.c_void_p(lse_ptr), int(B), int(Lk), int(kv_capacity),
        int(n_q), int(n_kv), int(d_h), float(scale), ctypes.c_void_p(ws_ptr), int(ws_bytes),
        ctypes.c_void_p(stream_ptr))


def decode_noalloc_raw(q_ptr, k_ptr, v_ptr, out_ptr, lse_ptr, B, Lk, kv_capacity, n_q, n_kv,
                       d_h, scale, stream_ptr):
    """Direct call of attn_decode_fwd_noalloc with integer pointers; returns status."""
    vp = ctypes.c_void_p
    return library().attn_decode_fwd_noalloc(
        vp(q_ptr), vp(k_ptr), vp(v_ptr), vp(out_ptr), vp(lse_ptr), int(B), int(Lk),
        int(kv_capacity), int(n_q), int(n_kv), int(d_h), float(scale), vp(stream_ptr))


def decode_scratch_bytes():
    """Bytes of the static scratch attn_decode_fwd_noalloc runs on."""
    return int(library().attn_decode_scratch_bytes())


def decode_workspace_bytes(B, Lk, n_q, n_kv, d_h):
    """Bytes of workspace attn_decode_fwd needs (0 for rejected sizes)."""
    return int(library().attn_decode_workspace_bytes(int(B), int(Lk), int(n_q), int(n_kv),
                                                     int(d_h)))


def _check(q, k, v, same_length=True):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a HIP device, got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, heads, L, d_h]")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    B, n_q, L, d_h = q.shape
    if (k.shape != v.shape or k.shape[0] != B or k.shape[3] != d_h
            or (same_length and k.shape[2] != L)):
        raise ValueError(f"k and v must be [B, n_kv, {'L' if same_length else 'Lk'}, d_h] "
                         f"matching q {tuple(q.shape)}; got k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, n_q, k.shape[1], L, d_h


def attn_prefill_into(q, k, v, out, lse, scale=None, causal=True, stream=None):
    """Run the forward pass into caller-provided out (bf16) and lse (fp32)."""
    import torch
    B, n_q, n_kv, L, d_h = _check(q, k, v)
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, n_q, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, n_q, L]")
    if out.device != q.device or lse.device != q.device:
        raise ValueError("out and lse must be on the inputs' device")
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), B, L, n_q, n_kv, d_h, scale, int(bool(causal)),
                         s.cuda_stream)
    if status != ATTN_PREFILL_OK:
        raise AttnPrefillError(status, strerror(status))
    return out, lse


def attn_prefill(q, k, v, scale=None, causal=True, stream=None):
    """Causal (or full) GQA prefill attention forward.

    q: bf16 [B, n_q, L, d_h]; k, v: bf16 [B, n_kv, L, d_h] (contiguous, HIP
    device).  scale defaults to 1/sqrt(d_h).  Returns (out bf16 like q,
    lse fp32 [B, n_q, L]), enqueued on `stream` (default: current stream).
    """
    import torch
    B, n_q, _, L, _ = _check(q, k, v)
    out = torch.empty_like(q)
    lse = torch.empty((B, n_q, L), dtype=torch.float32, device=q.device)
    return attn_prefill_into(q, k, v, out, lse, scale=scale, causal=causal, stream=stream)


def _check_outputs(q, out, lse):
    import torch
    B, n_q, L, _ = q.shape
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, n_q, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, n_q, Lq]")
    if out.device != q.device or lse.device != q.device:
        raise ValueError("out and lse must be on the inputs' device")


def attn_prefill_chunk_into(q, k, v, out, lse, q_offset, scale=None, causal=True, stream=None):
    """Chunked prefill into caller-provided out and lse: query row i of q sits at
    key position q_offset + i of k and v (see attn_prefill_fwd_chunk)."""
    import torch
    B, n_q, n_kv, Lq, d_h = _check(q, k, v, same_length=False)
    Lk = k.shape[2]
    _check_outputs(q, out, lse)
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = fwd_chunk_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, Lq, Lk, q_offset, n_q, n_kv, d_h, scale,
                               int(bool(causal)), s.cuda_stream)
    if status != ATTN_PREFILL_OK:
        raise AttnPrefillError(status, strerror(status))
    return out, lse


def attn_prefill_chunk(q, k, v, q_offset, scale=None, causal=True, stream=None):
    """Chunked prefill: q bf16 [B, n_q, Lq, d_h] at key positions q_offset ..
    q_offset + Lq - 1 of k, v bf16 [B, n_kv, Lk, d_h].  Returns (out bf16 like
    q, lse fp32 [B, n_q, Lq])."""
    import torch
    B, n_q, _, Lq, _ = _check(q, k, v, same_length=False)
    out = torch.empty_like(q)
    lse = torch.empty((B, n_q, Lq), dtype=torch.float32, device=q.device)
    return attn_prefill_chunk_into(q, k, v, out, lse, q_offset, scale=scale, causal=causal,
                                   stream=stream)


def merge_partials(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """LSE-weighted merge of two partial results over disjoint key sets (see
    attn_merge_partials).  o_a, o_b: bf16 [..., d_h]; lse_a, lse_b: fp32 with
    o's shape minus the last axis.  Returns (out, lse_out)."""
    import torch
    for name, t in (("o_a", o_a), ("o_b", o_b)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bfloat16 torch.Tensor")
    for name, t in (("lse_a", lse_a), ("lse_b", lse_b)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous float32 torch.Tensor")
    if o_a.shape != o_b.shape or lse_a.shape != lse_b.shape or tuple(lse_a.shape) != tuple(o_a.shape[:-1]):
        raise ValueError("o_a, o_b must match, and lse_a, lse_b must be their shape minus the last axis")
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    d_h = o_a.shape[-1]
    rows = lse_a.numel()
    with torch.cuda.device(o_a.device):
        s = stream if stream is not None else torch.cuda.current_stream(o_a.device)
        status = merge_raw(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(), lse_b.data_ptr(),
                           out.data_ptr(), lse_out.data_ptr(), rows, d_h, s.cuda_stream)
    if status != ATTN_PREFILL_OK:
        raise AttnPrefillError(status, strerror(status))
    return out, lse_out


def attn_decode_into(q, k, v, out, lse, Lk=None, scale=None, workspace=None, stream=None):
    """Decode into caller-provided out (bf16 like q) and lse (fp32 [B, n_q]):
    q bf16 [B, n_q, d_h], one query per sequence at position Lk - 1; k, v
    bf16 [B, n_kv, capacity, d_h], of which the first Lk rows (default: all)
    are read.  workspace: a contiguous device tensor of at least
    decode_workspace_bytes(...) bytes, allocated here when None."""
    import torch
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, n_q, d_h]; k and v [B, n_kv, capacity, d_h], equal shapes")
    B, n_q, d_h = q.shape
    if k.shape[0] != B or k.shape[3] != d_h:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)}")
    if not (q.device == k.device == v.device) or q.device.type != "cuda":
        raise ValueError("q, k and v must be on the same GPU")
    n_kv, cap = k.shape[1], k.shape[2]
    if Lk is None:
        Lk = cap
    if out.dtype != torch.bfloat16 or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, n_q) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, n_q]")
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    need = decode_workspace_bytes(B, Lk, n_q, n_kv, d_h)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous tensor on the inputs' device")
    ws_bytes = workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = decode_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                            lse.data_ptr(), B, Lk, cap, n_q, n_kv, d_h, scale,
                            workspace.data_ptr(), ws_bytes, s.cuda_stream)
    if status != ATTN_PREFILL_OK:
        raise AttnPrefillError(status, strerror(status))
    return out, lse


def attn_decode(q, k, v, Lk=None, scale=None, workspace=None, stream=None):
    """Decode attention: returns (out bf16 [B, n_q, d_h], lse fp32 [B, n_q])."""
    import torch
    out = torch.empty_like(q)
    lse = torch.empty(tuple(q.shape[:2]), dtype=torch.float32, device=q.device)
    return attn_decode_into(q, k, v, out, lse, Lk=Lk, scale=scale, workspace=workspace,
                            stream=stream)


def _check_fp8(q, k, v):
    import torch
    byte_types = (torch.uint8, torch.float8_e4m3fn)
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype not in byte_types:
            raise TypeError(f"{name} must hold e4m3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, heads, L, d_h]")
    if not (q.device == k.device == v.device) or q.device.type != "cuda":
        raise ValueError("q, k and v must be on the same GPU")
    B, n_q, Lq, d_h = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != d_h:
        raise ValueError(f"k and v must be [B, n_kv, Lk, d_h] matching q {tuple(q.shape)}; "
                         f"got k {tuple(k.shape)}, v {tuple(v.shape)}")
    return B, n_q, k.shape[1], Lq, k.shape[2], d_h


def attn_prefill_fp8_into(q, k, v, out, lse, descale_q, descale_k, descale_v, q_offset=0,
                          scale=None, causal=True, stream=None):
    """FP8 prefill (see attn_prefill_fwd_fp8) into caller-provided out (bf16
    [B, n_q, Lq, d_h]) and lse (fp32 [B, n_q, Lq]); q, k, v hold e4m3 codes."""
    import torch
    B, n_q, n_kv, Lq, Lk, d_h = _check_fp8(q, k, v)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != tuple(q.shape) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, n_q, Lq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, n_q, Lq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = fwd_fp8_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             lse.data_ptr(), B, Lq, Lk, q_offset, n_q, n_kv, d_h, scale,
                             descale_q, descale_k, descale_v, int(bool(causal)), s.cuda_stream)
    if status != ATTN_PREFILL_OK:
        raise AttnPrefillError(status, strerror(status))
    return out, lse


def attn_prefill_fp8(q, k, v, descale_q, descale_k, descale_v, q_offset=0, scale=None,
                     causal=True, stream=None):
    """FP8 prefill: returns (out bf16 [B, n_q, Lq, d_h], lse fp32 [B, n_q, Lq])."""
    import torch
    B, n_q, _, Lq, _, d_h = _check_fp8(q, k, v)
    out = torch.empty((B, n_q, Lq, d_h), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, n_q, Lq), dtype=torch.float32, device=q.device)
    return attn_prefill_fp8_into(q, k, v, out, lse, descale_q, descale_k, descale_v,
                                 q_offset=q_offset, scale=scale, causal=causal, stream=stream)


def attn_prefill_backward(q, k, v, out, lse, dout, scale=None, causal=True, stream=None,
                          grads=None):
    """Backward pass (see attn_prefill_bwd): q, out, dout bf16 [B, n_q, L, d_h];
    k, v bf16 [B, n_kv, L, d_h]; lse fp32 [B, n_q, L] from the forward pass.
    Returns (dq, dk, dv, delta); grads = (dq, dk, dv, delta) reuses buffers."""
    import torch
    B, n_q, n_kv, L, d_h = _check(q, k, v)
    for name, t in (("out", out), ("dout", dout)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or \
                tuple(t.shape) != tuple(q.shape) or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor shaped like q")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or \
            tuple(lse.shape) != (B, n_q, L) or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous float32 tensor [B, n_q, L]")
    if grads is None:
        grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
                 torch.empty((B, n_q, L), dtype=torch.float32, device=q.device))
    dq, dk, dv, delta = grads
    if scale is None:
        scale = 1.0 / math.sqrt(d_h)
    with torch.cuda.device(q.device):
        s = stream if stream is not None else torch.cuda.current_stream(q.device)
        status = bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                         lse.data_ptr(), dout.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                         dv.data_ptr(), delta.data_ptr(), B, L, n_q, n_kv, d_h, scale,
                         int(bool(causal)), s.cuda_stream)
    if status != ATTN_PREFILL_OK:
        raise AttnPrefillError(status, strerror(status))
    return dq, dk, dv, delta
