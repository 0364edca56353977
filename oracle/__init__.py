"""fp64 CPU oracle for causal GQA prefill attention -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
imports, links or calls it, and it imports nothing from the product package.

The arithmetic lives in attn_oracle.c (plain definition: materialise the score
row, mask, subtract the max, exponentiate, normalise, multiply by V, emit the
natural-log LSE).  This module only loads that library (building it with gcc
on first use if it is missing) and marshals numpy arrays.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

OK, BAD_ARG, NO_MEMORY = 0, 1, 2


def load_library(path):
    """Load an oracle shared library and declare its C signatures."""
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    lib.oracle_attn_rows.restype = ctypes.c_int
    lib.oracle_attn_rows.argtypes = [
        u16p, u16p, u16p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_float, ctypes.c_int,
        ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
        ctypes.POINTER(ctypes.c_uint64), ctypes.c_int,
    ]
    lib.oracle_attn_rows_chunk.restype = ctypes.c_int
    lib.oracle_attn_rows_chunk.argtypes = [
        u16p, u16p, u16p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
        ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
        ctypes.POINTER(ctypes.c_uint64), ctypes.c_int,
    ]
    u8p = ctypes.POINTER(ctypes.c_uint8)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.oracle_attn_rows_chunk_fp8.restype = ctypes.c_int
    lib.oracle_attn_rows_chunk_fp8.argtypes = [
        u8p, u8p, u8p,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
        ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_int,
        ctypes.POINTER(ctypes.c_int64), ctypes.c_int64,
        dp, dp, ctypes.POINTER(ctypes.c_uint64), ctypes.c_int,
    ]
    lib.oracle_e4m3_table.restype = None
    lib.oracle_e4m3_table.argtypes = [dp]
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_attn_bwd_rowstats.restype = ctypes.c_int
    lib.oracle_attn_bwd_rowstats.argtypes = [
        u16p, u16p, u16p, u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_int, i64p, ctypes.c_int64,
        dp, dp, dp, ctypes.c_int]
    lib.oracle_attn_bwd_dq.restype = ctypes.c_int
    lib.oracle_attn_bwd_dq.argtypes = [
        u16p, u16p, u16p, u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_int, dp, dp, i64p,
        ctypes.c_int64, dp, ctypes.c_int]
    lib.oracle_attn_bwd_dkdv.restype = ctypes.c_int
    lib.oracle_attn_bwd_dkdv.argtypes = [
        u16p, u16p, u16p, u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
        ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_int, dp, dp, i64p,
        ctypes.c_int64, dp, dp, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_version.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = load_library(_build.LIB)
    return _lib


def max_threads() -> int:
    """OpenMP threads the oracle uses by default."""
    return int(_load().oracle_max_threads())


def _bits(a, shape, name):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError(f"{name}: expected bf16 bit patterns as uint16, got {a.dtype}")
    if a.shape != shape:
        raise ValueError(f"{name}: expected shape {shape}, got {a.shape}")
    return a


def attention_rows(q, k, v, scale, causal=True, rows=None, threads=0, lib=None):
    """Oracle attention for selected query rows.

    q: uint16 [B, n_q, L, d_h] bf16 bits; k, v: uint16 [B, n_kv, L, d_h].
    scale: the fp32 scale applied to Q K^T (passed as float32).
    rows: None for every row, else flat row ids (b * n_q + h) * L + i.
    lib: a library from load_library() (default: the built oracle).
    Returns (out [n_rows, d_h] float64, lse [n_rows] float64, flops int).
    """
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, heads, L, d_h]")
    B, n_q, L, d_h = q.shape
    n_kv = k.shape[1]
    q = _bits(q, (B, n_q, L, d_h), "q")
    k = _bits(k, (B, n_kv, L, d_h), "k")
    v = _bits(v, (B, n_kv, L, d_h), "v")
    if rows is None:
        n_rows = B * n_q * L
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = int(rows.size)
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out = np.empty((n_rows, d_h), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    flops = ctypes.c_uint64(0)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = (lib or _load()).oracle_attn_rows(
        q.ctypes.data_as(u16p), k.ctypes.data_as(u16p), v.ctypes.data_as(u16p),
        B, L, n_q, n_kv, d_h, float(np.float32(scale)), int(causal),
        rows_p, n_rows, out.ctypes.data_as(dp), lse.ctypes.data_as(dp),
        ctypes.byref(flops), int(threads))
    if rc != OK:
        raise ValueError(f"oracle_attn_rows failed with code {rc}")
    return out, lse, int(flops.value)


def attention_rows_chunk(q, k, v, scale, causal=True, q_offset=0, rows=None, threads=0,
                         lib=None):
    """Oracle attention of a chunk: Lq queries, query row i at key position
    q_offset + i, against Lk keys ("flops / prefill-attention", section
    "Workarounds", chunked prefill).

    q: uint16 [B, n_q, Lq, d_h]; k, v: uint16 [B, n_kv, Lk, d_h] (bf16 bits).
    causal: key j visible to row i iff j <= q_offset + i (needs
    q_offset + Lq <= Lk); otherwise all Lk keys.
    rows: None for every row, else flat row ids (b * n_q + h) * Lq + i.
    Returns (out [n_rows, d_h] float64, lse [n_rows] float64, flops int).
    """
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, heads, L, d_h]")
    B, n_q, Lq, d_h = q.shape
    n_kv, Lk = k.shape[1], k.shape[2]
    q = _bits(q, (B, n_q, Lq, d_h), "q")
    k = _bits(k, (B, n_kv, Lk, d_h), "k")
    v = _bits(v, (B, n_kv, Lk, d_h), "v")
    if rows is None:
        n_rows = B * n_q * Lq
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = int(rows.size)
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out = np.empty((n_rows, d_h), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    flops = ctypes.c_uint64(0)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = (lib or _load()).oracle_attn_rows_chunk(
        q.ctypes.data_as(u16p), k.ctypes.data_as(u16p), v.ctypes.data_as(u16p),
        B, Lq, Lk, int(q_offset), n_q, n_kv, d_h, float(np.float32(scale)), int(causal),
        rows_p, n_rows, out.ctypes.data_as(dp), lse.ctypes.data_as(dp),
        ctypes.byref(flops), int(threads))
    if rc != OK:
        raise ValueError(f"oracle_attn_rows_chunk failed with code {rc}")
    return out, lse, int(flops.value)


def merge_partials(o_a, lse_a, o_b, lse_b):
    """Merge of two partial attention results over disjoint key sets, in
    float64 ("Long-Context Attention Explained", section "Online softmax":
    two running maxima and sums combine by rescaling to the larger max).

    o_a, o_b: [rows, d_h] partial outputs (each a softmax-weighted average
    over its own keys); lse_a, lse_b: [rows] their natural-log LSEs, -inf
    for a side with no visible key.  Returns (out [rows, d_h], lse [rows]):
    out = (w_a o_a + w_b o_b) / (w_a + w_b), lse = m + ln(w_a + w_b), with
    m = max(lse_a, lse_b) and w_x = exp(lse_x - m); a side of weight 0 adds
    nothing whatever its o holds (a side with no key may be left unwritten);
    a row with both sides -inf gives out 0 and lse -inf.
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    m = np.maximum(lse_a, lse_b)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    w_a = np.where(np.isneginf(lse_a), 0.0, np.exp(lse_a - m_safe))
    w_b = np.where(np.isneginf(lse_b), 0.0, np.exp(lse_b - m_safe))
    total = w_a + w_b
    safe_total = np.where(both_empty, 1.0, total)
    # a side of weight 0 contributes nothing, whatever its output holds
    part_a = np.where(w_a[:, None] > 0, w_a[:, None] * o_a, 0.0)
    part_b = np.where(w_b[:, None] > 0, w_b[:, None] * o_b, 0.0)
    out = (part_a + part_b) / safe_total[:, None]
    lse = np.where(both_empty, -np.inf, m_safe + np.log(safe_total))
    return out, lse


def e4m3_table(lib=None):
    """The oracle's decoded value of every OCP e4m3 code (float64 [256])."""
    out = np.empty(256, dtype=np.float64)
    (lib or _load()).oracle_e4m3_table(out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)))
    return out


def attention_rows_chunk_fp8(q, k, v, scale, descale_q, descale_k, descale_v, causal=True,
                             q_offset=0, rows=None, threads=0, lib=None):
    """Oracle attention of a chunk with OCP e4m3 inputs ("flops /
    prefill-attention", section "Workarounds", FP8 attention): codes decoded
    exactly, times their fp32 descale factors, then the plain fp64 attention.

    q: uint8 [B, n_q, Lq, d_h]; k, v: uint8 [B, n_kv, Lk, d_h] (e4m3 codes).
    Returns (out [n_rows, d_h], lse [n_rows], flops).
    """
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q, k, v must be 4-D [B, heads, L, d_h]")
    B, n_q, Lq, d_h = q.shape
    n_kv, Lk = k.shape[1], k.shape[2]
    for name, a, shape in (("q", q, (B, n_q, Lq, d_h)), ("k", k, (B, n_kv, Lk, d_h)),
                           ("v", v, (B, n_kv, Lk, d_h))):
        if a.dtype != np.uint8 or a.shape != shape:
            raise ValueError(f"{name} must be uint8 e4m3 codes of shape {shape}")
    q, k, v = (np.ascontiguousarray(a) for a in (q, k, v))
    if rows is None:
        n_rows = B * n_q * Lq
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n_rows = int(rows.size)
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out = np.empty((n_rows, d_h), dtype=np.float64)
    lse = np.empty((n_rows,), dtype=np.float64)
    flops = ctypes.c_uint64(0)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    dp = ctypes.POINTER(ctypes.c_double)
    rc = (lib or _load()).oracle_attn_rows_chunk_fp8(
        q.ctypes.data_as(u8p), k.ctypes.data_as(u8p), v.ctypes.data_as(u8p),
        B, Lq, Lk, int(q_offset), n_q, n_kv, d_h, float(np.float32(scale)),
        float(np.float32(descale_q)), float(np.float32(descale_k)),
        float(np.float32(descale_v)), int(causal), rows_p, n_rows,
        out.ctypes.data_as(dp), lse.ctypes.data_as(dp), ctypes.byref(flops), int(threads))
    if rc != OK:
        raise ValueError(f"oracle_attn_rows_chunk_fp8 failed with code {rc}")
    return out, lse, int(flops.value)


# ---------------------------------------------------------------------------
# backward pass ("Long-Context Attention Explained", section "What
# FlashAttention does not change": gradients recomputed from the saved row
# statistics); whole sequences, bf16 inputs as uint16 bits
# ---------------------------------------------------------------------------
def _bwd_shapes(q, k, v, dout):
    if q.ndim != 4 or k.ndim != 4:
        raise ValueError("q, k, v, dout must be 4-D [B, heads, L, d_h]")
    B, n_q, L, d = q.shape
    n_kv = k.shape[1]
    q = _bits(q, (B, n_q, L, d), "q")
    k = _bits(k, (B, n_kv, L, d), "k")
    v = _bits(v, (B, n_kv, L, d), "v")
    dout = _bits(dout, (B, n_q, L, d), "dout")
    if n_q % n_kv:
        raise ValueError("n_q must be a multiple of n_kv")
    return q, k, v, dout, B, n_q, n_kv, L, d


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def attention_bwd_rowstats(q, k, v, dout, scale, causal=True, rows=None, threads=0, lib=None):
    """Row statistics of the backward pass for flat query rows
    (b * n_q + h) * L + i (None: every row): (out [n, d_h], lse [n],
    delta [n]) with out the exact attention output and delta = dO . out,
    fp64."""
    q, k, v, dout, B, n_q, n_kv, L, d = _bwd_shapes(q, k, v, dout)
    if rows is None:
        n = B * n_q * L
        rows_p = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = int(rows.size)
        rows_p = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    out = np.empty((n, d))
    lse = np.empty(n)
    delta = np.empty(n)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    rc = (lib or _load()).oracle_attn_bwd_rowstats(
        q.ctypes.data_as(u16p), k.ctypes.data_as(u16p), v.ctypes.data_as(u16p),
        dout.ctypes.data_as(u16p), B, L, n_q, n_kv, d, float(np.float32(scale)), int(causal),
        rows_p, n, _ptr(out), _ptr(lse), _ptr(delta), int(threads))
    if rc != OK:
        raise ValueError(f"oracle_attn_bwd_rowstats failed with code {rc}")
    return out, lse, delta


def attention_bwd_dq(q, k, v, dout, scale, causal, lse, delta, rows, threads=0, lib=None):
    """dQ [len(rows), d_h] for flat query rows (b * n_q + h) * L + i; lse and
    delta indexed by flat row (only the requested rows are read)."""
    q, k, v, dout, B, n_q, n_kv, L, d = _bwd_shapes(q, k, v, dout)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    delta = np.ascontiguousarray(delta, dtype=np.float64)
    if lse.size != B * n_q * L or delta.size != B * n_q * L:
        raise ValueError("lse and delta must hold one entry per query row")
    out = np.empty((rows.size, d))
    u16p = ctypes.POINTER(ctypes.c_uint16)
    rc = (lib or _load()).oracle_attn_bwd_dq(
        q.ctypes.data_as(u16p), k.ctypes.data_as(u16p), v.ctypes.data_as(u16p),
        dout.ctypes.data_as(u16p), B, L, n_q, n_kv, d, float(np.float32(scale)), int(causal),
        _ptr(lse), _ptr(delta), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size,
        _ptr(out), int(threads))
    if rc != OK:
        raise ValueError(f"oracle_attn_bwd_dq failed with code {rc}")
    return out


def attention_bwd_dkdv(q, k, v, dout, scale, causal, lse, delta, rows, threads=0, lib=None):
    """(dK, dV) [len(rows), d_h] for flat key rows (b * n_kv + kvh) * L + j;
    lse and delta indexed by flat query row (the rows that see a requested
    key are read)."""
    q, k, v, dout, B, n_q, n_kv, L, d = _bwd_shapes(q, k, v, dout)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    lse = np.ascontiguousarray(lse, dtype=np.float64)
    delta = np.ascontiguousarray(delta, dtype=np.float64)
    if lse.size != B * n_q * L or delta.size != B * n_q * L:
        raise ValueError("lse and delta must hold one entry per query row")
    dk = np.empty((rows.size, d))
    dv = np.empty((rows.size, d))
    u16p = ctypes.POINTER(ctypes.c_uint16)
    rc = (lib or _load()).oracle_attn_bwd_dkdv(
        q.ctypes.data_as(u16p), k.ctypes.data_as(u16p), v.ctypes.data_as(u16p),
        dout.ctypes.data_as(u16p), B, L, n_q, n_kv, d, float(np.float32(scale)), int(causal),
        _ptr(lse), _ptr(delta), rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), rows.size,
        _ptr(dk), _ptr(dv), int(threads))
    if rc != OK:
        raise ValueError(f"oracle_attn_bwd_dkdv failed with code {rc}")
    return dk, dv


def attention_bwd(q, k, v, dout, scale, causal=True, threads=0, lib=None):
    """Every row of dQ [B, n_q, L, d_h], dK and dV [B, n_kv, L, d_h] (fp64),
    plus the row statistics (lse, delta)."""
    B, n_q, L, d = q.shape
    n_kv = k.shape[1]
    _, lse, delta = attention_bwd_rowstats(q, k, v, dout, scale, causal, threads=threads,
                                           lib=lib)
    dq = attention_bwd_dq(q, k, v, dout, scale, causal, lse, delta,
                          np.arange(B * n_q * L), threads=threads, lib=lib)
    dk, dv = attention_bwd_dkdv(q, k, v, dout, scale, causal, lse, delta,
                                np.arange(B * n_kv * L), threads=threads, lib=lib)
    return (dq.reshape(B, n_q, L, d), dk.reshape(B, n_kv, L, d), dv.reshape(B, n_kv, L, d),
            lse, delta)
