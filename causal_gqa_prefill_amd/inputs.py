"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention arithmetic: it draws normal samples, encodes
them as bf16 bit patterns (round to nearest even), and picks query rows to
sample.  Both the HIP path and the CPU oracle receive exactly these bits.

Recipe: numpy default_rng(seed) (PCG64) standard_normal in float32, drawn in
the order Q, K, V from one stream, each element rounded to bf16 with
round-to-nearest-even.
"""
import numpy as np


def bf16_bits(x) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), round to nearest even.

    Finite inputs only (the generators never produce NaN or Inf)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    t = np.right_shift(u, np.uint32(16))      # one temporary, updated in place
    np.bitwise_and(t, np.uint32(1), out=t)
    np.add(t, np.uint32(0x7FFF), out=t)
    np.add(t, u, out=t)
    np.right_shift(t, np.uint32(16), out=t)
    return t.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def make_qkv(B, L, n_q, n_kv, d_h, seed):
    """Q [B,n_q,L,d_h], K and V [B,n_kv,L,d_h] as bf16 bits from N(0, 1)."""
    rng = np.random.default_rng(seed)
    out = []
    for heads in (n_q, n_kv, n_kv):
        x = rng.standard_normal((B, heads, L, d_h), dtype=np.float32)
        out.append(bf16_bits(x))
        del x
    return tuple(out)


def _e4m3_positive_values():
    """Values of the OCP e4m3 codes 0x00 .. 0x7E (increasing): exponent bits
    6..3 with bias 7, mantissa bits 2..0, subnormals m * 2^-9."""
    codes = np.arange(127)
    e = codes >> 3
    m = codes & 7
    return np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))


def e4m3_bits(x) -> np.ndarray:
    """float32 array -> OCP e4m3 codes (uint8), round to nearest, ties to the
    even code.  |x| must not exceed 464 (the largest finite code's range).

    Normal range (|x| >= 2^-6): the float32 significand is rounded to 3 bits
    (nearest even) by integer arithmetic on the bit pattern, and the exponent
    re-biased from 127 to 7.  Below 2^-6 the codes are the subnormals
    m * 2^-9, m = |x| * 512 rounded to nearest even (m = 8 is the smallest
    normal, whose code is 8 as well).  Values in [448, 464] map to 448."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 22   # bounded temporaries for tensors of hundreds of millions of values
    for i0 in range(0, flat.size, step):
        xs = flat[i0:i0 + step]
        a = np.abs(xs)
        if np.any(a > 464.0) or not np.all(np.isfinite(a)):
            raise ValueError("values outside the e4m3 range")
        u = a.view(np.uint32)
        # nearest-even rounding of the significand to 3 bits (carry may bump the exponent)
        r = u + np.uint32(0x7FFFF) + ((u >> np.uint32(20)) & np.uint32(1))
        exp = (r >> np.uint32(23)).astype(np.int32) - 127 + 7
        normal = ((exp << 3) | ((r >> np.uint32(20)) & np.uint32(7)).astype(np.int32))
        sub = np.rint(a * np.float32(512.0)).astype(np.int32)   # exact scaling, then RNE
        code = np.where(a >= np.float32(2.0 ** -6), normal, sub)
        code = np.minimum(code, 126)
        code = code.astype(np.uint8)
        code[np.signbit(xs)] |= np.uint8(0x80)
        out[i0:i0 + step] = code
    return out.reshape(x.shape)


def make_fp8_qkv(B, Lq, Lk, n_q, n_kv, d_h, seed):
    """Q [B,n_q,Lq,d_h], K, V [B,n_kv,Lk,d_h] as OCP e4m3 codes with one fp32
    descale factor each: the same N(0, 1) float32 draws as make_chunk_qkv
    (order Q, K, V from one stream), each tensor divided by
    descale = max|x| / 448 and rounded to e4m3 (nearest even).  Returns
    (q, k, v, descale_q, descale_k, descale_v)."""
    rng = np.random.default_rng(seed)
    codes, scales = [], []
    for heads, length in ((n_q, Lq), (n_kv, Lk), (n_kv, Lk)):
        x = rng.standard_normal((B, heads, length, d_h), dtype=np.float32)
        s = np.float32(np.max(np.abs(x)) / np.float32(448.0))
        np.divide(x, s, out=x)
        codes.append(e4m3_bits(x))
        scales.append(float(s))
        del x
    return (*codes, *scales)


def make_config_qkv(cfg):
    return make_qkv(cfg.B, cfg.L, cfg.n_q, cfg.n_kv, cfg.d_h, cfg.seed)


def make_chunk_qkv(B, Lq, Lk, n_q, n_kv, d_h, seed):
    """A chunk's Q [B,n_q,Lq,d_h] and the K, V [B,n_kv,Lk,d_h] it attends to,
    as bf16 bits from N(0, 1), drawn in the order Q, K, V from one stream."""
    rng = np.random.default_rng(seed)
    out = []
    for heads, length in ((n_q, Lq), (n_kv, Lk), (n_kv, Lk)):
        x = rng.standard_normal((B, heads, length, d_h), dtype=np.float32)
        out.append(bf16_bits(x))
        del x
    return tuple(out)


def make_decode_qkv(B, Lk, n_q, n_kv, d_h, seed, capacity=None):
    """One query per sequence, Q [B,n_q,d_h], and its K/V cache
    [B,n_kv,capacity,d_h] (capacity >= Lk; rows past Lk are drawn too, as
    a stale cache would hold data), bf16 bits from N(0, 1), drawn in the
    order Q, K, V from one stream."""
    cap = Lk if capacity is None else capacity
    rng = np.random.default_rng(seed)
    out = [bf16_bits(rng.standard_normal((B, n_q, d_h), dtype=np.float32))]
    for _ in range(2):
        x = rng.standard_normal((B, n_kv, cap, d_h), dtype=np.float32)
        out.append(bf16_bits(x))
        del x
    return tuple(out)


def make_partials(rows, d_h, seed, empty_every=0):
    """Two partial results to merge: o_a, o_b bf16 bits [rows, d_h] from
    N(0, 1) and lse_a, lse_b float32 [rows] from 8 * N(0, 1) (so the two
    weights range from equal to many orders apart).  With empty_every = n > 0,
    every n-th row has lse_a = -inf, every n-th row offset by n // 2 has
    lse_b = -inf, every n-th row offset by n // 3 has both, and an empty side's
    o holds NaN bits (its content must not matter)."""
    rng = np.random.default_rng(seed)
    o_a = bf16_bits(rng.standard_normal((rows, d_h), dtype=np.float32))
    o_b = bf16_bits(rng.standard_normal((rows, d_h), dtype=np.float32))
    lse_a = (8.0 * rng.standard_normal(rows)).astype(np.float32)
    lse_b = (8.0 * rng.standard_normal(rows)).astype(np.float32)
    if empty_every > 0:
        r = np.arange(rows)
        ea = (r % empty_every == 0) | (r % empty_every == empty_every // 3)
        eb = (r % empty_every == empty_every // 2) | (r % empty_every == empty_every // 3)
        lse_a[ea] = -np.inf
        lse_b[eb] = -np.inf
        o_a[ea] = 0x7FC0
        o_b[eb] = 0x7FC0
    return o_a, lse_a, o_b, lse_b


def sample_rows(B, n_q, L, n, seed, block_rows=128):
    """n distinct flat row ids (b * n_q + h) * L + i.

    Four rows are always included: the first and last query of head 0, the
    last query of the last head, and the first row of the second q-block of
    the middle head.  The rest are drawn uniformly without replacement from the
    remaining rows with default_rng(seed + 7).  Returned sorted."""
    total = B * n_q * L
    if n >= total:
        return np.arange(total, dtype=np.int64)
    forced = [0, L - 1, (n_q - 1) * L + (L - 1),
              (n_q // 2) * L + min(block_rows, L - 1)]
    forced = sorted(set(forced))
    rng = np.random.default_rng(seed + 7)
    picked = set(forced)
    need = n - len(picked)
    while need > 0:
        cand = rng.integers(0, total, size=2 * need + 16, dtype=np.int64)
        for c in cand.tolist():
            if c not in picked:
                picked.add(c)
                need -= 1
                if need == 0:
                    break
    return np.array(sorted(picked), dtype=np.int64)


def row_coords(rows, n_q, L):
    """flat row ids -> (b, h, i) arrays."""
    rows = np.asarray(rows, dtype=np.int64)
    return rows // (n_q * L), (rows // L) % n_q, rows % L
