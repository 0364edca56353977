"""Work and traffic model for causal GQA prefill attention (host arithmetic).

"flops / prefill-attention", section "Arithmetic intensity": causal prefill
attention does 2 * n_q * d_h * L^2 flops per sequence (Q K^T and P V, each
halved by the mask) and must read K and V once, 4 * L * d_h * n_kv bytes in
bf16, so its arithmetic intensity is g * L / 2 flop per byte.  The ridge of an
accelerator is peak flop/s over peak byte/s, 1000 * TFLOP/s / (GB/s) in
flop/B, and L_ridge = 2 * ridge / g.
"Memory-bound vs compute-bound", researcher section: attainable throughput is
min(P_max, beta * I), ridge I* = P_max / beta.
"Long-Context Attention Explained", quadratic-cost section: without the causal
mask the count is 4 * L^2 * d_h * n_q (the FlashAttention-2 convention).
"""

# MI355X published peaks (AMD datasheet figures, dense, no sparsity)
MI355X_BF16_DENSE_TFLOPS = 2516.6   # 256 CU * 4096 flop/clk * 2.4 GHz
MI355X_HBM_GBPS = 8000.0
MI355X_FP8_DENSE_TFLOPS = 5000.0     # dense fp8 matrix-core peak (datasheet)


def attn_flops(B, L, n_q, d_h, causal=True):
    """Useful flops: 2*B*n_q*d_h*L^2 causal, 4*B*n_q*d_h*L^2 otherwise."""
    f = 2 * B * n_q * d_h * L * L
    return f if causal else 2 * f


def counted_pair_flops(B, L, n_q, d_h, causal=True):
    """Flops counted per visible (query, key) pair, 4*d_h each:
    causal pairs number L(L+1)/2 per head."""
    pairs = L * (L + 1) // 2 if causal else L * L
    return 4 * d_h * pairs * B * n_q


def kv_bytes(B, L, n_kv, d_h, elem=2):
    """Compulsory K and V bytes: 2 tensors * L * d_h * n_kv elements."""
    return 2 * B * L * d_h * n_kv * elem


def all_bytes(B, L, n_q, n_kv, d_h, elem=2):
    """Compulsory HBM bytes of one call: read Q, K, V, write O and fp32 LSE."""
    qo = 2 * B * n_q * L * d_h * elem
    return qo + kv_bytes(B, L, n_kv, d_h, elem) + 4 * B * n_q * L


def intensity_kv(L, g):
    """g * L / 2 flop per K/V byte."""
    return g * L / 2


def ridge(tflops, gbps):
    """flop per byte at which a roofline turns: 1000 * TFLOP/s / (GB/s)."""
    return 1000.0 * tflops / gbps


def l_ridge(ridge_flop_per_byte, g):
    """Sequence length at which g * L / 2 reaches the ridge."""
    return 2.0 * ridge_flop_per_byte / g


def attainable(intensity, p_max, beta):
    """Roofline: min(P_max, beta * I)."""
    return min(p_max, beta * intensity)


def chunk_flops(B, Lq, Lk, q_offset, n_q, d_h, causal=True):
    """Flops of a chunk ("flops / prefill-attention", section "Workarounds"):
    4 * d_h per (query, key) pair formed; causally query i of the chunk sees
    q_offset + i + 1 keys, otherwise all Lk."""
    if causal:
        pairs = (2 * q_offset + Lq + 1) * Lq // 2
    else:
        pairs = Lq * Lk
    return 4 * d_h * pairs * B * n_q


def chunk_bytes(B, Lq, Lk, n_q, n_kv, d_h, elem=2):
    """Compulsory HBM bytes of a chunk: read Q and the K, V rows, write O and
    the fp32 LSE (a causal chunk at q_offset reads only q_offset + Lq rows
    of K and V; this counts all Lk, the non-causal case)."""
    return 2 * B * n_q * Lq * d_h * elem + kv_bytes(B, Lk, n_kv, d_h, elem) + 4 * B * n_q * Lq


def merge_bytes(rows, d_h, elem=2):
    """Bytes of one merge: read two [rows, d_h] partials and two fp32 LSE
    rows, write one of each."""
    return 3 * rows * d_h * elem + 3 * rows * 4


def decode_bytes(B, Lk, n_q, n_kv, d_h, elem=2):
    """Compulsory HBM bytes of one decode step: the whole K/V cache of Lk
    rows, the query, the output and the fp32 LSE ("Memory-bound vs
    compute-bound", section "Arithmetic intensity of a decoder step": the
    K/V cache term)."""
    return kv_bytes(B, Lk, n_kv, d_h, elem) + 2 * B * n_q * d_h * elem + 4 * B * n_q
