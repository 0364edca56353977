/*
 * attn_prefill.h -- C ABI of the MI355X (gfx950) causal GQA prefill attention
 * forward pass (libattn_prefill.so).
 *
 * The operation.  For every batch b, query head h and query position i:
 *     s_j    = scale * sum_t Q[b,h,i,t] * K[b,kv,j,t]      for visible j
 *     O[b,h,i,:] = sum_j softmax(s)_j * V[b,kv,j,:]
 *     LSE[b,h,i] = ln sum_j exp(s_j)
 * with kv = floor(h / g), g = n_q / n_kv.
 *   - Scaled dot-product attention softmax(Q K^T / sqrt(d)) V: "Why Attention
 *     Scaling Breaks", section "The O(n^2) problem", and "Long-Context
 *     Attention Explained", section on quadratic cost.
 *   - Causal visibility: a token looks only backwards, itself included, so
 *     key j is visible to query i iff j <= i ("Long-Context Attention
 *     Explained", quadratic-cost section).  causal = 0 makes all L keys
 *     visible.
 *   - Grouped-query heads: n_q query heads share n_kv key/value heads ("flops /
 *     prefill-attention", section "Arithmetic intensity"); query head h reads
 *     key/value head floor(h / g), consecutive query heads forming a group.
 *   - The score matrix never reaches memory: tiles of keys are streamed past
 *     each block of queries with an online softmax ("Why Attention Scaling
 *     Breaks", section "Flash Attention: the tiling insight"; "Long-Context
 *     Attention Explained", sections "Tiling" and "Online softmax"); the
 *     result equals the plain definition up to rounding.
 *   - LSE is the per-row statistic a backward pass recomputes from
 *     ("Long-Context Attention Explained", section "What FlashAttention does
 *     not change"): natural log, of the scaled scores, fp32.
 *
 * Layouts (all row-major, contiguous, d_h fastest):
 *   q, out : bf16 [B, n_q,  L, d_h]
 *   k, v   : bf16 [B, n_kv, L, d_h]
 *   lse    : fp32 [B, n_q,  L]
 * bf16 is the 16-bit brain-float format (the upper half of an IEEE fp32).
 *
 * Numerics: Q K^T and P V run as bf16 matrix-core products with fp32
 * accumulation; the softmax runs in fp32; P is rounded to bf16 (nearest even)
 * before P V; O is rounded to bf16 (nearest even) once, after the division by
 * the row sum.
 *
 * Ownership: the caller allocates and frees all five buffers, on the device
 * that is current when the call is made and that `stream` belongs to.  The
 * library allocates nothing, never synchronises, and may be called from
 * several host threads at once.  out and lse must not overlap each other or
 * any input.
 *
 * Launch: the prefill kernels (bf16 and FP8) run a persistent grid of at
 * most one workgroup per CU of the current device (each walks several work
 * items); the result does not depend on the grid size or on which
 * workgroup computes an item.  A schedule of 16 or more rounds of work items
 * hands out the items of its last rounds through a pair of counters that
 * the call takes from a static per-device pool of 65536 pairs (512 KB of
 * device memory held until the process ends): the call's last workgroup
 * sets its pair back to zero, and a pair is handed out again only 65536
 * calls later, so at most 65536 such calls may be in flight on one device
 * at once.  A call made while its stream is being captured into a graph
 * takes no pair (a static schedule, the same result).
 *
 * Errors: every argument is checked on the host before anything is enqueued.
 * A nonzero return means nothing was enqueued, except ATTN_PREFILL_ERR_LAUNCH,
 * which reports the HIP launch error.  Faults inside the kernel surface at the
 * caller's next synchronisation, as for any HIP kernel.
 */
#ifndef ATTN_PREFILL_H
#define ATTN_PREFILL_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_prefill_status {
    ATTN_PREFILL_OK = 0,
    ATTN_PREFILL_ERR_NULL_PTR = 1,      /* a buffer pointer is NULL            */
    ATTN_PREFILL_ERR_BAD_SHAPE = 2,     /* B, L, n_q or n_kv < 1               */
    ATTN_PREFILL_ERR_BAD_GQA = 3,       /* n_q is not a multiple of n_kv       */
    ATTN_PREFILL_ERR_BAD_HEADDIM = 4,   /* d_h is not 64 or 128                */
    ATTN_PREFILL_ERR_BAD_SCALE = 5,     /* scale is NaN or infinite            */
    ATTN_PREFILL_ERR_BAD_CAUSAL = 6,    /* causal is not 0 or 1                */
    ATTN_PREFILL_ERR_MISALIGNED = 7,    /* q/k/v/out not 16-byte aligned, or
                                           lse not 4-byte aligned              */
    ATTN_PREFILL_ERR_SIZE_OVERFLOW = 8, /* a size or the grid overflows        */
    ATTN_PREFILL_ERR_ALIASING = 9,      /* out or lse overlaps another buffer  */
    ATTN_PREFILL_ERR_LAUNCH = 10,       /* the HIP launch failed, or the query
                                           of the current device's CU count
                                           that sizes the grid                 */
    ATTN_PREFILL_ERR_BAD_OFFSET = 11,   /* q_offset < 0, or (causal)
                                           q_offset + Lq > Lk, or (decode)
                                           kv_capacity < Lk                    */
    ATTN_PREFILL_ERR_UNSUPPORTED = 12,  /* (decode) more than 32 query heads
                                           per key/value head                  */
    ATTN_PREFILL_ERR_WORKSPACE = 13,    /* (decode) workspace_bytes too small  */
    ATTN_PREFILL_ERR_SCRATCH = 14       /* (decode, no allocation) the sizes
                                           need more than the static scratch */
};

/*
 * Causal (or full) GQA prefill attention forward pass.
 *   q, k, v : device pointers to the bf16 inputs (layouts above)
 *   out     : device pointer, bf16 [B, n_q, L, d_h], written entirely
 *   lse     : device pointer, fp32 [B, n_q, L], written entirely
 *   B, L, n_q, n_kv, d_h : sizes; n_q % n_kv == 0; d_h in {64, 128}
 *   scale   : multiplies Q K^T (1/sqrt(d_h) for standard attention); any
 *             finite value
 *   causal  : 1 = key j visible to query i iff j <= i; 0 = all keys visible
 *   stream  : HIP stream the work is enqueued on (0 = the null stream)
 * Returns ATTN_PREFILL_OK once the work is enqueued, else an error code.
 */
int attn_prefill_fwd(const void *q, const void *k, const void *v, void *out,
                     float *lse, int B, int L, int n_q, int n_kv, int d_h,
                     float scale, int causal, hipStream_t stream);

/*
 * Chunked prefill: a chunk of Lq queries against Lk keys, query row i sitting
 * at key position q_offset + i.  This is how a long prompt is prefilled in
 * pieces against the keys and values already computed for the earlier pieces
 * ("flops / prefill-attention", section "Workarounds", chunked prefill), and
 * with Lq = Lk, q_offset = 0 it is attn_prefill_fwd.
 *   q, out : bf16 [B, n_q, Lq, d_h];  k, v : bf16 [B, n_kv, Lk, d_h];
 *   lse    : fp32 [B, n_q, Lq]
 *   causal : 1 = key j visible to query row i iff j <= q_offset + i
 *            (requires q_offset + Lq <= Lk, so every query sees its own
 *            position); 0 = all Lk keys visible (q_offset is then unused)
 *   q_offset >= 0; other arguments, numerics, ownership and errors as for
 *   attn_prefill_fwd, ATTN_PREFILL_ERR_BAD_OFFSET for a bad q_offset.
 */
int attn_prefill_fwd_chunk(const void *q, const void *k, const void *v, void *out,
                           float *lse, int B, int Lq, int Lk, int q_offset, int n_q,
                           int n_kv, int d_h, float scale, int causal,
                           hipStream_t stream);

/*
 * Merge of two partial attention results over disjoint key sets into the
 * result over their union: with m = max(lse_a, lse_b),
 * w_x = exp(lse_x - m),
 *     out     = (w_a o_a + w_b o_b) / (w_a + w_b),
 *     lse_out = m + ln(w_a + w_b).
 * This is the online-softmax step ("Long-Context Attention Explained",
 * section "Online softmax": two running maxima and sums combine by rescaling
 * to the larger max) applied to finished rows, so a query block can attend
 * to keys held in separate buffers (say a cached prefix and the chunk's own
 * keys) or split over launches.  A side whose weight is 0 (lse = -inf: no
 * visible key) contributes nothing, whatever its o holds; if both lse are
 * -inf the row is 0 with lse -inf.
 *   o_a, o_b, out      : device pointers, bf16 [rows, d_h] (any row-major
 *                        tensor whose last axis is d_h, e.g. [B, n_q, L, d_h])
 *   lse_a, lse_b, lse_out : device pointers, fp32 [rows]
 *   rows >= 1, d_h in {64, 128}; out and lse_out may not overlap any other
 *   buffer (the inputs may overlap each other).  Arithmetic in fp32, out
 *   rounded to bf16 (nearest even).  Errors as for attn_prefill_fwd.
 */
int attn_merge_partials(const void *o_a, const float *lse_a, const void *o_b,
                        const float *lse_b, void *out, float *lse_out, long long rows,
                        int d_h, hipStream_t stream);

/*
 * FP8 chunked prefill: attn_prefill_fwd_chunk with Q, K and V given as OCP
 * e4m3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite 448) and one fp32 descale
 * factor per tensor, true value = decoded code x descale.  FP8 matrix-core
 * products buy throughput on the compute-dense part of prefill ("flops /
 * prefill-attention", section "Workarounds", FP8 attention).
 *   q      : device pointer, e4m3 [B, n_q, Lq, d_h]   (one byte per element)
 *   k, v   : device pointers, e4m3 [B, n_kv, Lk, d_h]
 *   out    : device pointer, bf16 [B, n_q, Lq, d_h]; lse: fp32 [B, n_q, Lq]
 *   d_h must be 128; scale, descale_q, descale_k, descale_v finite; the
 *   other arguments, the causal rule and q_offset as for
 *   attn_prefill_fwd_chunk.
 * Numerics: Q K^T in e4m3 x e4m3 with fp32 accumulation (exact products);
 * the softmax in fp32; the weights P, taken relative to a running reference
 * max that is never more than 2^8 below the row max seen so far, are rounded
 * to e4m3 (nearest even: relative error <= 2^-4, and weights below 2^-10 of
 * the reference round to 0) before P V; the row sum adds the unrounded
 * weights; O = descale_v x (P V) / sum, rounded once to bf16.
 * Errors as for attn_prefill_fwd_chunk (ATTN_PREFILL_ERR_BAD_HEADDIM for
 * d_h != 128, ATTN_PREFILL_ERR_BAD_SCALE also when scale x descale_q x
 * descale_k overflows fp32).
 */
int attn_prefill_fwd_fp8(const void *q, const void *k, const void *v, void *out, float *lse,
                         int B, int Lq, int Lk, int q_offset, int n_q, int n_kv, int d_h,
                         float scale, float descale_q, float descale_k, float descale_v,
                         int causal, hipStream_t stream);

/*
 * Backward pass: the gradients of O with respect to Q, K and V for an
 * upstream gradient dO, recomputed from the forward pass's LSE instead of a
 * stored score matrix ("Long-Context Attention Explained", section "What
 * FlashAttention does not change").  With P_ij = exp(s_ij - LSE_i) over the
 * visible keys:
 *     delta_i = dO_i . O_i
 *     dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . v_j - delta_i)
 *     dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i
 * dK and dV sum over the g query heads of each key/value head.
 *   q, out, dout : device pointers, bf16 [B, n_q, L, d_h] (out is the
 *                  forward output)
 *   k, v         : device pointers, bf16 [B, n_kv, L, d_h]
 *   lse          : device pointer, fp32 [B, n_q, L], the forward LSE
 *   dq           : device pointer, bf16 [B, n_q, L, d_h], written entirely
 *   dk, dv       : device pointers, bf16 [B, n_kv, L, d_h], written entirely
 *   delta        : device pointer, fp32 [B, n_q, L], written (delta_i)
 *   d_h in {64, 128}; other arguments as attn_prefill_fwd.
 * Numerics: P is recomputed in fp32 from lse, delta from the bf16 out; P and
 * dS are rounded to bf16 (nearest even) for the matrix-core products, which
 * accumulate in fp32; the gradients are rounded to bf16 once.  The outputs
 * may not overlap each other or any input.  Errors as for attn_prefill_fwd.
 */
int attn_prefill_bwd(const void *q, const void *k, const void *v, const void *out,
                     const float *lse, const void *dout, void *dq, void *dk, void *dv,
                     float *delta, int B, int L, int n_q, int n_kv, int d_h, float scale,
                     int causal, hipStream_t stream);

/*
 * Decode: one new query per sequence against the sequence's whole K/V cache.
 * The query is token Lk - 1 of its sequence, its own key and value already in
 * the cache, so it sees every cached key; attention becomes a matrix-vector
 * product against the cache and its cost is reading the cache
 * ("Memory-bound vs compute-bound", sections "Prefill against decode" and
 * "Attention itself"; "Long-Context Attention Explained", the paragraphs on
 * prefill against decode).  The
 * result is the chunked prefill of one query at q_offset = Lk - 1.
 *   q, out : device pointers, bf16 [B, n_q, d_h] (one token per sequence)
 *   k, v   : device pointers, bf16 [B, n_kv, kv_capacity, d_h]: the cache,
 *            of which rows 0 .. Lk - 1 of each (b, kv-head) are read
 *   lse    : device pointer, fp32 [B, n_q]
 *   Lk >= 1 keys, kv_capacity >= Lk rows allocated per (b, kv-head);
 *   n_q % n_kv == 0 with at most 32 query heads per key/value head;
 *   d_h in {64, 128}; scale any finite value.
 *   workspace : device pointer, 16-byte aligned, at least
 *               attn_decode_workspace_bytes(B, Lk, n_q, n_kv, d_h) bytes,
 *               owned by the caller; it holds fp32 partial results of key
 *               ranges between the two kernels of a call, so two calls that
 *               share a workspace must be ordered (same stream).  Its
 *               contents need no initialisation and are garbage afterwards.
 * Numerics: Q K^T and P V as in attn_prefill_fwd; the partial results of the
 * key ranges stay in fp32 and merge by their LSEs, O is rounded to bf16 once.
 * out, lse and workspace may not overlap each other or any input.  Errors as
 * for attn_prefill_fwd, plus ATTN_PREFILL_ERR_BAD_OFFSET (kv_capacity < Lk),
 * ATTN_PREFILL_ERR_UNSUPPORTED and ATTN_PREFILL_ERR_WORKSPACE.
 */
int attn_decode_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                    int B, int Lk, long long kv_capacity, int n_q, int n_kv, int d_h,
                    float scale, void *workspace, size_t workspace_bytes,
                    hipStream_t stream);

/* Workspace bytes attn_decode_fwd needs for these sizes; 0 for sizes it
 * rejects (or whose workspace size overflows). */
size_t attn_decode_workspace_bytes(int B, int Lk, int n_q, int n_kv, int d_h);

/*
 * attn_decode_fwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, layouts, numerics and
 * errors as attn_decode_fwd minus the workspace; the same kernels run, on a
 * static device scratch array of attn_decode_scratch_bytes() bytes (16 MiB)
 * that the library holds on each GPU it runs on until the process ends.  Its
 * device address is looked up on the first call on a device (with that device
 * current); nothing is allocated, neither there nor on any call.
 *   Sizes whose attn_decode_workspace_bytes() exceed the scratch return
 *   ATTN_PREFILL_ERR_SCRATCH and enqueue nothing; a failed address lookup
 *   returns ATTN_PREFILL_ERR_LAUNCH.
 *   The scratch needs no initialisation (every partial is written before it
 *   is read) and keeps the last call's partials afterwards.
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   in time on one GPU (different streams, or different host threads without
 *   ordering) race on it and must be ordered by the caller, e.g. by issuing
 *   them on one stream.
 */
int attn_decode_fwd_noalloc(const void *q, const void *k, const void *v, void *out, float *lse,
                            int B, int Lk, long long kv_capacity, int n_q, int n_kv, int d_h,
                            float scale, hipStream_t stream);

/* Bytes of the static scratch attn_decode_fwd_noalloc uses (16 MiB). */
size_t attn_decode_scratch_bytes(void);

/*
 * Diagnostic: the work list and static schedule a forward launch
 * (attn_prefill_fwd / attn_prefill_fwd_chunk, and attn_prefill_fwd_fp8, whose
 * work items are the same) of this shape would use on n_cu compute units,
 * computed on the host by the code the kernels run; no GPU call.  A work item
 * is (batch, kv-head, head group, q-block); the persistent grid computes the
 * list in rounds, the early ones statically, the rest as a dynamic tail in
 * list order ("Long-Context Attention Explained", the causal work and its
 * balance over thread blocks; the scheduling itself is this library's).
 *   B, Lq, Lk, q_offset, n_q, n_kv, d_h, causal : as for attn_prefill_fwd_chunk
 *   n_cu    : compute units the grid is sized for (>= 1)
 *   plan    : host pointer, 8 values written: grid, n_items, n_qblk, items
 *             per q-block, sg (stream-block run, 0 = none), pair_t (q-blocks
 *             below it form the tail of a balanced-pair list, 0 = no pairs),
 *             pair rounds, static rounds before the dynamic tail
 *   list    : host pointer to 3 * n_items ints or NULL: (q-block, head group,
 *             stream = b * n_kv + kv-head) of each list entry
 *   rounds  : host pointer to ceil(n_items / grid) * grid ints or NULL: the
 *             list entry workgroup w computes in round r of the all-static
 *             schedule (r * grid + w), -1 past the list
 * Call with list = rounds = NULL first to size them.  Returns ATTN_PREFILL_OK,
 * ATTN_PREFILL_ERR_NULL_PTR (plan NULL) or the shape errors of
 * attn_prefill_fwd_chunk (ATTN_PREFILL_ERR_BAD_SHAPE also for n_cu < 1).
 */
int attn_prefill_schedule(int B, int Lq, int Lk, int q_offset, int n_q, int n_kv, int d_h,
                          int causal, int n_cu, long long *plan, int *list, int *rounds);

/* Static text for a status code (never NULL). */
const char *attn_prefill_strerror(int status);

/* Library version: major * 10000 + minor * 100 + patch. */
int attn_prefill_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_PREFILL_H */
