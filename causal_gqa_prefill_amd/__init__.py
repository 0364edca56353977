"""Causal GQA prefill attention for AMD MI355X (gfx950).

attn_prefill(q, k, v, scale=None, causal=True) -> (out, lse) runs the
hand-written HIP kernels in libattn_prefill.so; attn_prefill_chunk(q, k, v,
q_offset) prefills a chunk of queries against a longer key/value sequence, and
merge_partials(...) combines results over disjoint key sets by their
log-sum-exp; attn_decode(q, k, v) attends one new query per sequence to its
whole K/V cache; attn_prefill_fp8(...) is the prefill on OCP e4m3 inputs, and
attn_prefill_backward(...) the gradients from the saved LSE.
Importing the package loads
nothing; the first use of the attention entry points loads the library and
raises if it is missing (there is no CPU fallback).
"""

__all__ = ["attn_prefill", "attn_prefill_into", "attn_prefill_chunk", "attn_prefill_chunk_into",
           "merge_partials", "attn_decode", "attn_decode_into", "decode_workspace_bytes",
           "attn_prefill_fp8", "attn_prefill_fp8_into", "attn_prefill_backward",
           "library", "AttnPrefillError"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
