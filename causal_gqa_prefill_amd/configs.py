"""The attention-layer workloads this library is measured and tested on.

Shapes: "flops / prefill-attention", section "Arithmetic intensity", names the
Llama-2-7B (MHA), Llama-3-8B (GQA-4) and Llama-2-70B (GQA-8) attention
geometries; "Long-Context Attention Explained" gives the made-up 36-query /
6-key-value-head, 128-wide shape at 128K tokens.  Inputs are synthetic
N(0, 1) bf16 tensors drawn from a seed (seed = 1000 + config index); no
trained weights or activations are involved.

Chunked-prefill workloads ("flops / prefill-attention", section
"Workarounds": a long prompt prefilled in pieces) put a chunk of Lq queries
at key position q_offset of a longer K/V; seed = 2000 + index.

Decode workloads (one new token per sequence against its whole cache,
"Memory-bound vs compute-bound", section "Prefill against decode") use the
same geometries, batched at 8K and 32K context, and the 128K-token prompt of
"Long-Context Attention Explained"; seed = 3000 + index.
"""
from dataclasses import dataclass
import math

import numpy as np


@dataclass(frozen=True)
class AttnConfig:
    index: int
    name: str
    B: int
    L: int
    n_q: int
    n_kv: int
    d_h: int
    causal: bool = True
    sampled_rows: int = 0  # 0: the oracle checks every row

    @property
    def g(self) -> int:
        return self.n_q // self.n_kv

    @property
    def scale(self) -> float:
        """1/sqrt(d_h) rounded to fp32, the value the library receives."""
        return float(np.float32(1.0 / math.sqrt(self.d_h)))

    @property
    def seed(self) -> int:
        return 1000 + self.index

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} L={self.L} n_q={self.n_q} "
                f"n_kv={self.n_kv} d_h={self.d_h} causal={int(self.causal)}")


CONFIGS = [
    AttnConfig(1, "tiny causal MHA", 1, 128, 4, 4, 64),
    AttnConfig(2, "Llama-2-7B-shaped MHA layer", 4, 2048, 32, 32, 128),
    AttnConfig(3, "Llama-3-8B-shaped GQA-4 layer", 1, 8192, 32, 8, 128),
    AttnConfig(4, "Llama-2-70B-shaped GQA-8 layer", 1, 32768, 64, 8, 128,
               sampled_rows=4096),
    AttnConfig(5, "synthetic wide GQA-6 long context", 1, 131072, 36, 6, 128,
               sampled_rows=4096),
]


# One GPU's share of the Llama-2-70B-shaped GQA-8 layer when the layer is
# split by key/value head over eight GPUs: each GPU holds one key/value head
# and its eight query heads, and no byte crosses between GPUs.  A whole GPU
# then works on a single key/value stream.
SHARE_CONFIG = AttnConfig(6, "one GPU's share (1 of 8 key/value heads) of the "
                          "Llama-2-70B-shaped GQA-8 layer", 1, 32768, 8, 1, 128,
                          sampled_rows=4096)


def config(index: int) -> AttnConfig:
    """Config by its 1-based index (6: the one-GPU share above)."""
    if index == SHARE_CONFIG.index:
        return SHARE_CONFIG
    if not 1 <= index <= len(CONFIGS):
        raise ValueError(f"no workload {index}")
    return CONFIGS[index - 1]


@dataclass(frozen=True)
class ChunkConfig:
    index: int
    name: str
    B: int
    Lq: int
    Lk: int
    q_offset: int
    n_q: int
    n_kv: int
    d_h: int
    causal: bool = True
    sampled_rows: int = 0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_h)))

    @property
    def seed(self) -> int:
        return 2000 + self.index

    def visible_pairs(self) -> int:
        """(query, key) pairs per head that attention actually forms."""
        if not self.causal:
            return self.Lq * self.Lk
        first = self.q_offset + 1
        last = self.q_offset + self.Lq
        return (first + last) * self.Lq // 2

    def flops(self) -> int:
        """2 * d_h flops per visible pair for Q K^T and as many for P V."""
        return 4 * self.B * self.n_q * self.d_h * self.visible_pairs()

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} Lq={self.Lq} Lk={self.Lk} q_offset={self.q_offset} "
                f"n_q={self.n_q} n_kv={self.n_kv} d_h={self.d_h} causal={int(self.causal)}")


CHUNK_CONFIGS = [
    ChunkConfig(1, "Llama-3-8B-shaped GQA-4, last 4K chunk of a 32K prompt",
                1, 4096, 32768, 28672, 32, 8, 128, sampled_rows=2048),
    ChunkConfig(2, "Llama-2-70B-shaped GQA-8, 2K chunk at 8K of a 16K cache",
                1, 2048, 16384, 8192, 64, 8, 128, sampled_rows=2048),
]


def chunk_config(index: int) -> ChunkConfig:
    return CHUNK_CONFIGS[index - 1]


@dataclass(frozen=True)
class DecodeConfig:
    index: int
    name: str
    B: int
    Lk: int
    n_q: int
    n_kv: int
    d_h: int
    sampled_rows: int = 0

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / math.sqrt(self.d_h)))

    @property
    def seed(self) -> int:
        return 3000 + self.index

    def kv_bytes(self) -> int:
        return 2 * self.B * self.n_kv * self.Lk * self.d_h * 2

    def describe(self) -> str:
        return (f"{self.name}: B={self.B} Lk={self.Lk} n_q={self.n_q} n_kv={self.n_kv} "
                f"d_h={self.d_h}")


DECODE_CONFIGS = [
    DecodeConfig(1, "Llama-3-8B-shaped GQA-4 decode, batch 32 at 8K context",
                 32, 8192, 32, 8, 128, sampled_rows=256),
    DecodeConfig(2, "synthetic wide GQA-6 decode after a 128K prompt",
                 1, 131072, 36, 6, 128),
    DecodeConfig(3, "Llama-2-70B-shaped GQA-8 decode, batch 8 at 32K context",
                 8, 32768, 64, 8, 128, sampled_rows=256),
]


def decode_config(index: int) -> DecodeConfig:
    return DECODE_CONFIGS[index - 1]
