"""Named synthetic workloads for the indexer -> top-k -> sparse-attention path.

Each workload fixes the shapes, the selection size k, the attention shape and the
input recipe (value distributions, planted keys, key-mean drift).  The sizes follow
the pages' regime: k = 2048 selected keys, which "The 2,048 tokens are 0.2 percent of
a 1M context" in "GLM 5.2: How Four Co-Designed Mechanisms Beat Raw Scale", Part II,
"DeepSeek Sparse Attention", Stage 2; a group of 4 sparse layers sharing one
selection ("IndexShare: Amortizing the Indexer" on the same page; the twiscan post on
GLM-5.2's IndexShare); a 1M-token context ("The 1M Context Mirage: What IndexShare
Actually Delivers").
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    name: str
    B: int            # sequences
    T: int            # query tokens per sequence
    S: int            # key capacity per sequence (S_max); kv_len defaults to S
    pos0: int         # position of query t=0 (query t sits at pos0 + t)
    H_I: int          # indexer heads
    d_I: int          # indexer head dim (FP8 e4m3)
    k: int            # keys kept per query
    H_q: int          # attention query heads
    H_kv: int         # attention KV heads
    d: int            # attention head dim (bf16)
    layers: int       # sparse-attention layers sharing one selection
    seed: int
    qkv_std: float    # std of the q/K/V draws before bf16 rounding
    planted: int = 0  # planted keys per query (+4 sigma boost through the query)
    drift: float = 0.0  # std of the per-1024-key-block random-walk step of the key mean
    kv_lens: Optional[Tuple[int, ...]] = None  # per-sequence kv_len (default: S for all)
    pos0s: Optional[Tuple[int, ...]] = None    # per-sequence pos0 (default: pos0 for all)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def kv_len_list(self):
        return list(self.kv_lens) if self.kv_lens is not None else [self.S] * self.B

    def pos0_list(self):
        return list(self.pos0s) if self.pos0s is not None else [self.pos0] * self.B

    def visible(self, b: int, t: int) -> int:
        """Keys visible to query t of sequence b: positions [0, n_t)."""
        return max(0, min(self.pos0_list()[b] + t + 1, self.kv_len_list()[b]))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


_R = 1.0 / math.sqrt(128.0)

WORKLOADS = {
    # 1K causal prefill, 4 indexer heads of width 64, top-64, 8-head MQA of width 64.
    "tiny_prefill_1k": Workload("tiny_prefill_1k", B=1, T=1024, S=1024, pos0=0, H_I=4, d_I=64,
                                k=64, H_q=8, H_kv=1, d=64, layers=1, seed=0, qkv_std=1.0,
                                planted=16),
    # 32K causal prefill, one layer.
    "prefill_32k": Workload("prefill_32k", B=1, T=32768, S=32768, pos0=0, H_I=64, d_I=128,
                            k=2048, H_q=16, H_kv=1, d=128, layers=1, seed=1, qkv_std=_R),
    # 128K causal prefill, one selection shared by a group of 4 layers.
    "group4_prefill_128k": Workload("group4_prefill_128k", B=1, T=131072, S=131072, pos0=0,
                                    H_I=64, d_I=128, k=2048, H_q=16, H_kv=1, d=128, layers=4,
                                    seed=2, qkv_std=_R),
    # Decode: 64 sequences, 1 new token each against a 128K cache, group of 4 layers.
    "decode_b64_128k": Workload("decode_b64_128k", B=64, T=1, S=131072, pos0=131071, H_I=64,
                                d_I=128, k=2048, H_q=16, H_kv=1, d=128, layers=4, seed=3,
                                qkv_std=_R, planted=32),
    # 1M-key chunked prefill: 4096 queries at positions 1044480..1048575, group of 4 layers.
    "chunk_prefill_1m": Workload("chunk_prefill_1m", B=1, T=4096, S=1048576, pos0=1044480,
                                 H_I=64, d_I=128, k=2048, H_q=16, H_kv=1, d=128, layers=4,
                                 seed=4, qkv_std=_R, planted=64, drift=0.02),
}

# The workload the throughput line is quoted on: 128K prefill with a 4-layer group.
BENCH_WORKLOAD = "group4_prefill_128k"
