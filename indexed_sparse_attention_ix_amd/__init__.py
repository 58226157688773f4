"""MI355X (gfx950) indexed sparse attention: FP8 indexer -> top-k -> sparse attention,
with one selection shared by a group of layers (IndexShare).

The compute lives in libix.so (hand-written HIP kernels behind the C ABI of
include/ix.h); `binding` is its ctypes mirror.  `synth` and `workloads` hold the
seeded synthetic inputs.
"""
from . import binding  # noqa: F401
from .binding import (IxError, ix_abi_version, ix_last_error, ix_score, ix_topk,  # noqa: F401
                      ix_topk_workspace_bytes, indexshare_group, indexshare_group_fwd,
                      indexshare_workspace_bytes, score, sparse_attention, sparse_attn_fwd,
                      sparse_attn_workspace_bytes, topk)

__all__ = ["binding", "IxError", "ix_abi_version", "ix_last_error", "ix_score", "ix_topk",
           "ix_topk_workspace_bytes", "indexshare_group", "indexshare_group_fwd",
           "indexshare_workspace_bytes", "score", "sparse_attention", "sparse_attn_fwd",
           "sparse_attn_workspace_bytes", "topk"]
