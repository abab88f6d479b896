"""block_wise_rank_amd -- MILO block-wise low-rank KV compression and decode
attention over the compressed blocks, as hand-written HIP kernels for the AMD
Instinct MI355X (gfx950) behind the C ABI in include/milo.h.

The Python side is a thin binding: tensors and streams come from PyTorch, every
computation runs in libmilo.so (built in-tree by ``build.build()``).  Importing
the binding functions requires the built library; there is no fallback path.
"""
from .binding import (  # noqa: F401
    Factors,
    MiloError,
    NotConvergedError,
    decode_workspace_bytes,
    milo_abi_version,
    milo_allocate_ranks,
    milo_allocate_ranks_ex,
    milo_arena_bytes,
    milo_compress_blocks,
    milo_compress_blocks_ex,
    milo_compress_workspace_bytes,
    milo_decode_attention,
    milo_decode_attention_noalloc,
    milo_fetch_blocks,
    milo_profile_enable,
    milo_profile_read,
    milo_reconstruct,
    reconstruct_then_attend,
)
from . import _capi  # noqa: F401

__all__ = [
    "Factors", "MiloError", "NotConvergedError", "decode_workspace_bytes", "milo_abi_version", "milo_allocate_ranks",
    "milo_allocate_ranks_ex", "milo_arena_bytes", "milo_compress_blocks", "milo_compress_blocks_ex",
    "milo_compress_workspace_bytes",
    "milo_decode_attention", "milo_decode_attention_noalloc", "milo_fetch_blocks", "milo_profile_enable", "milo_profile_read", "milo_reconstruct",
    "reconstruct_then_attend",
]
