"""MI355X (gfx950) FAVOR attention: HIP kernels behind a C ABI (include/favor.h).

The Python layer is a thin ctypes binding over libfavor.so; torch supplies
device memory and streams only.
"""
from ._lib import (  # noqa: F401
    EXPORTS, FavorError, LIB_PATH, favor_attention, favor_attention_noalloc,
    favor_attention_resolve_path,
    favor_attention_backward, favor_attention_backward_resolve_path,
    favor_attention_backward_workspace_bytes,
    favor_attention_workspace_bytes, favor_embed_bf16, favor_linear_bf16, favor_orf_omega,
    favor_pack_weight_bf16, favor_embed_linear_bf16, favor_block_weights, BlockWeights,
    favor_performer_block, favor_profile_attention, lib, loaded_hip_runtimes, status_string,
)
from .autograd import FavorAttentionFunction, favor_attention_fn  # noqa: F401,E402
