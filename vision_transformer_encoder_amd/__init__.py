"""MI355X-native forward pass of one pre-LayerNorm ViT encoder block.

The computation runs in hand-written HIP kernels for gfx950 inside
``libvitblk.so`` (C ABI declared in ``include/vitblk.h``); this package is the
thin ctypes binding over it plus the seeded synthetic-input generator
(``inputs``).  Importing the package loads neither torch nor the library; the
first call does, and it raises if the library has not been built.
"""

from ._lib import (  # noqa: F401
    AFFINE_KEYS,
    EPI_GELU,
    EPI_GELU_GRAD,
    GRAD_KEYS,
    EPI_NONE,
    EPI_RESIDUAL,
    NOALLOC_SCRATCH_BYTES,
    VITBLK_BF16,
    VITBLK_FP32,
    VitblkError,
    attention,
    attention_first_queries,
    attention_backward,
    attention_backward_workspace_bytes,
    affine_fold,
    backward,
    backward_workspace_bytes,
    encoder_forward,
    encoder_workspace_bytes,
    forward,
    forward_affine,
    forward_packed,
    forward_packed_affine,
    forward_packed_noalloc,
    layernorm,
    layernorm_backward,
    linear,
    linear_normed,
    linear_residual_row_stats,
    linear_residual_row_stats_workspace_bytes,
    load,
    pack_weights,
    packed_col_sums,
    packed_views,
    packed_weights_bytes,
    patch_embed,
    patch_embed_workspace_bytes,
    qkv_projection,
    row_stats,
    status_string,
    weight_grad,
    weight_grad_workspace_bytes,
    workspace_bytes,
)
