"""Float64 CPU oracle of the pre-LN ViT encoder block (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path never does.
"""

from .block import (  # noqa: F401
    AFFINE_KEYS,
    add_bias,
    affine,
    attention_scores,
    attention_weights,
    encoder,
    gelu_tanh,
    layer_norm,
    layer_norm_stats,
    merge_heads,
    multi_head_attention,
    project,
    softmax_rows,
    split_heads,
    vit_block,
    vit_block_stages,
)
from .embed import patch_embed, patchify  # noqa: F401
from .backward import (  # noqa: F401
    GRAD_KEYS,
    attention_backward,
    gelu_tanh_grad,
    layer_norm_backward,
    softmax_backward,
    vit_block_backward,
    vit_block_backward_stages,
)
