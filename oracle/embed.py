"""Float64 CPU oracle of the ViT front end: patch extraction and token embedding.

TEST INFRASTRUCTURE ONLY (as ``oracle.block``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg use it,
and it shares nothing with the HIP library.

Source: mlgrind.dev, "E2E: Tiny Vision Transformer" [MLG] -- "Architecture"
(patchify, then @ W_patch + b_patch, prepend the class token, add position
embeddings), "Details" (patches in row-major order over the (H/P, W/P) grid,
each flattened as (p1, p2, c), which matches a stride-P convolution) and
"Examples" (the printed patchify example).

Reading: the nipunbatra.github.io vision1 transcript flattens a patch channel
by channel ((c, p1, p2), the layout of a Conv2d weight); [MLG] states the
order explicitly and prints an example of it, so this follows [MLG].  Either
order is the same linear map up to a permutation of W_patch's rows.
"""

from __future__ import annotations

import numpy as np

__all__ = ["patchify", "patch_embed"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def patchify(images, patch: int) -> np.ndarray:
    """(B, C, H, W) -> (B, (H/P)(W/P), P*P*C): [MLG] "Details" patch order.

    Patch (i, j) of the grid is token i * (W/P) + j; inside it the value of
    pixel (p1, p2) of channel c sits at position (p1 * P + p2) * C + c.
    """
    x = _f64(images)
    b, c, h, w = x.shape
    if h % patch or w % patch:
        raise ValueError("image sides must be multiples of the patch size")
    gh, gw = h // patch, w // patch
    t = x.reshape(b, c, gh, patch, gw, patch)          # b c gh p1 gw p2
    t = t.transpose(0, 2, 4, 3, 5, 1)                  # b gh gw p1 p2 c
    return t.reshape(b, gh * gw, patch * patch * c)


def patch_embed(images, w_patch, patch: int, b_patch=None, cls_token=None,
                pos_emb=None) -> np.ndarray:
    """Tokens entering the encoder: (B, N [+1], D).

    [MLG] "Architecture": patchify(x) @ W_patch + b_patch, then the class
    token prepended as token 0 (if given), then position embeddings
    (N [+1], D) added to every sequence (if given).
    """
    t = np.matmul(patchify(images, patch), _f64(w_patch))
    if b_patch is not None:
        t = t + _f64(b_patch)
    if cls_token is not None:
        c = np.broadcast_to(_f64(cls_token), (t.shape[0], 1, t.shape[2]))
        t = np.concatenate([c, t], axis=1)
    if pos_emb is not None:
        t = t + _f64(pos_emb)[None]
    return t
