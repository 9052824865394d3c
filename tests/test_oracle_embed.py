"""Pins for the front-end oracle (patch extraction and token embedding), CPU only.

* the printed patchify example of mlgrind.dev "E2E: Tiny Vision Transformer",
  section "Examples" (tests/golden/mlg_patchify_example.json);
* the stride-P convolution the page says the patch order matches, computed
  by torch's conv2d in float64 (a different formulation of the same map);
* a scalar loop over (image, patch, pixel, channel) on tiny inputs;
* the invariance the page's "Why position embeddings matter" states: without
  position embeddings, permuting the patches permutes the tokens;
* planted mistakes (channel-first flattening, column-major patch grid,
  position embeddings added before the class token) are each caught.
"""

import json
import os

import numpy as np
import pytest

import oracle
from oracle import embed as oe

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mlg_patchify_example.json")


def _golden_ok():
    g = json.load(open(GOLDEN))
    x = np.arange(np.prod(g["image_shape"]), dtype=np.float64).reshape(g["image_shape"])
    p = oracle.patchify(x, g["patch_size"])
    return list(p.shape) == g["output_shape"] and np.array_equal(p[0, 0], g["first_patch"])


def _brute_embed(x, w, P, b=None, cls=None, pos=None):
    B, C, H, W = x.shape
    D = w.shape[1]
    gw = W // P
    toks = []
    for n in range(B):
        seq = []
        if cls is not None:
            seq.append([float(cls[d]) for d in range(D)])
        for i in range(H // P):
            for j in range(gw):
                row = [0.0] * D
                for p1 in range(P):
                    for p2 in range(P):
                        for c in range(C):
                            k = (p1 * P + p2) * C + c
                            v = x[n, c, i * P + p1, j * P + p2]
                            for d in range(D):
                                row[d] += v * w[k, d]
                if b is not None:
                    row = [row[d] + b[d] for d in range(D)]
                seq.append(row)
        if pos is not None:
            seq = [[seq[t][d] + pos[t, d] for d in range(D)] for t in range(len(seq))]
        toks.append(seq)
    return np.array(toks)


def _brute_err():
    rng = np.random.default_rng(5)
    worst = 0.0
    for (B, C, H, W, P, D, with_cls) in [(2, 3, 4, 6, 2, 5, True), (1, 2, 6, 6, 3, 4, False),
                                         (2, 1, 4, 4, 4, 3, True)]:
        x = rng.standard_normal((B, C, H, W))
        w = rng.standard_normal((P * P * C, D))
        b = rng.standard_normal(D)
        n = (H // P) * (W // P) + (1 if with_cls else 0)
        cls = rng.standard_normal(D) if with_cls else None
        pos = rng.standard_normal((n, D))
        got = oracle.patch_embed(x, w, P, b, cls, pos)
        worst = max(worst, float(np.abs(got - _brute_embed(x, w, P, b, cls, pos)).max()))
    return worst


def test_mlg_patchify_example():
    assert _golden_ok()


def test_patch_embed_brute_force_agrees():
    assert _brute_err() < 1e-12


def test_patch_embed_is_a_stride_p_convolution():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    B, C, H, W, P, D = 2, 3, 8, 12, 4, 7
    x = rng.standard_normal((B, C, H, W))
    w = rng.standard_normal((P * P * C, D))
    b = rng.standard_normal(D)
    # Conv weight [D, C, P, P] holding the same numbers: w[(p1 P + p2) C + c, d].
    conv_w = w.reshape(P, P, C, D).transpose(3, 2, 0, 1)
    y = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(conv_w.copy()),
                                   torch.from_numpy(b), stride=P)
    want = y.flatten(2).transpose(1, 2).numpy()  # (B, grid cells row-major, D)
    assert np.abs(oracle.patch_embed(x, w, P, b) - want).max() < 1e-12


def test_tokens_follow_patches_without_position_embeddings():
    rng = np.random.default_rng(7)
    B, C, H, W, P, D = 1, 2, 4, 4, 2, 3
    x = rng.standard_normal((B, C, H, W))
    w = rng.standard_normal((P * P * C, D))
    cls = rng.standard_normal(D)
    t = oracle.patch_embed(x, w, P, cls_token=cls)
    # swap grid cells (0, 0) and (1, 1): tokens 1 and 4 swap, the class token stays
    x2 = x.copy()
    x2[..., 0:2, 0:2], x2[..., 2:4, 2:4] = x[..., 2:4, 2:4], x[..., 0:2, 0:2]
    t2 = oracle.patch_embed(x2, w, P, cls_token=cls)
    assert np.array_equal(t2[:, [0, 4, 2, 3, 1]], t)


def test_patch_size_must_divide_the_image():
    with pytest.raises(ValueError):
        oracle.patchify(np.zeros((1, 1, 5, 4)), 2)


def _patchify_channel_first(images, patch):
    x = np.asarray(images, dtype=np.float64)
    b, c, h, w = x.shape
    t = x.reshape(b, c, h // patch, patch, w // patch, patch).transpose(0, 2, 4, 1, 3, 5)
    return t.reshape(b, (h // patch) * (w // patch), patch * patch * c)


def _patchify_column_major(images, patch):
    x = np.asarray(images, dtype=np.float64)
    b, c, h, w = x.shape
    t = x.reshape(b, c, h // patch, patch, w // patch, patch).transpose(0, 4, 2, 3, 5, 1)
    return t.reshape(b, (h // patch) * (w // patch), patch * patch * c)


_EMBED = oe.patch_embed


def _pos_before_cls(images, w_patch, patch, b_patch=None, cls_token=None, pos_emb=None):
    t = _EMBED(images, w_patch, patch, b_patch)
    if pos_emb is not None:
        t = t + np.asarray(pos_emb)[None, : t.shape[1]]
    if cls_token is not None:
        c = np.broadcast_to(np.asarray(cls_token, dtype=np.float64), (t.shape[0], 1, t.shape[2]))
        t = np.concatenate([c, t], axis=1)
    return t


EMBED_MUTANTS = {
    "channel-first flattening": ("patchify", _patchify_channel_first),
    "column-major patch grid": ("patchify", _patchify_column_major),
    "position added before the class token": ("patch_embed", _pos_before_cls),
}


@pytest.mark.parametrize("name", sorted(EMBED_MUTANTS))
def test_embed_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = EMBED_MUTANTS[name]
    monkeypatch.setattr(oe, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    assert not (_golden_ok() and _brute_err() < 1e-9), f"pins did not catch: {name}"
