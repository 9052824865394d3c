"""GPU parity of the front end (patch extraction + embedding GEMM + token rows)
against the float64 oracle (mlgrind.dev "E2E: Tiny Vision Transformer",
"Architecture" and "Details").  Bars: fp32 2e-4 (1 + |o|), bf16 3e-2 (1 + |o|).
"""

import math

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import round_to

from gpu_util import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu


def _case(B, C, H, W, P, D, dtype, seed, cls=True, pos=True, bias=True):
    rng = np.random.default_rng(seed)
    K = P * P * C
    img = round_to(rng.standard_normal((B, C, H, W)), dtype)
    w = round_to(rng.standard_normal((K, D)) / math.sqrt(K), dtype)
    b = round_to(0.1 * rng.standard_normal(D), dtype) if bias else None
    c = round_to(0.02 * rng.standard_normal(D), dtype) if cls else None
    T = (H // P) * (W // P) + (1 if cls else 0)
    p = round_to(0.02 * rng.standard_normal((T, D)), dtype) if pos else None
    return img, w, b, c, p


EMBEDS = [
    # (B, C, H, W, P, D, dtype)
    (2, 3, 8, 8, 4, 16, "fp32"),        # the tiny model's front end
    (3, 1, 8, 12, 4, 24, "fp32"),       # non-square image, one channel
    (4, 3, 224, 224, 16, 768, "bf16"),  # ViT-B/16
    (128, 3, 224, 224, 16, 768, "bf16"),  # 25088 patch rows: big tile + 128x128 tail, token rows
    (2, 3, 224, 224, 14, 1280, "bf16"),  # ViT-H/14: patch width 588 -> padded to 640
    (2, 3, 32, 48, 8, 100, "bf16"),     # D not a multiple of 8: generic GEMM, scalar token rows
    (2, 3, 12, 20, 4, 32, "bf16"),      # image rows not whole 16-byte vectors: per-vector gather
    (1, 3, 32, 32, 8, 64, "bf16"),      # one image: the token rows take a separate pass
]


@pytest.mark.parametrize("B,C,H,W,P,D,dtype", EMBEDS)
def test_patch_embed(B, C, H, W, P, D, dtype):
    img, w, b, c, p = _case(B, C, H, W, P, D, dtype, seed=B + C + H + P + D)
    dev = lambda a: None if a is None else to_dev(a, dtype)  # noqa: E731
    got = to_host(vb.patch_embed(dev(img), dev(w), P, dev(b), dev(c), dev(p)))
    assert_close(got, oracle.patch_embed(img, w, P, b, c, p), dtype,
                 f"patch embed {B}x{C}x{H}x{W} P={P} D={D}")


@pytest.mark.parametrize("cls,pos,bias", [(False, False, False), (True, False, True),
                                          (False, True, True), (True, True, False)])
def test_patch_embed_optional_parts(cls, pos, bias):
    img, w, b, c, p = _case(2, 3, 32, 32, 8, 64, "bf16", seed=11, cls=cls, pos=pos, bias=bias)
    dev = lambda a: None if a is None else to_dev(a, "bf16")  # noqa: E731
    got = to_host(vb.patch_embed(dev(img), dev(w), 8, dev(b), dev(c), dev(p)))
    assert got.shape == (2, 16 + (1 if cls else 0), 64)
    assert_close(got, oracle.patch_embed(img, w, 8, b, c, p), "bf16",
                 f"patch embed cls={cls} pos={pos} bias={bias}")


def test_front_end_into_the_encoder():
    # tokens from the front end feed the encoder directly (ViT-B/16 shapes, 2 blocks)
    from vision_transformer_encoder_amd.inputs import make_affine_params, make_block_inputs
    img, w, b, c, p = _case(2, 3, 224, 224, 16, 768, "bf16", seed=12)
    dev = lambda a: None if a is None else to_dev(a, "bf16")  # noqa: E731
    toks = vb.patch_embed(dev(img), dev(w), 16, dev(b), dev(c), dev(p))
    layers = []
    for l in range(2):
        inp = make_block_inputs(1, 1, 768, 3072, "bf16", seed=100 + l)
        layers.append(dict({k: inp[k] for k in ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]},
                           params=make_affine_params(768, 3072, "bf16", seed=100 + l)))
    packed = [vb.pack_weights(*(to_dev(lay[k], "bf16") for k in ["w_q", "w_k", "w_v", "w_o",
                                                                 "w_mlp1", "w_mlp2"]))
              for lay in layers]
    prm = [{k: to_dev(v, "bf16") for k, v in lay["params"].items()} for lay in layers]
    _, cls = vb.encoder_forward(toks, packed, 3072, 12, 1e-6, params=prm, want_tokens=False)
    ref_t = oracle.patch_embed(img, w, 16, b, c, p)
    _, ref_cls = oracle.encoder(ref_t, layers, 12, 1e-6)
    assert_close(to_host(cls), ref_cls, "bf16", "patch embed -> 2 blocks -> cls",
                 scale=math.sqrt(3))
