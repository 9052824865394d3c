"""Seeded synthetic inputs for the encoder block, shared by tests, bench and smoke.

This module holds no arithmetic of the block: it only draws the input tensors,
scales the weights to their initial spread and casts them to the device
dtype.  Both the HIP path and the float64 oracle consume exactly the values
returned here, so a parity check compares the two on identical inputs.

Recipe
------
* Generator: ``numpy.random.default_rng(seed)`` (PCG64), seed 0 by default.
* Draw order: x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, each ``standard_normal``
  in float64, row-major in the shapes (N, T, D), (D, D) x4, (D, F), (F, D).
* x ~ N(0, 1); every weight ~ N(0, 1/fan_in) (standard deviation
  1/sqrt(fan_in), fan_in = D for w_q, w_k, w_v, w_o, w_mlp1 and F for
  w_mlp2), the initialisation of mlgrind.dev "E2E: Tiny Vision Transformer",
  section "Details".
* Cast to the device dtype with round-to-nearest-even (bf16: the top 16 bits
  of the float32 value after RNE; fp32: numpy's float64 -> float32 cast).
  The float64 arrays returned are those rounded values, upcast exactly.

Backward (``make_dout``): the gradient arriving at the block's output is
drawn by a third generator, ``numpy.random.default_rng([seed, 4])``, as
standard_normal (N, T, D) then rounded: unit scale, like the output itself.
The pages train with a cross-entropy loss on class labels (nipunbatra.github.io
vision1 transcript, Page 113); its gradient at one block depends on the
layers above and the labels, and a seeded N(0, 1) tensor stands in for it.

Affine variant (``make_affine_params``): a second, independent generator,
``numpy.random.default_rng([seed, 1])``, draws in the order ln1_gamma,
ln1_beta, b_q, b_k, b_v, b_o, ln2_gamma, ln2_beta, b_mlp1, b_mlp2 (lengths D,
except F for b_mlp1): gains 1 + 0.1 N(0, 1), shifts and biases 0.1 N(0, 1),
then the same rounding.  The pages initialise gains to 1 and shifts and
biases to 0 (mlgrind.dev, "Details"); trained values differ from that, and
these stand in for them so that every term is visible in a parity check.

The workloads are the shapes of ViT-B/16, ViT-L/16 and ViT-H/14 (widths and
MLP sizes from ai-engineer-exhaustive.pages.dev "ViT Encoder Block", section
"Paper Context"), with T = patches + 1 class token (224/16 -> 197,
224/14 -> 257, 512/16 -> 1025), plus a tiny fp32 case (8x8 image, 4x4
patches -> 4 patches + CLS, as in mlgrind.dev's TinyViT example).  They stand
in for the photographs and pretrained checkpoints the pages use; no dataset
item is reproduced.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "bf16_round", "round_to", "make_block_inputs",
           "AFFINE_PARAM_ORDER", "make_affine_params", "make_dout"]

AFFINE_PARAM_ORDER = ("ln1_gamma", "ln1_beta", "b_q", "b_k", "b_v", "b_o",
                      "ln2_gamma", "ln2_beta", "b_mlp1", "b_mlp2")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    N: int
    T: int
    D: int
    H: int
    F: int
    eps: float
    dtype: str  # "fp32" | "bf16"

    @property
    def M(self) -> int:
        return self.N * self.T

    @property
    def dh(self) -> int:
        return self.D // self.H

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", N=4, T=5, D=16, H=2, F=32, eps=1e-5, dtype="fp32"),
    "vit_b16": Workload("vit_b16", N=64, T=197, D=768, H=12, F=3072, eps=1e-6, dtype="bf16"),
    "vit_l16": Workload("vit_l16", N=256, T=197, D=1024, H=16, F=4096, eps=1e-6, dtype="bf16"),
    "vit_h14": Workload("vit_h14", N=128, T=257, D=1280, H=16, F=5120, eps=1e-6, dtype="bf16"),
    "long_t1025": Workload("long_t1025", N=16, T=1025, D=768, H=12, F=3072, eps=1e-6,
                           dtype="bf16"),
}


def bf16_round(a) -> np.ndarray:
    """Round float values to the nearest bfloat16 (ties to even); return float64.

    The value is first rounded to float32, then its low 16 mantissa bits are
    rounded away with ties going to the even neighbour.  Finite inputs only.
    """
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = (u.astype(np.uint32) << 16).view(np.float32)
    return out.astype(np.float64)


def round_to(a, dtype: str) -> np.ndarray:
    """Round to the device dtype ("bf16" or "fp32") and return exact float64 values."""
    if dtype == "bf16":
        return bf16_round(a)
    if dtype == "fp32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_block_inputs(N: int, T: int, D: int, F: int, dtype: str, seed: int = 0) -> dict:
    """Draw x and the six weights; return float64 arrays holding device-exact values."""
    rng = np.random.default_rng(seed)
    shapes = [("x", (N, T, D), 1.0),
              ("w_q", (D, D), 1.0 / math.sqrt(D)),
              ("w_k", (D, D), 1.0 / math.sqrt(D)),
              ("w_v", (D, D), 1.0 / math.sqrt(D)),
              ("w_o", (D, D), 1.0 / math.sqrt(D)),
              ("w_mlp1", (D, F), 1.0 / math.sqrt(D)),
              ("w_mlp2", (F, D), 1.0 / math.sqrt(F))]
    out = {}
    for name, shape, std in shapes:
        out[name] = round_to(rng.standard_normal(shape) * std, dtype)
    return out


def make_affine_params(D: int, F: int, dtype: str, seed: int = 0) -> dict:
    """Draw the affine variant's gains, shifts and biases (device-exact float64)."""
    rng = np.random.default_rng([seed, 1])
    out = {}
    for name in AFFINE_PARAM_ORDER:
        n = F if name == "b_mlp1" else D
        z = rng.standard_normal(n)
        out[name] = round_to(1.0 + 0.1 * z if name.endswith("gamma") else 0.1 * z, dtype)
    return out


def make_dout(N: int, T: int, D: int, dtype: str, seed: int = 0) -> np.ndarray:
    """dL/d(out) for the backward: N(0, 1), device-exact float64."""
    rng = np.random.default_rng([seed, 4])
    return round_to(rng.standard_normal((N, T, D)), dtype)
