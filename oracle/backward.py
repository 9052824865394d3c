"""Float64 CPU oracle for the backward pass of one pre-LayerNorm ViT encoder block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
constant or helper with the HIP library in ``vision_transformer_encoder_amd``.

What it computes.  Training needs the gradient of a scalar loss with respect
to every parameter: [NB] Page 88 (the backward pass computes dL/dtheta for
all blocks), Page 113 (one training step: loss, backward, optimiser step),
and [MLG] "Method contract" (the PyTorch track lets autograd update every
parameter).  For one block this is its vector-Jacobian product: given the
gradient ``dout`` = dL/d(out) arriving from above, return dL/dx (passed on to
the block below) and dL/dW for its six weights.  The pages print no backward
formula, so the reading is the exact derivative of the forward definition in
``oracle.block`` (the plain block: no LayerNorm gain or shift, no biases).

How.  The forward stages are recomputed with ``oracle.block.vit_block_stages``
and then walked in reverse, one stage at a time, each stage's backward
written as the chain rule applied to the forward's own steps (no algebraic
shortcut beyond what each step states).  Sequences never interact, so the
batch is processed ``chunk`` sequences at a time; the weight gradients are
sums over every token and are accumulated over the chunks.

Sources:
  [NB]   nipunbatra.github.io, vision1 lecture transcript -- Page 88
         (gradients flow back through every block), Page 113 (one training
         step).
  [MLG]  mlgrind.dev, "E2E: Tiny Vision Transformer" -- "Method contract".
  [CAC]  crackedaicode.com, "ViT Encoder Block" -- the forward definition
         whose derivative is taken ("Normalize before each stage",
         "Multi-head attention", "Feed-forward stage").

Pins (``tests/test_oracle_backward.py``, none reusing this code): central
finite differences of the oracle's forward, element by element on tiny
inputs and along random directions on larger ones; closed forms (the GELU
derivative's odd-part identity and value at 0, a block whose residual
branches are switched off, a single-token sequence); invariants (the
LayerNorm input gradient is orthogonal to the all-ones vector and to the
normalised row, the key gradient sums to zero over a sequence's tokens,
batch additivity of the weight gradients); torch autograd in float64 as a
library cross-check; and planted mistakes that the pins must catch.
"""

from __future__ import annotations

import math

import numpy as np

from . import block as ob

__all__ = [
    "layer_norm_backward",
    "gelu_tanh_grad",
    "softmax_backward",
    "attention_backward",
    "vit_block_backward_stages",
    "vit_block_backward",
    "GRAD_KEYS",
]

# Gradients returned by vit_block_backward, in the order of the C interface.
GRAD_KEYS = ("dx", "dw_q", "dw_k", "dw_v", "dw_o", "dw_mlp1", "dw_mlp2")

_GELU_C = math.sqrt(2.0 / math.pi)
_GELU_A = 0.044715


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def layer_norm_backward(x, g, eps: float) -> np.ndarray:
    """dL/dx of y = (x - mean) / sqrt(var + eps) (population variance), given g = dL/dy.

    The forward steps of [CAC] "Normalize before each stage", reversed:
    dev = x - mean(x); var = mean(dev^2); r = (var + eps)^(-1/2); y = dev * r.
    """
    x = _f64(x)
    g = _f64(g)
    d = x.shape[-1]
    mean = x.mean(axis=-1, keepdims=True)
    dev = x - mean
    var = (dev * dev).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    # y = dev * r: both factors receive a gradient.
    g_dev = g * r
    g_r = (g * dev).sum(axis=-1, keepdims=True)
    # r = (var + eps)^(-1/2)
    g_var = g_r * (-0.5) * r ** 3
    # var = sum(dev^2) / D
    g_dev = g_dev + g_var * (2.0 / d) * dev
    # dev = x - sum(x) / D: every x_j also moves the mean.
    return g_dev - g_dev.sum(axis=-1, keepdims=True) / d


def gelu_tanh_grad(z) -> np.ndarray:
    """d/dz of 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3).

    Product rule on the tanh form of [CAC] "Feed-forward stage":
    0.5 (1 + tanh u) + 0.5 z (1 - tanh^2 u) du/dz, du/dz = sqrt(2/pi) (1 + 3 * 0.044715 z^2).
    """
    z = _f64(z)
    t = np.tanh(_GELU_C * (z + _GELU_A * z ** 3))
    du = _GELU_C * (1.0 + 3.0 * _GELU_A * z * z)
    return 0.5 * (1.0 + t) + 0.5 * z * (1.0 - t * t) * du


def softmax_backward(p, g) -> np.ndarray:
    """dL/ds of p = softmax(s) over the last axis, given p and g = dL/dp.

    The Jacobian of a softmax row is diag(p) - p p^T, so
    dL/ds_j = p_j (g_j - sum_k p_k g_k).
    """
    p = _f64(p)
    g = _f64(g)
    return p * (g - (p * g).sum(axis=-1, keepdims=True))


def attention_backward(qh, kh, vh, p, d_o):
    """Gradients of O = softmax(Q K^T / sqrt(d_h)) V for every sequence and head.

    Inputs are (N, H, T, d_h) per head (p: the weights, (N, H, T, T); d_o:
    dL/dO).  Reverse of [CAC] "Multi-head attention": O = P V gives
    dV = P^T dO and dP = dO V^T; P = softmax(S) gives dS (softmax_backward);
    S = Q K^T / sqrt(d_h) gives dQ = dS K / sqrt(d_h) and dK = dS^T Q / sqrt(d_h).
    Returns (dq, dk, dv), each (N, H, T, d_h).
    """
    qh, kh, vh, p, d_o = (_f64(a) for a in (qh, kh, vh, p, d_o))
    scale = 1.0 / math.sqrt(qh.shape[-1])
    dv = np.matmul(np.swapaxes(p, -1, -2), d_o)
    dp = np.matmul(d_o, np.swapaxes(vh, -1, -2))
    ds = softmax_backward(p, dp)
    dq = np.matmul(ds, kh) * scale
    dk = np.matmul(np.swapaxes(ds, -1, -2), qh) * scale
    return dq, dk, dv


def _wgrad(a, g) -> np.ndarray:
    """sum over every token of a^T g for (..., I) and (..., J) activations: (I, J)."""
    a = _f64(a)
    g = _f64(g)
    return np.matmul(a.reshape(-1, a.shape[-1]).T, g.reshape(-1, g.shape[-1]))


def vit_block_backward_stages(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, dout, num_heads: int,
                              eps: float) -> dict:
    """Every gradient of the block for a batch of sequences, float64.

    Forward (oracle.block.vit_block_stages): xn = LN(x); q, k, v = xn @ w_*;
    att = heads of softmax(q k^T / sqrt(d_h)) v; y = x + att @ w_o; yn = LN(y);
    z = yn @ w_mlp1; h = GELU(z); out = y + h @ w_mlp2.

    Returned keys: the gradients of GRAD_KEYS and, for the pins, the
    intermediate gradients dh, dz, dyn, dy, datt, dq, dk, dv, dxn (each
    dL/d of the forward tensor of that name).
    """
    w_q, w_k, w_v, w_o, w_mlp1, w_mlp2 = (_f64(w) for w in (w_q, w_k, w_v, w_o, w_mlp1, w_mlp2))
    st = ob.vit_block_stages(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, num_heads, eps)
    g = _f64(dout)
    if g.shape != st["out"].shape:
        raise ValueError("dout must have the shape of the block output")
    r = {}
    # out = y + h @ w_mlp2
    r["dw_mlp2"] = _wgrad(st["h"], g)
    r["dh"] = np.matmul(g, w_mlp2.T)
    # h = GELU(z)
    r["dz"] = r["dh"] * gelu_tanh_grad(st["z"])
    # z = yn @ w_mlp1
    r["dw_mlp1"] = _wgrad(st["yn"], r["dz"])
    r["dyn"] = np.matmul(r["dz"], w_mlp1.T)
    # yn = LN(y); y also reaches out through the residual.
    r["dy"] = g + layer_norm_backward(st["y"], r["dyn"], eps)
    # y = x + att @ w_o
    r["dw_o"] = _wgrad(st["att"], r["dy"])
    r["datt"] = np.matmul(r["dy"], w_o.T)
    # att = concatenated heads of softmax(q k^T / sqrt(d_h)) v
    dqh, dkh, dvh = attention_backward(
        ob.split_heads(st["q"], num_heads), ob.split_heads(st["k"], num_heads),
        ob.split_heads(st["v"], num_heads), st["weights"],
        ob.split_heads(r["datt"], num_heads))
    r["dq"], r["dk"], r["dv"] = ob.merge_heads(dqh), ob.merge_heads(dkh), ob.merge_heads(dvh)
    # q, k, v = xn @ w_q, xn @ w_k, xn @ w_v
    r["dw_q"] = _wgrad(st["xn"], r["dq"])
    r["dw_k"] = _wgrad(st["xn"], r["dk"])
    r["dw_v"] = _wgrad(st["xn"], r["dv"])
    r["dxn"] = (np.matmul(r["dq"], w_q.T) + np.matmul(r["dk"], w_k.T)
                + np.matmul(r["dv"], w_v.T))
    # xn = LN(x); x also reaches y through the residual.
    r["dx"] = r["dy"] + layer_norm_backward(x, r["dxn"], eps)
    return r


def vit_block_backward(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, dout, num_heads: int,
                       eps: float, chunk: int = 8) -> dict:
    """dL/dx (N, T, D) and dL/dW for the six weights, given dL/d(out); float64.

    ``chunk`` sequences at a time ([CAC] "Inputs and output": the N sequences
    are independent); dx is per sequence, each weight gradient is the sum of
    the chunks' sums over their tokens.  Returns a dict keyed by GRAD_KEYS.
    """
    x = _f64(x)
    dout = _f64(dout)
    if x.ndim != 3 or dout.shape != x.shape:
        raise ValueError("x and dout must both be (N, T, D)")
    out = {"dx": np.empty_like(x)}
    step = max(1, int(chunk))
    for s in range(0, x.shape[0], step):
        r = vit_block_backward_stages(x[s:s + step], w_q, w_k, w_v, w_o, w_mlp1, w_mlp2,
                                      dout[s:s + step], num_heads, eps)
        out["dx"][s:s + step] = r["dx"]
        for k in GRAD_KEYS[1:]:
            out[k] = r[k] if k not in out else out[k] + r[k]
    return out
