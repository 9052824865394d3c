"""Float64 CPU oracle for the forward pass of one pre-LayerNorm ViT encoder block.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
constant or helper with the HIP library in ``vision_transformer_encoder_amd``;
the only thing both sides consume is the seeded input arrays.

It is the plain definition of the block, written out step by step in float64
NumPy, vectorised over sequences and heads (no blocking, fusion or reordering
beyond what the definition states).  Matrix products use ``numpy.matmul``.

Sources (the pages this follows; each function names the section it restates):

  [CAC]  crackedaicode.com, "ViT Encoder Block" (PyTorch track) -- sections
         "Inputs and output", "Normalize before each stage",
         "Multi-head attention", "Feed-forward stage".
  [TT]   tensortonic.com, "ViT Encoder Block" -- the block equations,
         "Requirements" (population variance, eps 1e-6), "Examples".
  [AEE]  ai-engineer-exhaustive.pages.dev, "ViT Encoder Block" --
         "Key Equations" steps 1-6, "Numerical Example".
  [MLG]  mlgrind.dev, "E2E: Tiny Vision Transformer" -- "Details" (MHA, GELU),
         "Architecture" (final LayerNorm of the class token).
  [NB]   nipunbatra.github.io, vision1 lecture transcript -- Page 70
         (head h owns features h*d_h .. (h+1)*d_h-1), Pages 106-110 (code),
         Pages 24-26 and 36 (a linear layer is a weighted sum plus a bias).

Readings taken where the pages differ (all fixed by the block definition in
[CAC]): no LayerNorm scale/shift, no projection biases, tanh-GELU, and a
caller-supplied eps (1e-5 in [CAC], 1e-6 in [TT]).

The affine variant (``params`` of ``vit_block``) is the block of [AEE]
"Key Equations": each LayerNorm with its own per-feature gain gamma and
shift beta (steps 1 and 4; [MLG] "Details": learnable gain and bias), the MLP
with biases b_1, b_2 (step 5), and -- reading the projections as the linear
layers of [NB] Pages 24-26 -- optional biases on Q, K, V and the output
projection too.  Every parameter is optional; an absent one is gamma = 1,
beta = 0 or bias = 0, which is the plain block above ([MLG] "Details" has no
MHA bias and initialises gains to 1 and biases to 0).

Every function here has pins in ``tests/test_oracle.py`` that do not reuse
this code: the printed worked examples of [TT] "Examples" and the hand trace
of [AEE] "Numerical Example", closed forms, invariants and a brute-force
scalar loop.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "layer_norm",
    "layer_norm_stats",
    "project",
    "split_heads",
    "merge_heads",
    "attention_scores",
    "softmax_rows",
    "attention_weights",
    "multi_head_attention",
    "gelu_tanh",
    "vit_block",
    "vit_block_stages",
    "affine",
    "add_bias",
    "AFFINE_KEYS",
    "encoder",
]

# Optional parameters of the affine variant, in the order of the block.
AFFINE_KEYS = ("ln1_gamma", "ln1_beta", "b_q", "b_k", "b_v", "b_o",
               "ln2_gamma", "ln2_beta", "b_mlp1", "b_mlp2")


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def layer_norm(x, eps: float) -> np.ndarray:
    """Normalise every token over its last (feature) axis.

    [CAC] "Normalize before each stage": subtract the token mean and divide by
    sqrt(population variance + eps), the variance dividing by D (not D-1);
    there is no learned scale or shift.  [AEE] "Key Equations" step 1 gives the
    same mean/variance with gamma = 1, beta = 0.
    """
    x = _f64(x)
    mean = x.mean(axis=-1, keepdims=True)
    dev = x - mean
    var = (dev * dev).mean(axis=-1, keepdims=True)
    return dev / np.sqrt(var + eps)


def layer_norm_stats(x, eps: float):
    """Each token's mean and 1 / sqrt(population variance + eps), over its last axis.

    The two numbers [CAC] "Normalize before each stage" normalises a token
    with: layer_norm(x) = (x - mean) * rstd.  [AEE] "Numerical Example" prints
    the mean and the variance of its token.  Returns (mean, rstd), each of
    shape x.shape[:-1].
    """
    x = _f64(x)
    mean = x.mean(axis=-1)
    dev = x - mean[..., None]
    var = (dev * dev).mean(axis=-1)
    return mean, 1.0 / np.sqrt(var + eps)


def affine(t, gamma=None, beta=None) -> np.ndarray:
    """Per-feature gain and shift of a normalised tensor: gamma_j * t_ij + beta_j.

    [AEE] "Key Equations" step 1 (x_hat_ij = gamma_j (x_ij - mu_i) /
    sqrt(sigma_i^2 + eps) + beta_j) and step 4 (the second LayerNorm has its own
    gamma and beta).  Absent gamma is 1, absent beta is 0.
    """
    t = _f64(t)
    if gamma is not None:
        t = t * _f64(gamma)
    if beta is not None:
        t = t + _f64(beta)
    return t


def add_bias(t, b=None) -> np.ndarray:
    """A projection's bias, one value per output feature: t_ij + b_j.

    [AEE] "Key Equations" step 5 (x_hat' W_1 + b_1, then W_2 + b_2);
    [NB] Pages 24-26 (each output of a linear layer adds its bias).
    """
    t = _f64(t)
    return t if b is None else t + _f64(b)


def project(a, w) -> np.ndarray:
    """Row-vector projection ``a @ w`` with ``w`` stored (in_features, out_features).

    [CAC] "Multi-head attention": Q = LN(x) @ w_q with w_q of shape (D, D);
    "Inputs and output": w_mlp1 is (D, F) and w_mlp2 is (F, D).
    """
    return np.matmul(_f64(a), _f64(w))


def split_heads(t, num_heads: int) -> np.ndarray:
    """(N, T, D) -> (N, H, T, D/H): head h takes the h-th run of D/H consecutive features.

    [CAC] "Multi-head attention" (split into H consecutive chunks of width D/H);
    [NB] Page 70 (the first 64 features belong to head 1).
    """
    t = _f64(t)
    n, tt, d = t.shape
    dh = d // num_heads
    return t.reshape(n, tt, num_heads, dh).transpose(0, 2, 1, 3)


def merge_heads(o) -> np.ndarray:
    """(N, H, T, d_h) -> (N, T, H*d_h), heads concatenated in their original order.

    [CAC] "Multi-head attention" (concatenate head outputs in original order).
    """
    o = _f64(o)
    n, h, tt, dh = o.shape
    return o.transpose(0, 2, 1, 3).reshape(n, tt, h * dh)


def attention_scores(qh, kh) -> np.ndarray:
    """Q_h K_h^T / sqrt(d_h) for every sequence and head: (N, H, T, T).

    [CAC] "Multi-head attention" (scores scaled by 1/sqrt(D/H));
    [AEE] "Key Equations" step 2 (divide by sqrt(d_k)).
    """
    qh = _f64(qh)
    kh = _f64(kh)
    dh = qh.shape[-1]
    return np.matmul(qh, np.swapaxes(kh, -1, -2)) / math.sqrt(dh)


def softmax_rows(s) -> np.ndarray:
    """Stable softmax over the last (key) axis; no mask of any kind.

    [CAC] "Multi-head attention" (stable softmax across key positions, every
    token sees every token of its sequence); [AEE] "No Causal Mask".
    The row maximum is subtracted before exponentiating.
    """
    s = _f64(s)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_weights(xn, w_q, w_k, num_heads: int) -> np.ndarray:
    """softmax(Q_h K_h^T / sqrt(d_h)) for every sequence and head: (N, H, T, T)."""
    qh = split_heads(project(xn, w_q), num_heads)
    kh = split_heads(project(xn, w_k), num_heads)
    return softmax_rows(attention_scores(qh, kh))


def multi_head_attention(xn, w_q, w_k, w_v, num_heads: int) -> np.ndarray:
    """Concatenated head outputs before the output projection: (N, T, D).

    [CAC] "Multi-head attention": per sequence and head,
    head_output = softmax(Q_h K_h^T / sqrt(D/H)) @ V_h; heads concatenated.
    """
    a = attention_weights(xn, w_q, w_k, num_heads)
    vh = split_heads(project(xn, w_v), num_heads)
    return merge_heads(np.matmul(a, vh))


def gelu_tanh(z) -> np.ndarray:
    """GELU, tanh form: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).

    [CAC] "Feed-forward stage"; [MLG] "Details"; [AEE] "Key Equations" step 5.
    sqrt(2/pi) is evaluated, not the rounded 0.7979 of [AEE]'s hand trace.
    """
    z = _f64(z)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z ** 3)))


def _params(params) -> dict:
    p = dict(params or {})
    unknown = set(p) - set(AFFINE_KEYS)
    if unknown:
        raise ValueError(f"unknown block parameters: {sorted(unknown)}")
    return {k: p.get(k) for k in AFFINE_KEYS}


def vit_block_stages(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, num_heads: int,
                     eps: float, params=None) -> dict:
    """Every intermediate of the block for a batch of sequences, float64.

    Keys: xn = LN(x); q, k, v = xn @ w_{q,k,v}; att = concatenated heads;
    y = x + att @ w_o; yn = LN(y); z = yn @ w_mlp1; h = GELU(z);
    out = y + h @ w_mlp2.

    [CAC] "Multi-head attention" and "Feed-forward stage": the first residual
    adds the un-normalised x, the second LayerNorm normalises y (not x).
    [AEE] "Key Equations" steps 1-6 give the same order.

    ``params`` (optional; keys in ``AFFINE_KEYS``) adds the affine variant:
    xn = gamma_1 LN(x) + beta_1, q = xn @ w_q + b_q (and k, v), y = x + att @ w_o
    + b_o, yn = gamma_2 LN(y) + beta_2, z = yn @ w_mlp1 + b_mlp1,
    out = y + GELU(z) @ w_mlp2 + b_mlp2 ([AEE] "Key Equations" steps 1-6).
    """
    x = _f64(x)
    if x.ndim != 3:
        raise ValueError("x must be (N, T, D)")
    d = x.shape[-1]
    if num_heads <= 0 or d % num_heads:
        raise ValueError("num_heads must be positive and divide D")
    p = _params(params)
    xn = affine(layer_norm(x, eps), p["ln1_gamma"], p["ln1_beta"])
    q = add_bias(project(xn, w_q), p["b_q"])
    k = add_bias(project(xn, w_k), p["b_k"])
    v = add_bias(project(xn, w_v), p["b_v"])
    a = softmax_rows(attention_scores(split_heads(q, num_heads), split_heads(k, num_heads)))
    att = merge_heads(np.matmul(a, split_heads(v, num_heads)))
    y = x + add_bias(project(att, w_o), p["b_o"])
    yn = affine(layer_norm(y, eps), p["ln2_gamma"], p["ln2_beta"])
    z = add_bias(project(yn, w_mlp1), p["b_mlp1"])
    h = gelu_tanh(z)
    out = y + add_bias(project(h, w_mlp2), p["b_mlp2"])
    return dict(xn=xn, q=q, k=k, v=v, weights=a, att=att, y=y, yn=yn, z=z, h=h, out=out)


def vit_block(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, num_heads: int, eps: float,
              chunk: int = 8, params=None) -> np.ndarray:
    """Output of one pre-LN encoder block, (N, T, D) float64.

    Sequences never interact ([CAC] "Inputs and output": N independent
    sequences), so they are processed ``chunk`` at a time to bound memory;
    this changes no arithmetic.  ``params``: the affine variant's optional
    gains, shifts and biases (see ``vit_block_stages``).
    """
    x = _f64(x)
    out = np.empty_like(x)
    for s in range(0, x.shape[0], max(1, int(chunk))):
        st = vit_block_stages(x[s:s + chunk], w_q, w_k, w_v, w_o, w_mlp1, w_mlp2,
                              num_heads, eps, params=params)
        out[s:s + chunk] = st["out"]
    return out


def encoder(x, layers, num_heads: int, eps: float, final_gamma=None, final_beta=None,
            chunk: int = 8):
    """L encoder blocks in sequence, then the final LayerNorm; (tokens, cls).

    [AEE] "What It Is": the encoder stacks L identical blocks, each with its
    own weights (L = 12, 24, 32 for ViT-B/L/H, "Paper Context").  [MLG]
    "Architecture": after the last block, cls = LN_f(t[:, 0]), a LayerNorm
    with its own gain and shift.  ``layers`` is a sequence of dicts holding
    w_q, w_k, w_v, w_o, w_mlp1, w_mlp2 and, optionally, ``params`` (the affine
    variant's parameters of that block).  Returns tokens = LN_f(t) for every
    token, (N, T, D), and cls = LN_f(t[:, 0]), (N, D).
    """
    t = _f64(x)
    for layer in layers:
        t = vit_block(t, layer["w_q"], layer["w_k"], layer["w_v"], layer["w_o"],
                      layer["w_mlp1"], layer["w_mlp2"], num_heads, eps, chunk=chunk,
                      params=layer.get("params"))
    tokens = affine(layer_norm(t, eps), final_gamma, final_beta)
    return tokens, tokens[:, 0, :]
