"""GPU parity of the encoder stack: L blocks, final LayerNorm, class-token readout.

ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "What It Is" (L blocks,
each with its own weights); mlgrind.dev "E2E: Tiny Vision Transformer",
"Architecture" (cls = LN_f(t[:, 0])).  Bars: the one-block bar times sqrt(L)
(gpu_util.stack_scale): every block rounds its activations independently, so
the errors add in quadrature along the residual stream (measured on the GPU:
violation / sqrt(L) stays at 0.007-0.010 from L = 1 to 32 in bf16).
"""

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import (WORKLOADS, make_affine_params,
                                                   make_block_inputs, round_to)

from gpu_util import assert_close, stack_scale, to_dev, to_host

pytestmark = pytest.mark.gpu

WEIGHTS = ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]


def _layers(N, T, D, F, L, dtype, affine, seed=0):
    """x plus L blocks' weights (each block seeded on its own)."""
    x = make_block_inputs(N, T, D, F, dtype, seed=seed)["x"]
    layers = []
    for l in range(L):
        inp = make_block_inputs(1, 1, D, F, dtype, seed=seed * 1000 + l + 1)
        lay = {k: inp[k] for k in WEIGHTS}
        if affine:
            lay["params"] = make_affine_params(D, F, dtype, seed=seed * 1000 + l + 1)
        layers.append(lay)
    return x, layers


def _final(D, dtype, seed=0):
    rng = np.random.default_rng([seed, 2])
    return (round_to(1.0 + 0.1 * rng.standard_normal(D), dtype),
            round_to(0.1 * rng.standard_normal(D), dtype))


def _run(x, layers, H, eps, dtype, fg, fb, want_tokens=True, want_cls=True):
    dev_x = to_dev(x, dtype)
    packed = [vb.pack_weights(*(to_dev(lay[k], dtype) for k in WEIGHTS)) for lay in layers]
    prm = None
    if "params" in layers[0]:
        prm = [{k: to_dev(v, dtype) for k, v in lay["params"].items()} for lay in layers]
    F = layers[0]["w_mlp1"].shape[1]
    return vb.encoder_forward(dev_x, packed, F, H, eps, params=prm,
                              final_gamma=None if fg is None else to_dev(fg, dtype),
                              final_beta=None if fb is None else to_dev(fb, dtype),
                              want_tokens=want_tokens, want_cls=want_cls)


ENCODERS = [
    # (N, T, D, H, F, L, eps, dtype, affine)
    (2, 5, 16, 2, 32, 3, 1e-5, "fp32", False),
    (2, 5, 16, 2, 32, 2, 1e-5, "fp32", True),
    (2, 197, 256, 4, 1024, 4, 1e-6, "bf16", False),
    (2, 197, 256, 4, 1024, 3, 1e-6, "bf16", True),
    (2, 9, 24, 3, 40, 2, 1e-6, "bf16", True),   # generic kernels
]


@pytest.mark.parametrize("N,T,D,H,F,L,eps,dtype,affine", ENCODERS)
def test_encoder_small(N, T, D, H, F, L, eps, dtype, affine):
    x, layers = _layers(N, T, D, F, L, dtype, affine)
    fg, fb = _final(D, dtype)
    tok, cls = _run(x, layers, H, eps, dtype, fg, fb)
    ref_tok, ref_cls = oracle.encoder(x, layers, H, eps, fg, fb)
    assert_close(to_host(tok), ref_tok, dtype, f"encoder tokens L={L} D={D}",
                 scale=stack_scale(L))
    assert_close(to_host(cls), ref_cls, dtype, f"encoder cls L={L} D={D}", scale=stack_scale(L))
    # Class tokens only: the last block computes just their rows.
    _, cls_only = _run(x, layers, H, eps, dtype, fg, fb, want_tokens=False)
    assert_close(to_host(cls_only), ref_cls, dtype, f"encoder cls only L={L} D={D}",
                 scale=stack_scale(L))


def test_encoder_outputs_are_independent_of_each_other():
    import torch
    x, layers = _layers(2, 65, 128, 512, 2, "bf16", True, seed=3)
    fg, fb = _final(128, "bf16", seed=3)
    tok, cls = _run(x, layers, 2, 1e-6, "bf16", fg, fb)
    tok_only, none = _run(x, layers, 2, 1e-6, "bf16", fg, fb, want_cls=False)
    none2, cls_only = _run(x, layers, 2, 1e-6, "bf16", fg, fb, want_tokens=False)
    assert none is None and none2 is None
    assert torch.equal(tok, tok_only)
    assert torch.equal(cls, tok[:, 0])
    # Without the token output the last block computes only the class-token
    # rows, in smaller products whose K sums may run in the other order: the
    # same values to within the stack's bar rather than the same bits.
    _, ref_cls = oracle.encoder(x, layers, 2, 1e-6, fg, fb)
    assert_close(to_host(cls_only), ref_cls, "bf16", "encoder cls only", scale=stack_scale(2))


def test_encoder_of_one_block_is_the_block_then_the_final_layer_norm():
    import torch
    x, layers = _layers(2, 197, 256, 1024, 1, "bf16", False, seed=4)
    tok, _ = _run(x, layers, 4, 1e-6, "bf16", None, None, want_cls=False)
    dev = {k: to_dev(v, "bf16") for k, v in layers[0].items()}
    blk = vb.forward(to_dev(x, "bf16"), *(dev[k] for k in WEIGHTS), 4, 1e-6)
    assert torch.equal(tok, vb.layernorm(blk, 1e-6))


def test_encoder_vit_b16_depth12():
    w = WORKLOADS["vit_b16"]
    L = 12
    x, layers = _layers(w.N, w.T, w.D, w.F, L, w.dtype, True, seed=5)
    fg, fb = _final(w.D, w.dtype, seed=5)
    tok, cls = _run(x, layers, w.H, w.eps, w.dtype, fg, fb)
    seqs = [0, w.N - 1]
    ref_tok, ref_cls = oracle.encoder(x[seqs], layers, w.H, w.eps, fg, fb)
    got = to_host(tok)
    assert np.all(np.isfinite(got))
    assert_close(got[seqs], ref_tok, w.dtype, f"ViT-B/16 x{L} tokens, sequences {seqs}",
                 scale=stack_scale(L))
    assert_close(to_host(cls)[seqs], ref_cls, w.dtype, f"ViT-B/16 x{L} cls",
                 scale=stack_scale(L))


def test_encoder_class_tokens_only_vit_b16():
    # The class-token shortcut at ViT-B/16 shapes: first-query-tile attention
    # (T = 197, every key), the output projection and the MLP on N rows read
    # at row stride T * D.
    w = WORKLOADS["vit_b16"]
    L = 2
    x, layers = _layers(w.N, w.T, w.D, w.F, L, w.dtype, True, seed=6)
    fg, fb = _final(w.D, w.dtype, seed=6)
    _, cls_only = _run(x, layers, w.H, w.eps, w.dtype, fg, fb, want_tokens=False)
    got = to_host(cls_only)
    assert got.shape == (w.N, w.D) and np.all(np.isfinite(got))
    seqs = [0, w.N // 2, w.N - 1]
    _, ref_cls = oracle.encoder(x[seqs], layers, w.H, w.eps, fg, fb)
    assert_close(got[seqs], ref_cls, w.dtype, f"ViT-B/16 x{L} cls only, sequences {seqs}",
                 scale=stack_scale(L))


def test_encoder_each_block_at_the_one_block_bar_vit_b16_depth12():
    # Each block of a ViT-B/16 x 12 stack held to the one-block bar, given
    # its own GPU input: the stack's blocks are chained here through
    # vitblk_forward_packed_affine (the encoder's per-block launch sequence),
    # checked first to reproduce the stack's output bit for bit; then the
    # oracle runs block l on block l's GPU input, so no error carries over
    # from earlier blocks (ai-engineer-exhaustive.pages.dev "ViT Encoder
    # Block", "What It Is": L identical blocks in sequence).
    import torch
    w = WORKLOADS["vit_b16"]
    L = 12
    x, layers = _layers(w.N, w.T, w.D, w.F, L, w.dtype, True, seed=7)
    fg, fb = _final(w.D, w.dtype, seed=7)
    dev_x = to_dev(x, w.dtype)
    packed = [vb.pack_weights(*(to_dev(lay[k], w.dtype) for k in WEIGHTS)) for lay in layers]
    prm = [{k: to_dev(v, w.dtype) for k, v in lay["params"].items()} for lay in layers]
    tok, _ = vb.encoder_forward(dev_x, packed, w.F, w.H, w.eps, params=prm,
                                final_gamma=to_dev(fg, w.dtype),
                                final_beta=to_dev(fb, w.dtype), want_cls=False)
    chain = [dev_x]
    for l in range(L):
        chain.append(vb.forward_packed_affine(chain[-1], packed[l], w.F, w.H, w.eps,
                                              params=prm[l]))
    final = vb.layernorm(chain[-1].view(-1, w.D), w.eps, gamma=to_dev(fg, w.dtype),
                         beta=to_dev(fb, w.dtype)).view(tok.shape)
    assert torch.equal(final, tok)
    seqs = [0, w.N - 1]
    worst = 0.0
    for l in range(L):
        xin = to_host(chain[l])[seqs]
        ref = oracle.vit_block(xin, *(layers[l][k] for k in WEIGHTS), w.H, w.eps,
                               params=layers[l]["params"])
        v, _ = assert_close(to_host(chain[l + 1])[seqs], ref, w.dtype,
                            f"ViT-B/16 block {l} of {L}, sequences {seqs}")
        worst = max(worst, v)
    print(f"  worst block violation {worst:.3e} (one-block bar 3e-2)", flush=True)
