"""GPU parity of the block backward and its steps against the float64 oracle.

The backward is the exact derivative of the forward definition
(crackedaicode.com "ViT Encoder Block"), the gradients training needs
(nipunbatra.github.io vision1 transcript, Pages 88 and 113).  Inputs: the
forward's seeded inputs plus a seeded N(0, 1) output gradient
(vision_transformer_encoder_amd.inputs.make_dout).  Bars, per gradient
tensor (gpu_util.assert_close_grad): normwise ||g - o|| / ||o|| <= 1e-5
(fp32) or 1e-2 (bf16), and elementwise |g - o| <= tol * (rms(o) + |o|),
tol = 2e-4 (fp32) or 5e-2 (bf16) -- the tensor's RMS stands in for the
forward bar's unit scale, and the bf16 tol is the expected largest of the
measured per-element errors over the largest weight gradients.

At full size the oracle cannot afford every sequence, so the output gradient
is zero except on a few sampled sequences: the gradients are linear in it and
sequences never interact, so dx of every other sequence is exactly zero and
the weight gradients are exactly the sampled sequences' sums -- the oracle
computes those on the sampled sequences alone, while the GPU runs the full
batch in the launch configuration the benchmark times.
"""

import math

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import (WORKLOADS, make_block_inputs, make_dout,
                                                   round_to)

from gpu_util import assert_close_grad, to_dev, to_host

pytestmark = pytest.mark.gpu

WEIGHTS = ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]


def _rand(rng, shape, dtype, scale=1.0, offset=0.0):
    return round_to(rng.standard_normal(shape) * scale + offset, dtype)


def _gpu_backward(inp, dout, H, eps, dtype):
    g = vb.backward(to_dev(inp["x"], dtype), *(to_dev(inp[k], dtype) for k in WEIGHTS),
                    to_dev(dout, dtype), H, eps)
    return {k: to_host(v) for k, v in g.items()}


BLOCKS = [
    # (N, T, D, H, F, eps, dtype)
    (4, 5, 16, 2, 32, 1e-5, "fp32"),      # the tiny workload
    (2, 50, 192, 3, 320, 1e-6, "fp32"),
    (3, 37, 128, 2, 256, 1e-6, "bf16"),   # MFMA GEMMs, ragged token count
    (2, 197, 256, 4, 1024, 1e-6, "bf16"),  # ViT token count
    (2, 9, 24, 3, 40, 1e-6, "bf16"),      # generic GEMMs (widths not multiples of 64)
    (3, 257, 160, 2, 640, 1e-6, "bf16"),  # head width 80 (ViT-H/14), T = 257
]


@pytest.mark.parametrize("N,T,D,H,F,eps,dtype", BLOCKS)
def test_block_backward(N, T, D, H, F, eps, dtype):
    print(f"backward N={N} T={T} D={D} H={H} F={F} {dtype}", flush=True)
    inp = make_block_inputs(N, T, D, F, dtype, seed=1)
    dout = make_dout(N, T, D, dtype, seed=1)
    got = _gpu_backward(inp, dout, H, eps, dtype)
    ref = oracle.vit_block_backward(inp["x"], *(inp[k] for k in WEIGHTS), dout, H, eps)
    for k in oracle.GRAD_KEYS:
        assert_close_grad(got[k], ref[k], dtype, f"{k} N={N} T={T} D={D}")


def test_single_token_gives_exactly_zero_query_and_key_gradients():
    inp = make_block_inputs(3, 1, 64, 128, "bf16", seed=2)
    dout = make_dout(3, 1, 64, "bf16", seed=2)
    got = _gpu_backward(inp, dout, 2, 1e-6, "bf16")
    assert np.all(got["dw_q"] == 0.0) and np.all(got["dw_k"] == 0.0)
    ref = oracle.vit_block_backward(inp["x"], *(inp[k] for k in WEIGHTS), dout, 2, 1e-6)
    for k in ("dx", "dw_v", "dw_o", "dw_mlp1", "dw_mlp2"):
        assert_close_grad(got[k], ref[k], "bf16", f"{k} T=1")


def test_backward_is_deterministic_and_leaves_inputs_unchanged():
    import torch
    inp = make_block_inputs(2, 197, 256, 1024, "bf16", seed=3)
    dout = make_dout(2, 197, 256, "bf16", seed=3)
    dev = {k: to_dev(v, "bf16") for k, v in inp.items()}
    d = to_dev(dout, "bf16")
    before = {k: v.clone() for k, v in dev.items()}
    g1 = vb.backward(dev["x"], *(dev[k] for k in WEIGHTS), d, 4, 1e-6)
    g2 = vb.backward(dev["x"], *(dev[k] for k in WEIGHTS), d, 4, 1e-6)
    torch.cuda.synchronize()
    for k in vb.GRAD_KEYS:
        assert torch.equal(g1[k], g2[k]), k
    for k in dev:
        assert torch.equal(dev[k], before[k]), k


@pytest.mark.parametrize("name,sampled", [("vit_b16", (0, 63)), ("vit_l16", (5, 200))])
def test_full_size_sampled_sequences(name, sampled):
    w = WORKLOADS[name]
    print(f"backward full size {name} sampled {sampled}", flush=True)
    inp = make_block_inputs(w.N, w.T, w.D, w.F, w.dtype, seed=0)
    dout = make_dout(w.N, w.T, w.D, w.dtype, seed=0)
    mask = np.zeros(w.N, dtype=bool)
    mask[list(sampled)] = True
    dout[~mask] = 0.0
    got = _gpu_backward(inp, dout, w.H, w.eps, w.dtype)
    assert np.all(got["dx"][~mask] == 0.0)
    idx = list(sampled)
    ref = oracle.vit_block_backward(inp["x"][idx], *(inp[k] for k in WEIGHTS), dout[idx], w.H,
                                    w.eps, chunk=1)
    assert_close_grad(got["dx"][idx], ref["dx"], w.dtype, f"dx {name}")
    for k in oracle.GRAD_KEYS[1:]:
        assert_close_grad(got[k], ref[k], w.dtype, f"{k} {name}")


# ------------------------------------------------------------------ steps

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,I,J", [(300, 256, 512), (37, 24, 40), (5000, 64, 96),
                                   (12608, 768, 768), (1000, 1024, 3072)])
def test_weight_grad(dtype, M, I, J):
    rng = np.random.default_rng(M + I + J)
    a = _rand(rng, (M, I), dtype)
    b = _rand(rng, (M, J), dtype)
    got = to_host(vb.weight_grad(to_dev(a, dtype), to_dev(b, dtype)))
    assert_close_grad(got, a.T @ b, dtype, f"weight grad M={M} I={I} J={J}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,D,res", [(37, 768, True), (3, 20, False), (64, 1024, True),
                                        (5, 1280, False)])
def test_layernorm_backward(dtype, rows, D, res):
    rng = np.random.default_rng(rows + D)
    x = _rand(rng, (rows, D), dtype, scale=3.0, offset=1.0)
    x[0] = round_to(np.full(D, 0.5), dtype)  # constant row: variance 0
    g = _rand(rng, (rows, D), dtype)
    r = _rand(rng, (rows, D), dtype) if res else None
    got = to_host(vb.layernorm_backward(to_dev(x, dtype), to_dev(g, dtype), 1e-5,
                                        residual=None if r is None else to_dev(r, dtype)))
    ref = oracle.layer_norm_backward(x, g, 1e-5) + (0.0 if r is None else r)
    assert_close_grad(got, ref, dtype, f"LN backward rows={rows} D={D}")


@pytest.mark.parametrize("N,T,D,H,dtype", [(2, 5, 16, 2, "fp32"), (2, 197, 256, 4, "bf16"),
                                           (3, 50, 192, 3, "bf16"), (1, 1, 64, 1, "bf16"),
                                           (2, 257, 160, 2, "bf16"), (2, 33, 24, 4, "fp32")])
def test_attention_backward(N, T, D, H, dtype):
    rng = np.random.default_rng(N * T + D)
    qkv = _rand(rng, (N * T, 3 * D), dtype)
    datt = _rand(rng, (N * T, D), dtype)
    got = to_host(vb.attention_backward(to_dev(qkv, dtype), to_dev(datt, dtype), N, T, H))
    heads = lambda t: oracle.split_heads(t.reshape(N, T, D), H)  # noqa: E731
    qh, kh, vh = (heads(qkv[:, i * D:(i + 1) * D]) for i in range(3))
    p = oracle.softmax_rows(oracle.attention_scores(qh, kh))
    dq, dk, dv = oracle.attention_backward(qh, kh, vh, p, heads(datt))
    for i, (name, ref) in enumerate((("dq", dq), ("dk", dk), ("dv", dv))):
        assert_close_grad(got[:, i * D:(i + 1) * D], oracle.merge_heads(ref).reshape(N * T, D),
                          dtype, f"attention backward {name} N={N} T={T} D={D} H={H}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,K,N", [(300, 256, 512), (33, 40, 24), (600, 1024, 4096)])
def test_linear_gelu_grad_epilogue(dtype, M, K, N):
    rng = np.random.default_rng(M * K + N)
    a = _rand(rng, (M, K), dtype)
    w = _rand(rng, (K, N), dtype, scale=1 / math.sqrt(K))
    z = _rand(rng, (M, N), dtype, scale=2.0)
    got = to_host(vb.linear(to_dev(a, dtype), to_dev(np.ascontiguousarray(w.T), dtype),
                            epilogue=vb.EPI_GELU_GRAD, residual=to_dev(z, dtype)))
    ref = (a @ w) * oracle.gelu_tanh_grad(z)
    assert_close_grad(got, ref, dtype, f"linear GELU' M={M} K={K} N={N}")
