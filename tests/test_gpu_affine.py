"""GPU parity of the affine variant (LayerNorm gains and shifts, projection biases).

The block of ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "Key
Equations" steps 1-6, with the optional parameters of the oracle's ``params``;
same bars as the plain block (fp32 2e-4 (1 + |o|), bf16 3e-2 (1 + |o|)).
Parameters come from ``inputs.make_affine_params`` (gains 1 + 0.1 N(0, 1),
shifts and biases 0.1 N(0, 1), rounded to the device dtype).
"""

import math

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import (WORKLOADS, make_affine_params,
                                                   make_block_inputs, round_to)

from gpu_util import assert_close, to_dev, to_host, violation

pytestmark = pytest.mark.gpu

WEIGHTS = ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]


def _rand(rng, shape, dtype, scale=1.0, offset=0.0):
    return round_to(rng.standard_normal(shape) * scale + offset, dtype)


# ------------------------------------------------------------------ steps

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,D", [(37, 768), (64, 1024), (3, 20), (9, 16)])
@pytest.mark.parametrize("which", ["both", "gamma", "beta"])
def test_layernorm_affine(dtype, rows, D, which):
    rng = np.random.default_rng(rows * 31 + D)
    x = _rand(rng, (rows, D), dtype, scale=2.0, offset=0.5)
    g = _rand(rng, (D,), dtype, scale=0.3, offset=1.0) if which != "beta" else None
    b = _rand(rng, (D,), dtype, scale=0.5) if which != "gamma" else None
    got = to_host(vb.layernorm(to_dev(x, dtype), 1e-6,
                               gamma=None if g is None else to_dev(g, dtype),
                               beta=None if b is None else to_dev(b, dtype)))
    ref = oracle.affine(oracle.layer_norm(x, 1e-6), g, b)
    assert_close(got, ref, dtype, f"LN affine ({which}) rows={rows} D={D}")


EPIS = {"none": vb.EPI_NONE, "residual": vb.EPI_RESIDUAL, "gelu": vb.EPI_GELU}


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("epi", sorted(EPIS))
@pytest.mark.parametrize("M,K,N", [(300, 256, 512), (129, 1024, 200), (33, 40, 24),
                                   (70 * 256 + 77, 256, 1024)])
def test_linear_bias(dtype, epi, M, K, N):
    if dtype == "fp32" and M > 10000:
        pytest.skip("the big ragged case exercises the bf16 tile split only")
    rng = np.random.default_rng(M * 5 + K + N)
    a = _rand(rng, (M, K), dtype)
    w = _rand(rng, (K, N), dtype, scale=1 / math.sqrt(K))
    bias = _rand(rng, (N,), dtype, scale=0.5)
    r = _rand(rng, (M, N), dtype)
    res = to_dev(r, dtype) if epi == "residual" else None
    got = to_host(vb.linear(to_dev(a, dtype), to_dev(w.T, dtype), EPIS[epi], residual=res,
                            bias=to_dev(bias, dtype)))
    ref = oracle.add_bias(oracle.project(a, w), bias)
    if epi == "residual":
        ref = r + ref
    elif epi == "gelu":
        ref = oracle.gelu_tanh(ref)
    assert_close(got, ref, dtype, f"linear+bias {epi} M={M} K={K} N={N}")


# ------------------------------------------------------------------ the fold

@pytest.mark.parametrize("Nout,K", [(768, 256), (40, 16), (3072, 1024), (24, 2056)])
@pytest.mark.parametrize("which", ["all", "gamma", "beta", "bias", "none"])
def test_affine_fold_step(Nout, K, which):
    # w_scaled = bf16(gamma_k w[n, k]): the product of two bf16 values is
    # exact in fp32, so one rounding, bit for bit; the column sums are fp32
    # sums of those values; bias_out = bf16(b + beta @ W) within one bf16 ulp
    # (fp32 against float64 accumulation may land on either side of a tie).
    import torch
    rng = np.random.default_rng(Nout * 7 + K)
    w_t = _rand(rng, (Nout, K), "bf16", scale=1 / math.sqrt(K))
    g = _rand(rng, (K,), "bf16", scale=0.5, offset=1.0) if which in ("all", "gamma") else None
    be = _rand(rng, (K,), "bf16", scale=0.5) if which in ("all", "beta") else None
    b = _rand(rng, (Nout,), "bf16", scale=0.5) if which in ("all", "bias") else None
    dev = lambda a: None if a is None else to_dev(a, "bf16")  # noqa: E731
    ws, cs, bo = vb.affine_fold(dev(w_t), dev(g), dev(be), dev(b))
    torch.cuda.synchronize()
    ref_ws = round_to(w_t * (1.0 if g is None else g[None, :]), "bf16")
    assert np.array_equal(to_host(ws), ref_ws)
    got_cs = cs.cpu().double().numpy()
    assert np.all(np.abs(got_cs - ref_ws.sum(1)) <= 1e-6 * np.abs(ref_ws).sum(1) + 1e-30)
    ref_b = (0.0 if b is None else b) + (0.0 if be is None else w_t @ be)
    ref_b = np.broadcast_to(np.asarray(ref_b, dtype=np.float64), (Nout,))
    got_b = to_host(bo)
    assert np.all(np.abs(got_b - ref_b) <= 2.0 ** -7 * np.abs(ref_b) + 1e-30), \
        np.max(np.abs(got_b - ref_b))


@pytest.mark.parametrize("M,K,N,epi", [(300, 256, 512, "gelu"), (517, 1024, 768, "none"),
                                       (33, 64, 24, "none")])
def test_affine_fold_then_normed_product(M, K, N, epi):
    # The fold's operands in vitblk_linear_normed give (LN(a) gamma + beta) @ W
    # + b of the oracle's LayerNorm, gain and shift, and product.
    rng = np.random.default_rng(M + K + N)
    a = _rand(rng, (M, K), "bf16", scale=2.0, offset=0.5)
    w = _rand(rng, (K, N), "bf16", scale=1 / math.sqrt(K))
    g = _rand(rng, (K,), "bf16", scale=0.3, offset=1.0)
    be = _rand(rng, (K,), "bf16", scale=0.5)
    b = _rand(rng, (N,), "bf16", scale=0.5)
    da = to_dev(a, "bf16")
    ws, cs, bo = vb.affine_fold(to_dev(w.T, "bf16"), to_dev(g, "bf16"), to_dev(be, "bf16"),
                                to_dev(b, "bf16"))
    st = vb.row_stats(da, 1e-6)
    got = to_host(vb.linear_normed(da, ws, cs, st, EPIS[epi], bias=bo))
    ref = oracle.add_bias(oracle.project(oracle.affine(oracle.layer_norm(a, 1e-6), g, be), w), b)
    if epi == "gelu":
        ref = oracle.gelu_tanh(ref)
    assert_close(got, ref, "bf16", f"fold + normed product {epi} M={M} K={K} N={N}")


# ------------------------------------------------------------------ the block

def _run(inp, prm, H, eps, dtype, packed=False, drop=()):
    dev = {k: to_dev(v, dtype) for k, v in inp.items()}
    dprm = {k: to_dev(v, dtype) for k, v in prm.items() if k not in drop}
    if packed:
        pk = vb.pack_weights(*(dev[k] for k in WEIGHTS))
        out = vb.forward_packed_affine(dev["x"], pk, inp["w_mlp1"].shape[1], H, eps, params=dprm)
    else:
        out = vb.forward_affine(dev["x"], *(dev[k] for k in WEIGHTS), H, eps, params=dprm)
    return out, dev


def _oracle(inp, prm, H, eps, seqs=None, drop=()):
    x = inp["x"] if seqs is None else inp["x"][seqs]
    p = {k: v for k, v in prm.items() if k not in drop}
    return oracle.vit_block(x, *(inp[k] for k in WEIGHTS), H, eps, params=p)


AFFINE_BLOCKS = [
    # (N, T, D, H, F, eps, dtype)
    (4, 5, 16, 2, 32, 1e-5, "fp32"),       # the tiny workload
    (2, 50, 64, 4, 256, 1e-6, "fp32"),
    (3, 197, 256, 4, 1024, 1e-6, "bf16"),  # several tiles, ragged M tail
    (2, 257, 320, 4, 1280, 1e-6, "bf16"),  # d_h 80
    (2, 9, 24, 3, 40, 1e-6, "bf16"),       # shapes only the generic kernels take
]


@pytest.mark.parametrize("N,T,D,H,F,eps,dtype", AFFINE_BLOCKS)
def test_affine_block_small(N, T, D, H, F, eps, dtype):
    inp = make_block_inputs(N, T, D, F, dtype, seed=0)
    prm = make_affine_params(D, F, dtype, seed=0)
    out, _ = _run(inp, prm, H, eps, dtype)
    assert_close(to_host(out), _oracle(inp, prm, H, eps), dtype, f"affine block N={N} T={T} D={D}")


@pytest.mark.parametrize("name", ["vit_b16", "vit_l16"])
def test_affine_block_full_size(name):
    w = WORKLOADS[name]
    inp = make_block_inputs(w.N, w.T, w.D, w.F, w.dtype, seed=0)
    prm = make_affine_params(w.D, w.F, w.dtype, seed=0)
    out, _ = _run(inp, prm, w.H, w.eps, w.dtype)
    got = to_host(out)
    assert np.all(np.isfinite(got))
    seqs = sorted({0, w.N // 2, w.N - 1})
    assert_close(got[seqs], _oracle(inp, prm, w.H, w.eps, seqs), w.dtype,
                 f"affine {name} sequences {seqs}")


def test_affine_block_large_key_bias():
    # A consistency check, not a parity case: a large key bias adds q_i . b_k
    # to every score of query i, so some queries' scores all lie hundreds of
    # log2 units below 0 and others' far above (the output itself does not
    # depend on b_k).  Keys of size ~40 keep only bf16's precision of the
    # per-key differences, so the input is ill-conditioned for any bf16
    # implementation: the block must stay finite and as close to the oracle
    # as the same block composed from the step entries.  The attention step
    # is held to the oracle at such scores in test_gpu_attention_extreme.py.
    inp = make_block_inputs(2, 197, 256, 1024, "bf16", seed=14)
    prm = make_affine_params(256, 1024, "bf16", seed=14)
    prm["b_k"] = round_to(np.asarray(prm["b_k"]) * 400.0, "bf16")
    ref = _oracle(inp, prm, 4, 1e-6)
    # Per-query maximum score, in log2 units: both extremes occur.
    xn = oracle.affine(oracle.layer_norm(inp["x"], 1e-6), prm["ln1_gamma"], prm["ln1_beta"])
    q = oracle.add_bias(oracle.project(xn, inp["w_q"]), prm["b_q"])
    k = oracle.add_bias(oracle.project(xn, inp["w_k"]), prm["b_k"])
    qh, kh = oracle.split_heads(q, 4), oracle.split_heads(k, 4)
    smax = (qh @ np.swapaxes(kh, -1, -2)).max(-1) / 8.0 * math.log2(math.e)
    assert (smax < -96).any() and (smax > 96).any()

    out, dev = _run(inp, prm, 4, 1e-6, "bf16")
    got = to_host(out)
    assert np.all(np.isfinite(got))
    # The same block from the step entries.
    import torch
    dp = {k2: to_dev(v, "bf16") for k2, v in prm.items()}
    x2 = dev["x"].view(-1, 256)
    wt = {k2: dev[k2].t().contiguous() for k2 in WEIGHTS}
    xn_d = vb.layernorm(x2, 1e-6, gamma=dp["ln1_gamma"], beta=dp["ln1_beta"])
    wqkv = torch.cat([wt["w_q"], wt["w_k"], wt["w_v"]], 0)
    qkv = vb.linear(xn_d, wqkv, vb.EPI_NONE, bias=torch.cat([dp["b_q"], dp["b_k"], dp["b_v"]]))
    att = vb.attention(qkv, 2, 197, 4)
    y = vb.linear(att, wt["w_o"], vb.EPI_RESIDUAL, residual=x2, bias=dp["b_o"])
    yn = vb.layernorm(y, 1e-6, gamma=dp["ln2_gamma"], beta=dp["ln2_beta"])
    h = vb.linear(yn, wt["w_mlp1"], vb.EPI_GELU, bias=dp["b_mlp1"])
    steps = to_host(vb.linear(h, wt["w_mlp2"], vb.EPI_RESIDUAL, residual=y, bias=dp["b_mlp2"]))
    v_block, _ = violation(got, ref)
    v_steps, _ = violation(steps.reshape(got.shape), ref)
    assert v_block <= v_steps * 1.1 + 1e-3, (v_block, v_steps)


def test_affine_block_split_k_tail_rows():
    # As the plain block's split-K case: the MLP2 bias is added by the
    # reduction of the tail rows' K-range partials.
    N, T, D, H, F = 85, 197, 1024, 16, 4096
    inp = make_block_inputs(N, T, D, F, "bf16", seed=10)
    prm = make_affine_params(D, F, "bf16", seed=10)
    out, _ = _run(inp, prm, H, 1e-6, "bf16")
    seqs = [83, 84]
    assert_close(to_host(out)[seqs], _oracle(inp, prm, H, 1e-6, seqs), "bf16",
                 f"affine split-K tail {seqs}")


@pytest.mark.parametrize("drop", [("b_q", "b_v"), ("ln1_gamma", "ln2_beta", "b_mlp1"),
                                  ("b_k",), tuple(oracle.AFFINE_KEYS)])
def test_affine_block_with_some_parameters_absent(drop):
    # A null QKV bias segment is zero while its neighbours are not.
    inp = make_block_inputs(2, 197, 256, 1024, "bf16", seed=1)
    prm = make_affine_params(256, 1024, "bf16", seed=1)
    out, _ = _run(inp, prm, 4, 1e-6, "bf16", drop=drop)
    assert_close(to_host(out), _oracle(inp, prm, 4, 1e-6, drop=drop), "bf16",
                 f"affine block without {drop}")


# Sizes where both affine LayerNorms fold into the products after them (bf16):
# the gain-scaled weight copy of Q|K|V ([3D, D]) fits in the token-sized region
# y (M >= 3D) and that of MLP1 ([F, D]) beside the row statistics in another
# (8 M + 2 F D + 6 F bytes, each part rounded up to 256, <= 2 M D).  The
# smaller blocks above (M < 3D) write their LayerNorms out.
FOLDED = (4, 197, 128, 2, 512)


def _folds(N, T, D, F):
    M = N * T
    up = lambda v: (v + 255) // 256 * 256  # noqa: E731
    f1 = up(up(3 * D * D * 2) + 3 * D * 4) + 3 * D * 2
    f2 = up(up(up(8 * M) + F * D * 2) + F * 4) + F * 2
    return f1 <= M * D * 2 and f2 <= M * D * 2


@pytest.mark.parametrize("drop", [(), ("ln1_gamma",), ("ln1_beta",), ("ln2_gamma", "b_mlp1"),
                                  ("ln2_beta", "b_q", "b_v"), ("ln1_gamma", "ln2_gamma"),
                                  ("ln1_beta", "ln2_beta", "b_o")])
def test_affine_block_folded(drop):
    # The folded path: diag(gamma) W, its column sums and b + beta @ W, per
    # call, with either of gain and shift absent, and the output projection's
    # bias on the LN2 row-partials epilogue.
    N, T, D, H, F = FOLDED
    assert _folds(N, T, D, F)
    inp = make_block_inputs(N, T, D, F, "bf16", seed=21)
    prm = make_affine_params(D, F, "bf16", seed=21)
    out, _ = _run(inp, prm, H, 1e-6, "bf16", drop=drop)
    assert_close(to_host(out), _oracle(inp, prm, H, 1e-6, drop=drop), "bf16",
                 f"folded affine block without {drop}")


@pytest.mark.parametrize("N,T,D,H,F", [(2, 197, 72, 2, 288), (3, 97, 64, 4, 128)])
def test_affine_block_folded_other_kernels(N, T, D, H, F):
    # Folded with products outside the matrix-core kernel's shapes (K = 72:
    # the any-shape kernel, with the LN2 statistics from their own pass) and
    # with a narrow F (MLP1's copy beside the statistics of 291 rows).
    assert _folds(N, T, D, F)
    inp = make_block_inputs(N, T, D, F, "bf16", seed=23)
    prm = make_affine_params(D, F, "bf16", seed=23)
    out, _ = _run(inp, prm, H, 1e-6, "bf16")
    assert_close(to_host(out), _oracle(inp, prm, H, 1e-6), "bf16",
                 f"folded affine block N={N} T={T} D={D} F={F}")


def test_affine_block_folded_large_gains():
    # Gains far from 1 (N(0, 1): near 0 and of both signs) and unit shifts:
    # the scaled copy is rounded to bf16 once, as the written-out LayerNorm's
    # output is.  (Much larger gains scale the attention scores by gamma^2 and
    # leave any bf16 block outside the bar: at 3 N(0, 1) a CPU emulation of
    # the written-out path's roundings is off by 0.38, the fold's by 0.30.)
    N, T, D, H, F = FOLDED
    rng = np.random.default_rng(22)
    inp = make_block_inputs(N, T, D, F, "bf16", seed=22)
    prm = make_affine_params(D, F, "bf16", seed=22)
    for k in ("ln1_gamma", "ln2_gamma", "ln1_beta", "ln2_beta"):
        prm[k] = round_to(rng.standard_normal(D), "bf16")
    out, _ = _run(inp, prm, H, 1e-6, "bf16")
    assert_close(to_host(out), _oracle(inp, prm, H, 1e-6), "bf16", "folded, large gains")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_affine_without_parameters_is_the_plain_block(dtype):
    import torch
    inp = make_block_inputs(2, 65, 128, 512, dtype, seed=2)
    dev = {k: to_dev(v, dtype) for k, v in inp.items()}
    plain = vb.forward(dev["x"], *(dev[k] for k in WEIGHTS), 2, 1e-6)
    assert torch.equal(vb.forward_affine(dev["x"], *(dev[k] for k in WEIGHTS), 2, 1e-6), plain)
    assert torch.equal(vb.forward_affine(dev["x"], *(dev[k] for k in WEIGHTS), 2, 1e-6,
                                         params={}), plain)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("N,T,D,H,F", [(2, 197, 256, 4, 1024), FOLDED])
def test_affine_packed_matches_unpacked(dtype, N, T, D, H, F):
    import torch
    inp = make_block_inputs(N, T, D, F, dtype, seed=3)
    prm = make_affine_params(D, F, dtype, seed=3)
    a, _ = _run(inp, prm, H, 1e-6, dtype)
    b, _ = _run(inp, prm, H, 1e-6, dtype, packed=True)
    assert torch.equal(a, b)


def test_affine_key_bias_barely_matters_on_the_gpu_too():
    # The key bias shifts each query's scores by one constant: the output
    # moves only by rounding.
    inp = make_block_inputs(2, 65, 128, 512, "bf16", seed=4)
    prm = make_affine_params(128, 512, "bf16", seed=4)
    a, _ = _run(inp, prm, 2, 1e-6, "bf16")
    prm2 = dict(prm, b_k=round_to(prm["b_k"] + 1.0, "bf16"))
    b, _ = _run(inp, prm2, 2, 1e-6, "bf16")
    assert_close(to_host(b), to_host(a), "bf16", "key bias shifted by 1")
