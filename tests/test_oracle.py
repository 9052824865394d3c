"""Pins for the float64 oracle (CPU only).

The oracle is trusted only through checks that do not reuse its code:

* the three worked examples printed on tensortonic.com "ViT Encoder Block",
  section "Examples" (6 printed decimals);
* the hand trace of ai-engineer-exhaustive.pages.dev "ViT Encoder Block",
  section "Numerical Example" (4 printed decimals, hand-rounded: 1e-3);
* closed forms (GELU odd part, two-way softmax as a logistic, uniform
  attention when the queries vanish, T = 1) and invariants (zero update,
  LayerNorm moments, row-stochastic weights, token-permutation equivariance,
  batch independence);
* a brute-force scalar loop written from the block's definition on
  crackedaicode.com "ViT Encoder Block" (sections "Normalize before each
  stage", "Multi-head attention", "Feed-forward stage"), run on tiny inputs;
* float64 library cross-checks (torch's layer_norm, tanh-GELU and
  scaled-dot-product attention), used here only, never by the oracle.

The affine variant (LayerNorm gains and shifts, projection biases, from
ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "Key Equations" steps
1, 4 and 5) is pinned the same way: the scalar loop takes the parameters
too, and closed forms fix each parameter's place (the value path with
w_v = 0, the MLP with w_mlp1 = 0, the second LayerNorm through torch's
layer_norm with weight and bias), plus the invariance of the output to the
key bias (it shifts every score of a query by the same amount).

The last group plants plausible mistakes into one oracle step at a time and
asserts that the pins above catch every one of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import block as ob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _tt_case_args(c):
    a = lambda k: np.array(c[k], dtype=np.float64)  # noqa: E731
    return (a("x"), a("Wq"), a("Wk"), a("Wv"), a("Wo"), a("W1"), a("W2"), c["num_heads"])


def _tt_max_err():
    """Largest |oracle - printed| over the three printed worked examples."""
    g = _load("tt_worked_examples.json")
    worst = 0.0
    for c in g["cases"]:
        x, wq, wk, wv, wo, w1, w2, h = _tt_case_args(c)
        out = oracle.vit_block(x, wq, wk, wv, wo, w1, w2, h, g["eps"])
        worst = max(worst, float(np.abs(out - np.array(c["out"])).max()))
    return worst


# 6 printed decimals: half a unit in the last place, plus float64 slack.
TT_TOL = 5e-7 + 1e-12


# ---------------------------------------------------------------- brute force

def _brute_ln(row, eps):
    d = len(row)
    mu = sum(row) / d
    var = sum((v - mu) ** 2 for v in row) / d
    return [(v - mu) / math.sqrt(var + eps) for v in row]


def _brute_gelu(z):
    return 0.5 * z * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (z + 0.044715 * z * z * z)))


def brute_force_block(x, wq, wk, wv, wo, w1, w2, H, eps, params=None):
    """Scalar loops over (sequence, token, head, key, feature); tiny inputs only.

    ``params``: the affine variant's gains, shifts and biases by name (absent:
    gain 1, shift 0, bias 0), applied where the "Key Equations" put them.
    """
    x = np.asarray(x).tolist()
    wq, wk, wv, wo, w1, w2 = (np.asarray(w).tolist() for w in (wq, wk, wv, wo, w1, w2))
    N, T, D = len(x), len(x[0]), len(x[0][0])
    F = len(w1[0])
    dh = D // H
    prm = {k: np.asarray(v).tolist() for k, v in (params or {}).items()}

    def vec(name, n, fill):
        return prm.get(name, [fill] * n)

    g1, be1, g2, be2 = vec("ln1_gamma", D, 1.0), vec("ln1_beta", D, 0.0), \
        vec("ln2_gamma", D, 1.0), vec("ln2_beta", D, 0.0)
    bq, bk, bv, bo = (vec(k, D, 0.0) for k in ("b_q", "b_k", "b_v", "b_o"))
    b1, b2 = vec("b_mlp1", F, 0.0), vec("b_mlp2", D, 0.0)
    out = [[[0.0] * D for _ in range(T)] for _ in range(N)]
    for n in range(N):
        xn = [[g1[j] * val + be1[j] for j, val in enumerate(_brute_ln(x[n][t], eps))]
              for t in range(T)]

        def mat(a, w, cols, b):
            return [[sum(a[t][i] * w[i][j] for i in range(len(w))) + b[j] for j in range(cols)]
                    for t in range(len(a))]

        q, k, v = mat(xn, wq, D, bq), mat(xn, wk, D, bk), mat(xn, wv, D, bv)
        att = [[0.0] * D for _ in range(T)]
        for h in range(H):
            c0 = h * dh
            for i in range(T):
                s = [sum(q[i][c0 + c] * k[j][c0 + c] for c in range(dh)) / math.sqrt(dh)
                     for j in range(T)]
                m = max(s)
                e = [math.exp(sj - m) for sj in s]
                z = sum(e)
                for c in range(dh):
                    att[i][c0 + c] = sum(e[j] / z * v[j][c0 + c] for j in range(T))
        proj = mat(att, wo, D, bo)
        y = [[x[n][t][j] + proj[t][j] for j in range(D)] for t in range(T)]
        yn = [[g2[j] * val + be2[j] for j, val in enumerate(_brute_ln(y[t], eps))]
              for t in range(T)]
        hid = [[_brute_gelu(val) for val in row] for row in mat(yn, w1, F, b1)]
        upd = mat(hid, w2, D, b2)
        for t in range(T):
            for j in range(D):
                out[n][t][j] = y[t][j] + upd[t][j]
    return np.array(out)


def _rand_block(rng, N, T, D, F):
    x = rng.standard_normal((N, T, D))
    ws = [rng.standard_normal(s) / math.sqrt(s[0]) for s in
          [(D, D), (D, D), (D, D), (D, D), (D, F), (F, D)]]
    return [x] + ws


BRUTE_SHAPES = [(2, 3, 4, 1, 6), (2, 3, 4, 2, 6), (1, 4, 4, 4, 5), (2, 2, 6, 3, 7)]


def _brute_max_err():
    rng = np.random.default_rng(1234)
    worst = 0.0
    for (N, T, D, H, F) in BRUTE_SHAPES:
        args = _rand_block(rng, N, T, D, F)
        ref = brute_force_block(*args, H, 1e-5)
        got = oracle.vit_block(*args, H, 1e-5)
        worst = max(worst, float(np.abs(ref - got).max()))
    return worst


def _rand_params(rng, D, F):
    """Gains near 1, shifts and biases of a few tenths: every term visible."""
    p = {}
    for k in oracle.AFFINE_KEYS:
        n = F if k == "b_mlp1" else D
        p[k] = (1.0 + 0.3 * rng.standard_normal(n)) if k.endswith("gamma") \
            else 0.3 * rng.standard_normal(n)
    return p


def _brute_affine_max_err():
    rng = np.random.default_rng(4321)
    worst = 0.0
    for (N, T, D, H, F) in BRUTE_SHAPES:
        args = _rand_block(rng, N, T, D, F)
        prm = _rand_params(rng, D, F)
        ref = brute_force_block(*args, H, 1e-5, params=prm)
        got = oracle.vit_block(*args, H, 1e-5, params=prm)
        worst = max(worst, float(np.abs(ref - got).max()))
    return worst


# ------------------------------------------------------------------ the pins

def test_tt_worked_examples():
    assert _tt_max_err() <= TT_TOL


def test_tt_example2_constant_token_passes_through():
    # A constant token normalises to zero, so both updates vanish for it and
    # its output row equals its input row (example 2, third token).
    g = _load("tt_worked_examples.json")
    c = g["cases"][1]
    x, wq, wk, wv, wo, w1, w2, h = _tt_case_args(c)
    out = oracle.vit_block(x, wq, wk, wv, wo, w1, w2, h, g["eps"])
    np.testing.assert_array_equal(out[0, 2], x[0, 2])


def test_brute_force_agrees():
    assert _brute_max_err() <= 1e-12


def test_aee_layer_norm_trace():
    g = _load("aee_hand_trace.json")
    ln = g["layer_norm"]
    x = np.array(ln["x"])
    np.testing.assert_allclose(x.mean(-1), ln["mean"], atol=1e-15)
    np.testing.assert_allclose(x.var(-1), ln["variance"], atol=1e-15)
    got = oracle.layer_norm(x, 1e-6)
    assert np.abs(got - np.array(ln["normalized"])).max() <= g["tolerance"]


def test_aee_softmax_trace():
    g = _load("aee_hand_trace.json")
    s = np.array(g["softmax"]["scaled_scores"])
    got = oracle.softmax_rows(s)
    assert np.abs(got - np.array(g["softmax"]["weights"])).max() <= g["tolerance"]
    # Two-way softmax is the logistic function of the score difference.
    for r in range(2):
        p0 = 1.0 / (1.0 + math.exp(s[r, 1] - s[r, 0]))
        assert abs(got[r, 0] - p0) < 1e-15 and abs(got[r, 1] - (1.0 - p0)) < 1e-15


def test_aee_gelu_trace():
    g = _load("aee_hand_trace.json")
    got = float(oracle.gelu_tanh(np.array(g["gelu"]["z"])))
    assert abs(got - g["gelu"]["value"]) <= g["tolerance"]


def test_aee_residual_trace():
    g = _load("aee_hand_trace.json")["residual"]
    x = np.array(_load("aee_hand_trace.json")["layer_norm"]["x"])
    np.testing.assert_allclose(x + np.array(g["msa_out"]), g["x_prime"], atol=1e-15)


def test_gelu_closed_forms():
    z = np.linspace(-8, 8, 2001)
    gz = oracle.gelu_tanh(z)
    # tanh is odd, so GELU(z) - GELU(-z) = z exactly in real arithmetic.
    np.testing.assert_allclose(gz - oracle.gelu_tanh(-z), z, atol=1e-14)
    assert oracle.gelu_tanh(np.array(0.0)) == 0.0
    assert oracle.gelu_tanh(np.array(30.0)) == 30.0
    assert abs(float(oracle.gelu_tanh(np.array(-30.0)))) < 1e-300
    # It is the tanh form, not the erf form: they differ by up to ~5e-4.
    erf_form = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in z])
    diff = np.abs(gz - erf_form).max()
    assert 1e-4 < diff < 1e-3


def test_gelu_matches_torch_tanh_gelu():
    torch = pytest.importorskip("torch")
    z = np.random.default_rng(0).standard_normal(4096) * 4
    ref = torch.nn.functional.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(z), ref, rtol=1e-14, atol=1e-15)


def test_layer_norm_moments_and_constant_row():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 33)) * rng.uniform(0.1, 10, (7, 1)) + rng.uniform(-5, 5, (7, 1))
    eps = 1e-5
    y = oracle.layer_norm(x, eps)
    np.testing.assert_allclose(y.mean(-1), 0.0, atol=1e-14)
    var = x.var(-1)
    np.testing.assert_allclose(y.var(-1), var / (var + eps), rtol=1e-12)
    c = np.full((1, 16), 3.25)
    assert np.all(oracle.layer_norm(c, 1e-6) == 0.0)


def test_layer_norm_matches_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(4).standard_normal((9, 48)) * 3 + 1
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x), (48,), eps=1e-6).numpy()
    np.testing.assert_allclose(oracle.layer_norm(x, 1e-6), ref, rtol=1e-12, atol=1e-13)


def test_attention_rows_are_stochastic():
    rng = np.random.default_rng(5)
    x, wq, wk, *_ = _rand_block(rng, 3, 9, 12, 8)
    a = oracle.attention_weights(oracle.layer_norm(x, 1e-6), wq, wk, 3)
    assert a.shape == (3, 3, 9, 9)
    assert np.all(a >= 0)
    np.testing.assert_allclose(a.sum(-1), 1.0, atol=1e-14)
    # Columns need not sum to one (no symmetry between queries and keys).
    assert np.abs(a.sum(-2) - 1.0).max() > 1e-3


def test_attention_closed_forms():
    rng = np.random.default_rng(6)
    x, wq, wk, wv, *_ = _rand_block(rng, 2, 6, 8, 8)
    xn = oracle.layer_norm(x, 1e-6)
    v = xn @ wv
    # Zero queries: every score is 0, weights are uniform, output = token mean of V.
    att = oracle.multi_head_attention(xn, np.zeros_like(wq), wk, wv, 4)
    np.testing.assert_allclose(att, np.broadcast_to(v.mean(1, keepdims=True), att.shape),
                               atol=1e-14)
    # One token: it attends only to itself, output = V.
    att1 = oracle.multi_head_attention(xn[:, :1], wq, wk, wv, 4)
    np.testing.assert_allclose(att1, v[:, :1], atol=1e-15)


def test_attention_matches_torch_sdpa():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    N, T, D, H = 2, 11, 24, 3
    x, wq, wk, wv, *_ = _rand_block(rng, N, T, D, 8)
    xn = oracle.layer_norm(x, 1e-6)
    q, k, v = (torch.from_numpy(xn @ w).view(N, T, H, D // H).transpose(1, 2).contiguous()
               for w in (wq, wk, wv))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)
    ref = ref.transpose(1, 2).reshape(N, T, D).numpy()
    np.testing.assert_allclose(oracle.multi_head_attention(xn, wq, wk, wv, H), ref,
                               rtol=1e-12, atol=1e-13)


def test_zero_update_identity():
    rng = np.random.default_rng(8)
    x, wq, wk, wv, wo, w1, w2 = _rand_block(rng, 3, 5, 8, 12)
    out = oracle.vit_block(x, wq, wk, wv, np.zeros_like(wo), w1, np.zeros_like(w2), 2, 1e-5)
    np.testing.assert_array_equal(out, x)
    # Only the MLP branch, or only the attention branch.
    st = oracle.vit_block_stages(x, wq, wk, wv, wo, w1, w2, 2, 1e-5)
    out_no_mlp = oracle.vit_block(x, wq, wk, wv, wo, w1, np.zeros_like(w2), 2, 1e-5)
    np.testing.assert_array_equal(out_no_mlp, st["y"])
    out_no_att = oracle.vit_block(x, wq, wk, wv, np.zeros_like(wo), w1, w2, 2, 1e-5)
    xn = oracle.layer_norm(x, 1e-5)
    mlp_x = oracle.gelu_tanh(xn @ w1) @ w2
    np.testing.assert_allclose(out_no_att, x + mlp_x, atol=1e-14)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(9)
    args = _rand_block(rng, 2, 7, 8, 16)
    out = oracle.vit_block(*args, 2, 1e-6)
    perm = rng.permutation(7)
    args_p = [args[0][:, perm]] + args[1:]
    out_p = oracle.vit_block(*args_p, 2, 1e-6)
    np.testing.assert_allclose(out_p, out[:, perm], atol=1e-13)


def test_batch_independence_and_chunking():
    rng = np.random.default_rng(10)
    args = _rand_block(rng, 5, 4, 8, 16)
    out = oracle.vit_block(*args, 4, 1e-6, chunk=8)
    x2 = args[0].copy()
    x2[3] = rng.standard_normal(x2[3].shape)
    out2 = oracle.vit_block(*([x2] + args[1:]), 4, 1e-6, chunk=8)
    np.testing.assert_allclose(np.delete(out2, 3, 0), np.delete(out, 3, 0), atol=1e-14)
    out_c1 = oracle.vit_block(*args, 4, 1e-6, chunk=1)
    np.testing.assert_allclose(out_c1, out, atol=1e-14)


def test_shape_checks():
    x = np.zeros((1, 2, 6))
    w = np.zeros((6, 6))
    with pytest.raises(ValueError):
        oracle.vit_block(x, w, w, w, w, w, w, 4, 1e-6)
    with pytest.raises(ValueError):
        oracle.vit_block(x[0], w, w, w, w, w, w, 2, 1e-6)


# ------------------------------------------------------- planted mistakes

# ------------------------------------------------------- the affine variant

def test_affine_brute_force_agrees():
    assert _brute_affine_max_err() < 1e-12


def test_affine_with_identity_parameters_is_the_plain_block():
    rng = np.random.default_rng(7)
    N, T, D, H, F = 2, 5, 8, 2, 12
    args = _rand_block(rng, N, T, D, F)
    ident = {k: (np.ones(D) if k.endswith("gamma") else
                 np.zeros(F if k == "b_mlp1" else D)) for k in oracle.AFFINE_KEYS}
    plain = oracle.vit_block(*args, H, 1e-6)
    assert np.array_equal(oracle.vit_block(*args, H, 1e-6, params=ident), plain)
    assert np.array_equal(oracle.vit_block(*args, H, 1e-6, params={}), plain)


def test_value_path_biases_closed_form():
    # w_v = 0: every value row is b_v, so whatever the weights, each head
    # outputs its part of b_v and y = x + b_v @ w_o + b_o, token by token.
    rng = np.random.default_rng(8)
    N, T, D, H, F = 2, 4, 6, 3, 5
    x, wq, wk, _, wo, w1, w2 = _rand_block(rng, N, T, D, F)
    prm = _rand_params(rng, D, F)
    st = oracle.vit_block_stages(x, wq, wk, np.zeros((D, D)), wo, w1, w2, H, 1e-6, params=prm)
    want = x + (prm["b_v"] @ wo + prm["b_o"])[None, None, :]
    assert np.abs(st["y"] - want).max() < 1e-12


def test_key_bias_does_not_change_the_output():
    # b_k adds q_i . b_k to every score of query i: softmax is unchanged.
    rng = np.random.default_rng(9)
    N, T, D, H, F = 2, 6, 8, 2, 10
    args = _rand_block(rng, N, T, D, F)
    prm = _rand_params(rng, D, F)
    a = oracle.vit_block(*args, H, 1e-6, params=prm)
    prm2 = dict(prm, b_k=prm["b_k"] + 3.0 * rng.standard_normal(D))
    b = oracle.vit_block(*args, H, 1e-6, params=prm2)
    assert np.abs(a - b).max() < 1e-11
    # ... while the same shift on the query bias does change it.
    prm3 = dict(prm, b_q=prm["b_q"] + 3.0 * rng.standard_normal(D))
    assert np.abs(oracle.vit_block(*args, H, 1e-6, params=prm3) - a).max() > 1e-3


def test_mlp_biases_closed_form():
    # w_mlp1 = 0: every hidden row is GELU(b_1), so out = y + GELU(b_1) @ w_mlp2 + b_2.
    rng = np.random.default_rng(10)
    N, T, D, H, F = 1, 3, 4, 2, 6
    x, wq, wk, wv, wo, _, w2 = _rand_block(rng, N, T, D, F)
    prm = _rand_params(rng, D, F)
    st = oracle.vit_block_stages(x, wq, wk, wv, wo, np.zeros((D, F)), w2, H, 1e-6, params=prm)
    g = np.array([_brute_gelu(float(b)) for b in prm["b_mlp1"]])
    want = st["y"] + (g @ w2 + prm["b_mlp2"])[None, None, :]
    assert np.abs(st["out"] - want).max() < 1e-12


def test_second_layer_norm_affine_matches_torch():
    # w_o = 0 (so y = x + b_o), w_mlp1 = w_mlp2 = I, no MLP biases:
    # out = y + GELU(gamma_2 LN(y) + beta_2), LN from torch.
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    N, T, D, H = 2, 3, 8, 2
    x, wq, wk, wv, _, _, _ = _rand_block(rng, N, T, D, D)
    prm = _rand_params(rng, D, D)
    prm["b_mlp1"] = np.zeros(D)
    prm["b_mlp2"] = np.zeros(D)
    eye = np.eye(D)
    out = oracle.vit_block(x, wq, wk, wv, np.zeros((D, D)), eye, eye, H, 1e-6, params=prm)
    y = torch.from_numpy(x + prm["b_o"])
    ln = torch.nn.functional.layer_norm(y, (D,), torch.from_numpy(prm["ln2_gamma"]),
                                        torch.from_numpy(prm["ln2_beta"]), eps=1e-6)
    want = y + torch.nn.functional.gelu(ln, approximate="tanh")
    assert np.abs(out - want.numpy()).max() < 1e-12


def test_affine_rejects_unknown_parameter():
    rng = np.random.default_rng(12)
    args = _rand_block(rng, 1, 2, 4, 4)
    with pytest.raises(ValueError):
        oracle.vit_block(*args, 2, 1e-6, params={"b_qkv": np.zeros(12)})


# ------------------------------------------------------- the encoder stack

def _brute_final_ln(t, eps, g, b):
    return [[g[j] * v + b[j] for j, v in enumerate(_brute_ln(row, eps))] for row in t]


def test_encoder_brute_force_agrees():
    # L blocks by the scalar loop, then the final LN by scalar loops too.
    rng = np.random.default_rng(99)
    N, T, D, H, F, L = 2, 3, 4, 2, 6, 3
    x = rng.standard_normal((N, T, D))
    layers = []
    for _ in range(L):
        ws = _rand_block(rng, N, T, D, F)[1:]
        layers.append(dict(zip(["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"], ws),
                           params=_rand_params(rng, D, F)))
    g, b = 1.0 + 0.3 * rng.standard_normal(D), 0.3 * rng.standard_normal(D)
    t = x
    for lay in layers:
        t = brute_force_block(t, *(lay[k] for k in ["w_q", "w_k", "w_v", "w_o", "w_mlp1",
                                                     "w_mlp2"]), H, 1e-5, params=lay["params"])
    want = np.array([_brute_final_ln(t[n].tolist(), 1e-5, g.tolist(), b.tolist())
                     for n in range(N)])
    tokens, cls = oracle.encoder(x, layers, H, 1e-5, g, b)
    assert np.abs(tokens - want).max() < 1e-12
    assert np.array_equal(cls, tokens[:, 0])


def test_encoder_of_zero_updates_is_the_final_layer_norm():
    # Every block with w_o = w_mlp2 = 0 passes x through; the stack is then LN_f(x).
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(98)
    N, T, D, H, F = 2, 5, 8, 2, 12
    x = rng.standard_normal((N, T, D))
    layers = []
    for _ in range(4):
        ws = _rand_block(rng, N, T, D, F)[1:]
        lay = dict(zip(["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"], ws))
        lay["w_o"] = np.zeros((D, D))
        lay["w_mlp2"] = np.zeros((F, D))
        layers.append(lay)
    g, b = 1.0 + 0.3 * rng.standard_normal(D), 0.3 * rng.standard_normal(D)
    tokens, cls = oracle.encoder(x, layers, H, 1e-6, g, b)
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (D,), torch.from_numpy(g),
                                          torch.from_numpy(b), eps=1e-6).numpy()
    assert np.abs(tokens - want).max() < 1e-12
    assert np.abs(cls - want[:, 0]).max() < 1e-12


def test_encoder_of_one_block_is_the_block_then_layer_norm():
    rng = np.random.default_rng(97)
    N, T, D, H, F = 2, 4, 8, 2, 10
    args = _rand_block(rng, N, T, D, F)
    lay = dict(zip(["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"], args[1:]))
    tokens, _ = oracle.encoder(args[0], [lay], H, 1e-6)
    blk = brute_force_block(*args, H, 1e-6)
    want = np.array([[_brute_ln(row, 1e-6) for row in blk[n].tolist()] for n in range(N)])
    assert np.abs(tokens - want).max() < 1e-12


def _ln_unbiased(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return (x - x.mean(-1, keepdims=True)) / np.sqrt(x.var(-1, ddof=1, keepdims=True) + eps)


def _ln_eps_outside(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return (x - x.mean(-1, keepdims=True)) / (np.sqrt(x.var(-1, keepdims=True)) + eps)


def _scores_unscaled(qh, kh):
    return np.matmul(qh, np.swapaxes(kh, -1, -2))


def _scores_over_dh(qh, kh):
    return np.matmul(qh, np.swapaxes(kh, -1, -2)) / qh.shape[-1]


def _project_transposed(a, w):
    w = np.asarray(w, dtype=np.float64)
    return np.matmul(a, w.T) if w.shape[0] == w.shape[1] else np.matmul(a, w)


def _gelu_erf(z):
    z = np.asarray(z, dtype=np.float64)
    return np.vectorize(lambda v: 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))))(z)


def _gelu_bad_constant(z):
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (z + 0.04471 * z ** 3)))


def _split_interleaved(t, num_heads):
    n, tt, d = t.shape
    return t.reshape(n, tt, d // num_heads, num_heads).transpose(0, 3, 1, 2)


def _softmax_wrong_axis(s):
    e = np.exp(s - s.max(-2, keepdims=True))
    return e / e.sum(-2, keepdims=True)


def _softmax_causal(s):
    t = s.shape[-1]
    s = np.where(np.triu(np.ones((t, t), bool), 1), -np.inf, s)
    e = np.exp(s - s.max(-1, keepdims=True))
    return e / e.sum(-1, keepdims=True)


_MERGE = ob.merge_heads


def _merge_reversed(o):
    return _MERGE(np.asarray(o)[:, ::-1])


def _affine_shift_then_gain(t, gamma=None, beta=None):
    t = np.asarray(t, dtype=np.float64)
    if beta is not None:
        t = t + beta
    return t if gamma is None else t * gamma


def _affine_ignored(t, gamma=None, beta=None):
    return np.asarray(t, dtype=np.float64)


def _bias_ignored(t, b=None):
    return np.asarray(t, dtype=np.float64)


def _bias_subtracted(t, b=None):
    t = np.asarray(t, dtype=np.float64)
    return t if b is None else t - b


AFFINE_MUTANTS = {
    "shift before gain": ("affine", _affine_shift_then_gain),
    "gain and shift ignored": ("affine", _affine_ignored),
    "biases ignored": ("add_bias", _bias_ignored),
    "biases subtracted": ("add_bias", _bias_subtracted),
}


@pytest.mark.parametrize("name", sorted(AFFINE_MUTANTS))
def test_affine_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = AFFINE_MUTANTS[name]
    monkeypatch.setattr(ob, attr, fn)
    assert _brute_affine_max_err() > 1e-9, f"pins did not catch: {name}"


MUTANTS = {
    "unbiased variance": ("layer_norm", _ln_unbiased),
    "eps outside sqrt": ("layer_norm", _ln_eps_outside),
    "no score scale": ("attention_scores", _scores_unscaled),
    "scale 1/d_h": ("attention_scores", _scores_over_dh),
    "nn.Linear weight layout": ("project", _project_transposed),
    "erf GELU": ("gelu_tanh", _gelu_erf),
    "GELU constant 0.04471": ("gelu_tanh", _gelu_bad_constant),
    "interleaved heads": ("split_heads", _split_interleaved),
    "softmax over queries": ("softmax_rows", _softmax_wrong_axis),
    "causal mask": ("softmax_rows", _softmax_causal),
    "heads merged in reverse": ("merge_heads", _merge_reversed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ob, attr, fn)
    caught_tt = _tt_max_err() > TT_TOL
    caught_brute = _brute_max_err() > 1e-9
    assert caught_tt or caught_brute, f"pins did not catch: {name}"


# ------------------------------------------------------- LayerNorm statistics
#
# oracle.layer_norm_stats (each token's mean and 1 / sqrt(var + eps), the two
# numbers a LayerNorm normalises with) is the reference of the row-statistics
# kernel and of the products that fold the LayerNorm in.  Pins: the token of
# [AEE] "Numerical Example" with its printed mean and variance, closed forms
# (a constant token; a two-value token) and a scalar loop.

def _stats_pins_max_err():
    errs = []
    g = _load("aee_hand_trace.json")["layer_norm"]
    mean, rstd = oracle.layer_norm_stats(np.array(g["x"]), 1e-6)
    errs.append(np.abs(mean - np.array(g["mean"])).max())
    errs.append(np.abs(rstd - 1.0 / np.sqrt(np.array(g["variance"]) + 1e-6)).max())
    # A constant token: mean c, variance 0, so rstd = 1 / sqrt(eps).
    m, r = oracle.layer_norm_stats(np.full((1, 6), 2.5), 1e-6)
    errs += [abs(m[0] - 2.5), abs(r[0] - 1.0 / math.sqrt(1e-6)) * 1e-3]
    # Two values a, b: mean (a + b) / 2, population variance ((a - b) / 2)^2.
    a, b = 1.75, -0.5
    m, r = oracle.layer_norm_stats(np.array([[a, b]]), 1e-5)
    errs += [abs(m[0] - (a + b) / 2), abs(r[0] - 1.0 / math.sqrt(((a - b) / 2) ** 2 + 1e-5))]
    # Scalar loop over random tokens.
    x = np.random.default_rng(3).standard_normal((5, 7)) * 2.0 + 0.3
    m, r = oracle.layer_norm_stats(x, 1e-5)
    for i, row in enumerate(x.tolist()):
        mu = sum(row) / len(row)
        var = sum((v - mu) ** 2 for v in row) / len(row)
        errs += [abs(m[i] - mu), abs(r[i] - 1.0 / math.sqrt(var + 1e-5))]
    return max(errs)


def test_layer_norm_stats_pins():
    assert _stats_pins_max_err() <= 1e-12


def test_layer_norm_stats_give_the_layer_norm():
    x = np.random.default_rng(4).standard_normal((3, 4, 10)) * 1.5 - 0.7
    m, r = oracle.layer_norm_stats(x, 1e-6)
    np.testing.assert_allclose((x - m[..., None]) * r[..., None], oracle.layer_norm(x, 1e-6),
                               rtol=1e-13, atol=1e-13)


def _stats_unbiased(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x.mean(-1), 1.0 / np.sqrt(x.var(-1, ddof=1) + eps)


def _stats_eps_outside(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x.mean(-1), 1.0 / (np.sqrt(x.var(-1)) + eps)


def _stats_not_inverted(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x.mean(-1), np.sqrt(x.var(-1) + eps)


def _stats_mean_of_squares(x, eps):
    x = np.asarray(x, dtype=np.float64)
    return x.mean(-1), 1.0 / np.sqrt((x * x).mean(-1) + eps)


STATS_MUTANTS = {
    "unbiased variance": _stats_unbiased,
    "eps outside sqrt": _stats_eps_outside,
    "sqrt not inverted": _stats_not_inverted,
    "uncentred second moment": _stats_mean_of_squares,
}


@pytest.mark.parametrize("name", sorted(STATS_MUTANTS))
def test_layer_norm_stats_pins_catch_planted_mistake(name, monkeypatch):
    monkeypatch.setattr(ob, "layer_norm_stats", STATS_MUTANTS[name])
    monkeypatch.setattr(oracle, "layer_norm_stats", STATS_MUTANTS[name])
    assert _stats_pins_max_err() > 1e-9, f"pins did not catch: {name}"
