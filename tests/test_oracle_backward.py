"""Pins for the float64 backward oracle (CPU only).

The backward oracle (``oracle.backward``) is the exact derivative of the
block's forward definition (crackedaicode.com "ViT Encoder Block"); the pages
ask for the gradients of every parameter (nipunbatra.github.io vision1
transcript, Pages 88 and 113; mlgrind.dev "E2E: Tiny Vision Transformer",
"Method contract") but print none.  It is trusted only through checks that do
not reuse its code:

* central finite differences of a forward pass: element by element against
  the brute-force scalar loop of ``test_oracle`` (written from the pages'
  definition, independent of the oracle), and along random directions
  against the oracle's pinned forward on larger shapes;
* closed forms: GELU'(0) = 1/2 and GELU'(z) + GELU'(-z) = 1 (the derivative
  of the tanh form's odd-part identity), a block with both residual branches
  switched off (w_o = w_mlp2 = 0: out = x, so dx = dout exactly and the
  branch weights get the gradients of plain linear maps), a single-token
  sequence (its attention weight is 1 whatever q and k are, so dw_q = dw_k =
  0);
* invariants: a LayerNorm's input gradient is orthogonal to the all-ones
  vector and to the normalised row; softmax input gradients sum to zero over
  a row, so the key gradient sums to zero over a sequence; weight gradients
  add over sequences and dx of one sequence ignores the others;
* torch autograd in float64 over a forward built from torch's own layer_norm,
  tanh-GELU and scaled-dot-product attention (a library cross-check);
* planted mistakes, one oracle step at a time, each of which the finite
  differences must catch.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import backward as obw
from oracle import block as ob
from test_oracle import brute_force_block


def _rand(rng, N, T, D, F, scale=1.0):
    x = rng.standard_normal((N, T, D)) * scale
    ws = [rng.standard_normal(s) / math.sqrt(s[0]) for s in
          [(D, D), (D, D), (D, D), (D, D), (D, F), (F, D)]]
    dout = rng.standard_normal((N, T, D))
    return x, ws, dout


def _loss(fwd, x, ws, dout):
    return float(np.sum(fwd(x, ws) * dout))


def _brute_fwd(H, eps):
    return lambda x, ws: brute_force_block(x, *ws, H, eps)


def _oracle_fwd(H, eps):
    return lambda x, ws: ob.vit_block(x, *ws, H, eps)


def _fd_elementwise(fwd, x, ws, dout, step=1e-5):
    """Central differences of sum(dout * fwd) for every entry of x and of each weight."""
    params = [x] + list(ws)
    grads = []
    for pi, p in enumerate(params):
        g = np.zeros_like(p)
        for idx in np.ndindex(p.shape):
            vals = []
            for sgn in (1.0, -1.0):
                q = [a.copy() for a in params]
                q[pi][idx] += sgn * step
                vals.append(_loss(fwd, q[0], q[1:], dout))
            g[idx] = (vals[0] - vals[1]) / (2.0 * step)
        grads.append(g)
    return dict(zip(oracle.GRAD_KEYS, grads))


def _max_rel_err(got, want):
    return max(float(np.abs(got[k] - want[k]).max() / (1.0 + np.abs(want[k]).max()))
               for k in oracle.GRAD_KEYS)


TINY = dict(N=2, T=3, D=4, H=2, F=8, eps=1e-5)


def _brute_fd_case(seed=0, shape=TINY):
    rng = np.random.default_rng(seed)
    x, ws, dout = _rand(rng, shape["N"], shape["T"], shape["D"], shape["F"])
    fd = _fd_elementwise(_brute_fwd(shape["H"], shape["eps"]), x, ws, dout)
    return x, ws, dout, fd


_FD_CACHE = {}


def _brute_fd_err(seed=0):
    """Largest relative gap between the oracle's gradients and brute-force finite differences."""
    if seed not in _FD_CACHE:
        _FD_CACHE[seed] = _brute_fd_case(seed)
    x, ws, dout, fd = _FD_CACHE[seed]
    got = oracle.vit_block_backward(x, *ws, dout, TINY["H"], TINY["eps"])
    return _max_rel_err(got, fd)


# Central differences with step 1e-5 in float64: truncation ~1e-10, rounding ~1e-11.
FD_TOL = 1e-7


# ------------------------------------------------------------ finite differences

@pytest.mark.parametrize("seed", [0, 1])
def test_gradients_match_brute_force_finite_differences(seed):
    assert _brute_fd_err(seed) < FD_TOL


@pytest.mark.parametrize("shape", [
    dict(N=2, T=7, D=16, H=4, F=32, eps=1e-6),
    dict(N=1, T=5, D=6, H=6, F=12, eps=1e-5),   # d_h = 1
    dict(N=2, T=4, D=8, H=1, F=8, eps=1e-5),    # one head
    dict(N=3, T=1, D=8, H=2, F=16, eps=1e-5),   # one token
    dict(N=1, T=33, D=32, H=2, F=64, eps=1e-6),
])
def test_directional_finite_differences(shape):
    """<grad, delta> against the central difference of the loss along random delta."""
    rng = np.random.default_rng(7)
    x, ws, dout = _rand(rng, shape["N"], shape["T"], shape["D"], shape["F"])
    got = oracle.vit_block_backward(x, *ws, dout, shape["H"], shape["eps"])
    fwd = _oracle_fwd(shape["H"], shape["eps"])
    params = [x] + ws
    step = 1e-5
    for pi, key in enumerate(oracle.GRAD_KEYS):
        for _ in range(3):
            delta = rng.standard_normal(params[pi].shape)
            plus = [a.copy() for a in params]
            minus = [a.copy() for a in params]
            plus[pi] += step * delta
            minus[pi] -= step * delta
            fd = (_loss(fwd, plus[0], plus[1:], dout)
                  - _loss(fwd, minus[0], minus[1:], dout)) / (2 * step)
            an = float(np.sum(got[key] * delta))
            assert abs(fd - an) <= FD_TOL * (1.0 + abs(an)), (key, fd, an)


def test_constant_row_gradient_is_finite_and_matches_finite_differences():
    """A token whose features are all equal (variance 0, LN output 0) keeps a finite gradient."""
    rng = np.random.default_rng(3)
    x, ws, dout = _rand(rng, 1, 3, 4, 8)
    x[0, 1, :] = 0.75
    got = oracle.vit_block_backward(x, *ws, dout, 2, 1e-5)
    fd = _fd_elementwise(_brute_fwd(2, 1e-5), x, ws, dout, step=1e-6)
    assert all(np.isfinite(got[k]).all() for k in oracle.GRAD_KEYS)
    # The variance is quadratic in the perturbation here, so use a smaller step.
    assert _max_rel_err(got, fd) < 1e-5


# -------------------------------------------------------------- LayerNorm step

def test_layer_norm_backward_invariants_and_finite_differences():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 12)) * 3 + 1
    g = rng.standard_normal((5, 12))
    eps = 1e-5
    dx = oracle.layer_norm_backward(x, g, eps)
    xhat = oracle.layer_norm(x, eps)
    # LN is invariant to adding a constant to a row, and nearly to scaling it.
    assert np.abs(dx.sum(axis=-1)).max() < 1e-12
    # d/dt LN((1 + t) x) at t = 0 is (eps / (var + eps)) * xhat; so <dx, x - mean> = eps-term.
    dev = x - x.mean(axis=-1, keepdims=True)
    var = (dev ** 2).mean(axis=-1)
    want = (g * xhat).sum(axis=-1) * eps / (var + eps)
    assert np.allclose((dx * dev).sum(axis=-1), want, rtol=1e-10, atol=1e-12)
    step = 1e-6
    for idx in [(0, 0), (2, 5), (4, 11)]:
        xp, xm = x.copy(), x.copy()
        xp[idx] += step
        xm[idx] -= step
        fd = (np.sum(oracle.layer_norm(xp, eps) * g) - np.sum(oracle.layer_norm(xm, eps) * g)) \
            / (2 * step)
        assert abs(fd - dx[idx]) < 1e-7


# ------------------------------------------------------------------- GELU step

def test_gelu_grad_closed_forms():
    z = np.linspace(-8, 8, 161)
    g = oracle.gelu_tanh_grad(z)
    assert oracle.gelu_tanh_grad(np.array([0.0]))[0] == 0.5
    # GELU(z) - GELU(-z) = z  =>  GELU'(z) + GELU'(-z) = 1.
    assert np.abs(g + oracle.gelu_tanh_grad(-z) - 1.0).max() < 1e-15
    assert abs(oracle.gelu_tanh_grad(np.array([30.0]))[0] - 1.0) < 1e-12
    assert abs(oracle.gelu_tanh_grad(np.array([-30.0]))[0]) < 1e-12
    step = 1e-6
    fd = (oracle.gelu_tanh(z + step) - oracle.gelu_tanh(z - step)) / (2 * step)
    assert np.abs(fd - g).max() < 1e-8


def test_gelu_grad_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    z = torch.linspace(-6, 6, 97, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.gelu(z, approximate="tanh").sum().backward()
    assert np.abs(z.grad.numpy() - oracle.gelu_tanh_grad(z.detach().numpy())).max() < 1e-14


# -------------------------------------------------------- softmax / attention

def test_softmax_backward_rows_sum_to_zero_and_match_finite_differences():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((3, 6)) * 2
    g = rng.standard_normal((3, 6))
    p = oracle.softmax_rows(s)
    ds = oracle.softmax_backward(p, g)
    assert np.abs(ds.sum(axis=-1)).max() < 1e-15
    step = 1e-6
    for idx in [(0, 0), (1, 3), (2, 5)]:
        sp, sm = s.copy(), s.copy()
        sp[idx] += step
        sm[idx] -= step
        fd = (np.sum(oracle.softmax_rows(sp) * g) - np.sum(oracle.softmax_rows(sm) * g)) \
            / (2 * step)
        assert abs(fd - ds[idx]) < 1e-8


def test_key_gradient_sums_to_zero_over_each_sequence():
    """Adding one vector to every key of a head shifts a query's scores equally: no effect."""
    rng = np.random.default_rng(2)
    N, T, D, H, F = 3, 9, 12, 3, 24
    x, ws, dout = _rand(rng, N, T, D, F)
    r = oracle.vit_block_backward_stages(x, *ws, dout, H, 1e-6)
    assert np.abs(r["dk"].sum(axis=1)).max() < 1e-12 * (1 + np.abs(r["dk"]).max())


def test_single_token_has_no_query_or_key_gradient():
    rng = np.random.default_rng(4)
    x, ws, dout = _rand(rng, 4, 1, 8, 16)
    g = oracle.vit_block_backward(x, *ws, dout, 2, 1e-5)
    assert np.all(g["dw_q"] == 0.0) and np.all(g["dw_k"] == 0.0)
    assert np.abs(g["dw_v"]).max() > 0.1


# ----------------------------------------------------------------- whole block

def test_residual_branches_off_closed_form():
    """w_o = w_mlp2 = 0: out = x, dx = dout exactly; the branch weights see plain linear maps."""
    rng = np.random.default_rng(5)
    N, T, D, H, F, eps = 2, 5, 8, 2, 16, 1e-5
    x, ws, dout = _rand(rng, N, T, D, F)
    ws[3] = np.zeros((D, D))
    ws[5] = np.zeros((F, D))
    g = oracle.vit_block_backward(x, *ws, dout, H, eps)
    assert np.array_equal(g["dx"], dout)
    for k in ("dw_q", "dw_k", "dw_v", "dw_mlp1"):
        assert np.all(g[k] == 0.0), k
    xn = oracle.layer_norm(x, eps)
    att = oracle.multi_head_attention(xn, ws[0], ws[1], ws[2], H).reshape(-1, D)
    hid = oracle.gelu_tanh(xn.reshape(-1, D) @ ws[4])
    assert np.allclose(g["dw_o"], att.T @ dout.reshape(-1, D), rtol=1e-12, atol=1e-12)
    assert np.allclose(g["dw_mlp2"], hid.T @ dout.reshape(-1, D), rtol=1e-12, atol=1e-12)


def test_layer_norm_gradients_are_orthogonal_to_ones():
    """dx - dy and dy - dout are LayerNorm input gradients: zero row sums."""
    rng = np.random.default_rng(6)
    x, ws, dout = _rand(rng, 2, 6, 16, 32)
    r = oracle.vit_block_backward_stages(x, *ws, dout, 4, 1e-6)
    assert np.abs((r["dx"] - r["dy"]).sum(axis=-1)).max() < 1e-12
    assert np.abs((r["dy"] - dout).sum(axis=-1)).max() < 1e-12


def test_batch_additivity_and_independence():
    rng = np.random.default_rng(8)
    N, T, D, H, F = 4, 5, 8, 2, 16
    x, ws, dout = _rand(rng, N, T, D, F)
    whole = oracle.vit_block_backward(x, *ws, dout, H, 1e-5, chunk=3)
    parts = [oracle.vit_block_backward(x[n:n + 1], *ws, dout[n:n + 1], H, 1e-5)
             for n in range(N)]
    assert np.allclose(whole["dx"], np.concatenate([p["dx"] for p in parts]), rtol=0, atol=1e-13)
    for k in oracle.GRAD_KEYS[1:]:
        assert np.allclose(whole[k], sum(p[k] for p in parts), rtol=0, atol=1e-12), k
    # A sequence whose output gradient is zero contributes nothing.
    d2 = dout.copy()
    d2[1:] = 0.0
    g2 = oracle.vit_block_backward(x, *ws, d2, H, 1e-5)
    assert np.all(g2["dx"][1:] == 0.0)
    for k in oracle.GRAD_KEYS[1:]:
        assert np.allclose(g2[k], parts[0][k], rtol=0, atol=1e-12), k


def test_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    F_ = torch.nn.functional
    rng = np.random.default_rng(9)
    N, T, D, H, Fd, eps = 3, 11, 24, 4, 48, 1e-6
    x, ws, dout = _rand(rng, N, T, D, Fd)
    tx = torch.tensor(x, requires_grad=True)
    tw = [torch.tensor(w, requires_grad=True) for w in ws]
    wq, wk, wv, wo, w1, w2 = tw

    def heads(t):
        return t.reshape(N, T, H, D // H).transpose(1, 2)

    xn = F_.layer_norm(tx, (D,), eps=eps)
    a = F_.scaled_dot_product_attention(heads(xn @ wq), heads(xn @ wk), heads(xn @ wv))
    y = tx + a.transpose(1, 2).reshape(N, T, D) @ wo
    out = y + F_.gelu(F_.layer_norm(y, (D,), eps=eps) @ w1, approximate="tanh") @ w2
    (out * torch.tensor(dout)).sum().backward()
    want = dict(zip(oracle.GRAD_KEYS, [tx.grad.numpy()] + [w.grad.numpy() for w in tw]))
    got = oracle.vit_block_backward(x, *ws, dout, H, eps)
    assert _max_rel_err(got, want) < 1e-12


def test_rejects_mismatched_dout():
    rng = np.random.default_rng(0)
    x, ws, dout = _rand(rng, 2, 3, 4, 8)
    with pytest.raises(ValueError):
        oracle.vit_block_backward(x, *ws, dout[:, :2], 2, 1e-5)


# ------------------------------------------------------------- planted mistakes

def _ln_bwd_no_mean(x, g, eps):
    d = x.shape[-1]
    dev = x - x.mean(axis=-1, keepdims=True)
    var = (dev * dev).mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt(var + eps)
    g_var = (g * dev).sum(axis=-1, keepdims=True) * (-0.5) * r ** 3
    return g * r + g_var * (2.0 / d) * dev


def _ln_bwd_no_var(x, g, eps):
    dev = x - x.mean(axis=-1, keepdims=True)
    r = 1.0 / np.sqrt((dev * dev).mean(axis=-1, keepdims=True) + eps)
    g_dev = g * r
    return g_dev - g_dev.mean(axis=-1, keepdims=True)


def _gelu_grad_erf(z):
    z = np.asarray(z, dtype=np.float64)
    from scipy.special import erf
    return 0.5 * (1 + erf(z / math.sqrt(2))) + z * np.exp(-0.5 * z * z) / math.sqrt(2 * math.pi)


def _gelu_grad_no_cubic(z):
    z = np.asarray(z, dtype=np.float64)
    c = math.sqrt(2 / math.pi)
    t = np.tanh(c * (z + 0.044715 * z ** 3))
    return 0.5 * (1 + t) + 0.5 * z * (1 - t * t) * c


def _softmax_bwd_no_row_term(p, g):
    return p * g


def _attn_bwd_unscaled(qh, kh, vh, p, d_o):
    dq, dk, dv = _ORIG_ATTN_BWD(qh, kh, vh, p, d_o)
    s = math.sqrt(qh.shape[-1])
    return dq * s, dk * s, dv


def _attn_bwd_dk_untransposed(qh, kh, vh, p, d_o):
    dq, _, dv = _ORIG_ATTN_BWD(qh, kh, vh, p, d_o)
    dp = np.matmul(d_o, np.swapaxes(vh, -1, -2))
    ds = oracle.softmax_backward(p, dp)
    return dq, np.matmul(ds, qh) / math.sqrt(qh.shape[-1]), dv


def _attn_bwd_dv_untransposed(qh, kh, vh, p, d_o):
    dq, dk, _ = _ORIG_ATTN_BWD(qh, kh, vh, p, d_o)
    return dq, dk, np.matmul(p, d_o)


def _wgrad_transposed(a, g):
    w = _ORIG_WGRAD(a, g)
    return w.T if w.shape[0] == w.shape[1] else w


_ORIG_ATTN_BWD = obw.attention_backward
_ORIG_WGRAD = obw._wgrad

MUTANTS = {
    "LayerNorm backward without the mean term": ("layer_norm_backward", _ln_bwd_no_mean),
    "LayerNorm backward without the variance term": ("layer_norm_backward", _ln_bwd_no_var),
    "GELU derivative of the erf form": ("gelu_tanh_grad", _gelu_grad_erf),
    "GELU derivative without the cubic term": ("gelu_tanh_grad", _gelu_grad_no_cubic),
    "softmax backward without the row term": ("softmax_backward", _softmax_bwd_no_row_term),
    "score scale missing in dq and dk": ("attention_backward", _attn_bwd_unscaled),
    "dk from dS instead of dS^T": ("attention_backward", _attn_bwd_dk_untransposed),
    "dv from P instead of P^T": ("attention_backward", _attn_bwd_dv_untransposed),
    "square weight gradients transposed": ("_wgrad", _wgrad_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    _brute_fd_err(0)  # fill the finite-difference cache with the true oracle untouched
    monkeypatch.setattr(obw, attr, fn)
    assert _brute_fd_err(0) > 1e-4, f"pins did not catch: {name}"
