"""GPU parity on seeded random shapes: products, attention and the front end.

The parity tests elsewhere pick shapes for the cases each kernel decides on;
these draw shapes at random (seeded, so every run checks the same ones) over
the ranges the kernels accept: rows and columns that leave ragged last tiles,
K and N that do or do not reach the MFMA kernels' multiples (both dtypes, so
the bf16 and fp32 matrix-core kernels and the any-shape VALU kernels all run),
sequence lengths from 1 to a few hundred, and head widths from 8 to 128.
Every case is held to the plain bars against the float64 oracle.
"""

import math

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import round_to

from gpu_util import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

EPIS = {"none": vb.EPI_NONE, "residual": vb.EPI_RESIDUAL, "gelu": vb.EPI_GELU}


def _rand(rng, shape, dtype, scale=1.0):
    return round_to(rng.standard_normal(shape) * scale, dtype)


def _linear_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 700))
        # K: a multiple of 64 (bf16 MFMA), of 4 (fp32 MFMA) or anything.
        K = int(rng.choice([64 * rng.integers(1, 20), 4 * rng.integers(1, 200),
                            rng.integers(1, 300)]))
        N = int(rng.choice([8 * rng.integers(1, 100), 4 * rng.integers(1, 150),
                            rng.integers(1, 400)]))
        epi = ["none", "residual", "gelu"][i % 3]
        out.append((M, K, N, epi, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("M,K,N,epi,bias", _linear_cases(18, 2024))
def test_linear_random(dtype, M, K, N, epi, bias):
    rng = np.random.default_rng(M * 131 + K * 17 + N)
    a = _rand(rng, (M, K), dtype)
    w = _rand(rng, (K, N), dtype, scale=1 / math.sqrt(K))
    r = _rand(rng, (M, N), dtype)
    b = _rand(rng, (N,), dtype, scale=0.5) if bias else None
    got = to_host(vb.linear(to_dev(a, dtype), to_dev(w.T, dtype), EPIS[epi],
                            residual=to_dev(r, dtype) if epi == "residual" else None,
                            bias=None if b is None else to_dev(b, dtype)))
    ref = oracle.add_bias(oracle.project(a, w), b)
    if epi == "residual":
        ref = r + ref
    elif epi == "gelu":
        ref = oracle.gelu_tanh(ref)
    assert_close(got, ref, dtype, f"linear {epi} M={M} K={K} N={N} bias={bias}")


def _attention_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dh = int(rng.choice([8, 16, 24, 32, 40, 48, 64, 80, 96, 128]))
        H = int(rng.integers(1, 5))
        T = int(rng.choice([rng.integers(1, 70), rng.integers(70, 400)]))
        N = int(rng.integers(1, 4))
        out.append((N, T, H * dh, H))
    return out


def _attention_ref(q, k, v, H):
    a = oracle.softmax_rows(oracle.attention_scores(oracle.split_heads(q, H),
                                                    oracle.split_heads(k, H)))
    return oracle.merge_heads(np.matmul(a, oracle.split_heads(v, H)))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("N,T,D,H", _attention_cases(16, 7))
def test_attention_random(dtype, N, T, D, H):
    rng = np.random.default_rng(N * 1000 + T * 10 + D)
    q, k, v = (_rand(rng, (N, T, D), dtype, scale=1.5) for _ in range(3))
    qkv = np.concatenate([q, k, v], axis=-1).reshape(N * T, 3 * D)
    got = to_host(vb.attention(to_dev(qkv, dtype), N, T, H)).reshape(N, T, D)
    assert_close(got, _attention_ref(q, k, v, H), dtype,
                 f"attention N={N} T={T} D={D} H={H} dh={D // H}")


def _embed_cases(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        P = int(rng.choice([2, 4, 8, 14, 16]))
        gh, gw = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        C = int(rng.choice([1, 3]))
        D = int(rng.choice([8 * rng.integers(1, 40), rng.integers(1, 100)]))
        out.append((int(rng.integers(1, 5)), C, gh * P, gw * P, P, D,
                    bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("B,C,H,W,P,D,cls,pos", _embed_cases(10, 11))
def test_patch_embed_random(dtype, B, C, H, W, P, D, cls, pos):
    rng = np.random.default_rng(B + C * 7 + H * 13 + W * 17 + D)
    K = P * P * C
    img = _rand(rng, (B, C, H, W), dtype)
    w = _rand(rng, (K, D), dtype, scale=1 / math.sqrt(K))
    b = _rand(rng, (D,), dtype, scale=0.1)
    c = _rand(rng, (D,), dtype, scale=0.02) if cls else None
    Tn = (H // P) * (W // P) + (1 if cls else 0)
    p = _rand(rng, (Tn, D), dtype, scale=0.02) if pos else None
    dev = lambda a: None if a is None else to_dev(a, dtype)  # noqa: E731
    got = to_host(vb.patch_embed(dev(img), dev(w), P, dev(b), dev(c), dev(p)))
    assert_close(got, oracle.patch_embed(img, w, P, b, c, p), dtype,
                 f"patch embed {B}x{C}x{H}x{W} P={P} D={D} cls={cls} pos={pos}")
