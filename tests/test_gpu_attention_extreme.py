"""GPU parity of the attention step at extreme score ranges, against the oracle.

crackedaicode.com "ViT Encoder Block", "Multi-head attention" asks for a
softmax that is stable across key positions.  The attention kernels walk the
keys in chunks with a running reference maximum per query; these cases make
that reference move far and often: later chunks raise a query's maximum by
tens to hundreds of log2 units (keys whose norms grow along the sequence, a
dominant key planted in a late or the last partial chunk, a large per-key
score bias), or leave every later chunk far below the first (keys that
shrink, so later probabilities underflow).  Given bf16 q, k, v the step is
well conditioned (scores are exact products of the given values summed in
fp32; each probability is rounded once), so it is held to the plain bar,
3e-2 (1 + |o|) elementwise, against the float64 oracle.

Covered: the streaming kernel (head widths 64 and 80 at every T: eight- and
four-wave workgroups), the resident kernel (head widths 96 and 128 at T = 257
and 197), the first-queries entry used by the class-token readout, and fp32
cases (the fp32 matrix-core kernel and the VALU kernel) at the fp32 bar.
"""

import math

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import round_to

from gpu_util import assert_close, to_dev, to_host

pytestmark = pytest.mark.gpu

LOG2E = math.log2(math.e)


def _attention_ref(q, k, v, H):
    a = oracle.softmax_rows(oracle.attention_scores(oracle.split_heads(q, H),
                                                    oracle.split_heads(k, H)))
    return oracle.merge_heads(np.matmul(a, oracle.split_heads(v, H)))


def _scores_log2(q, k, H):
    """(N, H, T, T) scores in log2 units (float64, from the given values)."""
    return oracle.attention_scores(oracle.split_heads(q, H), oracle.split_heads(k, H)) * LOG2E


def _max_jump(s):
    """Largest rise of a query's running maximum from one 64-key chunk to the
    next, in log2 units: (N, H, T)."""
    T = s.shape[-1]
    prev = np.max(s[..., :min(64, T)], axis=-1)
    jump = np.zeros_like(prev)
    for c in range(64, T, 64):
        cur = np.maximum(prev, np.max(s[..., c:c + 64], axis=-1))
        jump = np.maximum(jump, cur - prev)
        prev = cur
    return jump


def _case(kind, N, T, D, H, dtype, seed):
    """Seeded q, k, v (N, T, D) rounded to dtype, for one pattern."""
    rng = np.random.default_rng([seed, T, D])
    q = rng.standard_normal((N, T, D))
    k = rng.standard_normal((N, T, D))
    v = rng.standard_normal((N, T, D))
    j = np.arange(T, dtype=np.float64)[None, :, None]
    dh = D // H
    if kind == "growing":      # key norms grow ~3x per 64 keys: maxima keep jumping
        q *= 6.0
        k *= 1.0 + 3.0 * j / 64.0
    elif kind == "shrinking":  # the largest scores come first; later chunks underflow
        q *= 6.0
        k *= 1.0 + 3.0 * (T - 1 - j) / 64.0
    elif kind in ("late_key", "tail_key"):
        # Feature 0 of every head: all queries share a large value and one
        # key (in the third chunk, or the last, partial one) gets a large
        # value too: that key's score rises by ~96 natural units for every
        # query, so every running maximum jumps there.
        star = min(150, T - 1) if kind == "late_key" else T - 2
        for h in range(H):
            q[:, :, h * dh] = 16.0
            k[:, :, h * dh] = rng.standard_normal((N, T)) * 0.5
            k[:, star, h * dh] = 48.0
    elif kind == "key_bias":
        # A per-key score bias through feature 0 of every head: keys carry
        # 40 + 30 (j // 64) + 10 sin(0.37 j), stepping up with every chunk of
        # 64 keys.  Even heads' queries carry +16 there (their maxima rise by
        # ~60 natural units per chunk), odd heads' -24 (every score of theirs
        # lies ~90 or more natural units below 0, the maximum in the first chunk).
        # Heads wider than 80 scale those query values by sqrt(dh / 80) so the
        # 1 / sqrt(dh) score scale leaves the same ranges.
        bias = 40.0 + 30.0 * (np.arange(T) // 64) + 10.0 * np.sin(np.arange(T) * 0.37)
        amp = max(1.0, math.sqrt(dh / 80.0))
        for h in range(H):
            q[:, :, h * dh] = (16.0 if h % 2 == 0 else -24.0) * amp
            k[:, :, h * dh] = bias[None, :]
    else:
        raise ValueError(kind)
    return tuple(round_to(a, dtype) for a in (q, k, v))


KINDS = ["growing", "shrinking", "late_key", "tail_key", "key_bias"]
SHAPES = [
    # (N, T, D, H): head widths 64 and 80 stream at every T; 96 and 128 are
    # resident while the sequence fits in LDS.
    (2, 197, 128, 2),
    (2, 257, 128, 2),
    (1, 1025, 128, 2),
    (2, 197, 160, 2),
    (2, 257, 160, 2),
    (1, 1025, 160, 2),
    (2, 257, 192, 2),
    (2, 197, 256, 2),
]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("N,T,D,H", SHAPES)
def test_attention_extreme_scores(kind, N, T, D, H):
    q, k, v = _case(kind, N, T, D, H, "bf16", seed=21)
    s = _scores_log2(q, k, H)
    if kind in ("growing", "late_key", "tail_key", "key_bias"):
        # Running maxima rise by far more than any lazy-rescale slack.
        assert np.max(_max_jump(s)) > 64.0
    assert np.max(np.abs(s)) > 96.0  # scores in the hundreds of log2 units
    if kind == "key_bias":
        assert (s.max(-1) < -96).any()  # some queries' scores all far below 0
    qkv = np.concatenate([q, k, v], axis=-1).reshape(N * T, 3 * D)
    got = to_host(vb.attention(to_dev(qkv, "bf16"), N, T, H)).reshape(N, T, D)
    assert_close(got, _attention_ref(q, k, v, H), "bf16",
                 f"attention {kind} N={N} T={T} D={D} H={H}")


@pytest.mark.parametrize("kind", ["growing", "tail_key", "key_bias"])
@pytest.mark.parametrize("N,T,D,H", [(2, 197, 128, 2), (1, 1025, 128, 2), (2, 257, 160, 2)])
def test_attention_first_queries_extreme_scores(kind, N, T, D, H):
    # The class-token readout's attention: the first 32 queries of each
    # sequence against every key.
    q, k, v = _case(kind, N, T, D, H, "bf16", seed=22)
    qkv = np.concatenate([q, k, v], axis=-1).reshape(N * T, 3 * D)
    got = to_host(vb.attention_first_queries(to_dev(qkv, "bf16"), N, T, H)).reshape(N, T, D)
    nq = min(T, 32)
    ref = _attention_ref(q[:, :nq], k, v, H)
    assert_close(got[:, :nq], ref, "bf16", f"first queries {kind} N={N} T={T} D={D}")


@pytest.mark.parametrize("N,T,D,H", [(2, 197, 128, 2), (3, 40, 96, 3), (2, 1, 128, 2),
                                     (2, 257, 160, 2)])
def test_attention_first_queries_matches_attention(N, T, D, H):
    # Ordinary inputs: the written rows are bit for bit those of the full step.
    import torch
    rng = np.random.default_rng(N * 1000 + T)
    qkv = round_to(rng.standard_normal((N * T, 3 * D)) * 1.5, "bf16")
    dq = to_dev(qkv, "bf16")
    full = vb.attention(dq, N, T, H).view(N, T, D)
    first = vb.attention_first_queries(dq, N, T, H).view(N, T, D)
    nq = min(T, 32)
    assert torch.equal(full[:, :nq], first[:, :nq])


@pytest.mark.parametrize("N,T,D,H", [(2, 197, 128, 2), (2, 257, 160, 2), (2, 197, 96, 2)])
def test_attention_extreme_scores_fp32(N, T, D, H):
    # Head widths 64 and 80: the fp32 matrix-core kernel; 48: the VALU kernel.
    q, k, v = _case("late_key", N, T, D, H, "fp32", seed=23)
    qkv = np.concatenate([q, k, v], axis=-1).reshape(N * T, 3 * D)
    got = to_host(vb.attention(to_dev(qkv, "fp32"), N, T, H)).reshape(N, T, D)
    assert_close(got, _attention_ref(q, k, v, H), "fp32", f"attention fp32 late key D={D} H={H}")
