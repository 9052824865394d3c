"""Helpers for the GPU parity tests (device upload, violation ratio, tolerances)."""

import numpy as np

# Elementwise bars for |gpu - oracle| <= tol * (1 + |oracle|), per dtype.
TOL = {"fp32": 2e-4, "bf16": 3e-2}


def torch_dtype(name):
    import torch
    return {"fp32": torch.float32, "bf16": torch.bfloat16}[name]


def to_dev(a, dtype):
    """float64 array holding device-exact values -> contiguous GPU tensor (exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device="cuda", dtype=torch_dtype(dtype)).contiguous()


def to_host(t):
    import torch
    return t.detach().to(device="cpu", dtype=torch.float64).numpy()


def violation(gpu, ref):
    """max |g - o| / (1 + |o|), and the mean absolute error."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if not np.all(np.isfinite(gpu)):
        return float("inf"), float("inf")
    err = np.abs(gpu - ref)
    return float((err / (1.0 + np.abs(ref))).max()), float(err.mean())


def assert_close(gpu, ref, dtype, what="", scale=1.0):
    """Bar: TOL[dtype] * scale (scale > 1 only for stacks of blocks, see stack_scale)."""
    v, mae = violation(gpu, ref)
    bar = TOL[dtype] * scale
    print(f"  {what}: violation {v:.3e} (bar {bar:.2e}), mean abs err {mae:.3e}", flush=True)
    assert v <= bar, f"{what}: violation {v:.3e} > {bar}"
    return v, mae


def stack_scale(L):
    """Bar multiplier for L blocks in sequence: each block's rounding error is
    independent of the others', so in the residual stream they add in
    quadrature and the one-block bar grows as sqrt(L)."""
    import math
    return math.sqrt(L)


def grad_violation(gpu, ref):
    """max |g - o| / (rms(o) + |o|), and the mean absolute error."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if not np.all(np.isfinite(gpu)):
        return float("inf"), float("inf")
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    err = np.abs(gpu - ref)
    return float((err / (rms + np.abs(ref))).max()), float(err.mean())


def assert_close_grad(gpu, ref, dtype, what=""):
    """Gradient bar: TOL[dtype] * (rms(o) + |o|).

    A gradient has no unit scale of its own (a weight gradient is a sum over
    every token of the batch), so the forward bar's "1 +" -- the block
    output's unit scale -- becomes the RMS of the oracle's tensor: the bar is
    the forward's relative bar measured in the tensor's own units.
    """
    v, mae = grad_violation(gpu, ref)
    bar = TOL[dtype]
    print(f"  {what}: violation {v:.3e} (bar {bar:.2e}), mean abs err {mae:.3e}", flush=True)
    assert v <= bar, f"{what}: violation {v:.3e} > {bar}"
    return v, mae
