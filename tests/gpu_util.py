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


# Gradient bars (see assert_close_grad): normwise and elementwise, per dtype.
GRAD_NORM_TOL = {"fp32": 1e-5, "bf16": 1e-2}
GRAD_ELEM_TOL = {"fp32": 2e-4, "bf16": 5e-2}


def grad_violation(gpu, ref):
    """(max |g - o| / (rms(o) + |o|), ||g - o|| / ||o||, mean abs err)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if not np.all(np.isfinite(gpu)):
        return float("inf"), float("inf"), float("inf")
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    err = np.abs(gpu - ref)
    norm = float(np.sqrt(np.sum(err * err)) / (np.sqrt(np.sum(ref * ref)) or 1.0))
    return float((err / (rms + np.abs(ref))).max()), norm, float(err.mean())


def assert_close_grad(gpu, ref, dtype, what=""):
    """Gradient bars: ||g - o|| / ||o|| <= GRAD_NORM_TOL and
    max |g - o| / (rms(o) + |o|) <= GRAD_ELEM_TOL.

    A gradient has no unit scale of its own (a weight gradient is a sum over
    every token of the batch), so the elementwise bar is taken against the
    tensor's RMS instead of the forward bar's unit "1 +".  In bf16 every
    gradient has passed through about ten roundings to bf16 (relative error
    up to 2^-9 each) on its way from the output gradient, and the measured
    relative RMS error of the weight gradients is 0.5-0.6 %; the largest of
    n such errors is about sqrt(2 ln n) = 5.5 standard deviations for the 4M
    elements of an MLP weight, i.e. about 3 %.  Hence 5e-2 elementwise, and
    1e-2 normwise (twice the measured RMS error; a dropped or wrong term
    shows up at order 1 in both).  fp32: 2e-4 and 1e-5.
    """
    v, norm, mae = grad_violation(gpu, ref)
    bar, nbar = GRAD_ELEM_TOL[dtype], GRAD_NORM_TOL[dtype]
    print(f"  {what}: elementwise {v:.3e} (bar {bar:.0e}), normwise {norm:.3e} (bar {nbar:.0e}), "
          f"mean abs err {mae:.3e}", flush=True)
    assert norm <= nbar, f"{what}: normwise error {norm:.3e} > {nbar}"
    assert v <= bar, f"{what}: elementwise violation {v:.3e} > {bar}"
    return v, mae
