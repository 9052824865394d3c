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


def assert_close(gpu, ref, dtype, what=""):
    v, mae = violation(gpu, ref)
    print(f"  {what}: violation {v:.3e} (bar {TOL[dtype]:.0e}), mean abs err {mae:.3e}",
          flush=True)
    assert v <= TOL[dtype], f"{what}: violation {v:.3e} > {TOL[dtype]}"
    return v, mae
