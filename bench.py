"""Throughput of one pre-LN ViT encoder block forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit_l16]
                    [--variant plain|affine|encoder|embed|backward] [--layers L]

A step is one full block forward (vitblk_forward: the weights' packing with the
first LayerNorm's statistics, then the block's steps, 11 launches at ViT-L/16) over
one batch of synthetic inputs already resident in HBM.  Prints ONE JSON line:
tokens/s for the whole job, ms per step, the block's achieved TFLOP/s and
fraction of the bf16 dense MFMA peak, per-kernel times (each step's kernel
timed alone with HIP events on the launch stream), the roofline of the
dominant kernel, a parity check of the timed output against the float64
oracle on sampled sequences, and the oracle's own throughput on the host
cores (cpu_baseline).  ``--variant affine`` times the affine block instead
(LayerNorm gains and shifts, projection biases: vitblk_forward_affine);
``--variant encoder`` times the encoder stack (L affine blocks on pre-packed
weights, the final LayerNorm of every token and of the class tokens:
vitblk_encoder_forward), L = the model's depth unless --layers is given;
``--variant embed`` times the front end (vitblk_patch_embed: N images of
(sqrt(T-1) * P)^2 pixels, 3 channels, P = 16 for ViT-B/L and 14 for ViT-H,
with class token and position embeddings) and reports tokens/s out of it;
``--variant backward`` times the block backward (vitblk_backward: the forward
recomputed, then dx and the six weight gradients for a seeded N(0, 1) output
gradient) and checks dx on sampled sequences against the float64 backward
oracle (the weight gradients, sums over the whole batch, are checked by the
GPU tests).
"""

from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "encoder-block fwd tokens/sec + % bf16 MFMA peak, ViT-L/16 shape N=256"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector (published; counts packed FMA, which this
                            # build does not emit, so its fp32 kernels top out at half)
# Measured HBM traffic of the dominant step (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# calibrated on a plain copy); used only while the kernel source is unchanged.
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "vit_l16_mlp1_gelu_traffic.json")


def source_digest(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(step, workload):
    """Bytes per launch from the committed counter record, or None if stale."""
    try:
        with open(TRAFFIC_RECORD) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("step") != step or rec.get("workload") != workload:
        return None
    if rec.get("source_digest") != source_digest(rec.get("sources", [])):
        return None
    return rec.get("bytes_per_launch")


def block_flops(N, T, D, F):
    """Matmul FLOPs of one block: N*T*(8 D^2 + 4 D F + 4 T D)."""
    return N * T * (8 * D * D + 4 * D * F + 4 * T * D)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="vit_l16")
    ap.add_argument("--kernel-reps", type=int, default=20,
                    help="launches per step kernel in the per-kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target host time for the oracle baseline sample (0 = skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--variant", choices=["plain", "affine", "encoder", "embed", "backward"],
                    default="plain",
                    help="plain block (default), the affine variant, the encoder stack, "
                         "the front end, or the block backward")
    ap.add_argument("--layers", type=int, default=0,
                    help="encoder depth (default: 12 / 24 / 32 for ViT-B / L / H)")
    ap.add_argument("--dtype", choices=["bf16", "fp32"], default=None,
                    help="element type (default: the workload's own; fp32 runs the generic "
                         "VALU kernels, a correctness path whose speed is reported, not tuned)")
    ap.add_argument("--no-vendor-ref", action="store_true",
                    help="skip the torch.mm (hipBLASLt) reference timings of the GEMM shapes")
    ap.add_argument("--profile-step", default=None,
                    help="run only a 512 MiB copy (counter calibration) and 3 launches of this "
                         "step's kernel, for rocprofv3 --pmc; prints no JSON")
    return ap.parse_args()


def time_steps(step, steps, torch):
    """Run step() `steps` times between HIP events recorded on the launch stream
    (one before the first step and one after each): returns (mean ms per step
    over the whole run, per-step ms list, host wall seconds).  The events sit
    between the steps, so the mean is the plain end-to-end time / steps."""
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    # Python's cyclic garbage collector off while the steps are enqueued (as
    # timeit does): a collection pause on the host would otherwise show up as
    # an idle GPU gap wherever the host is only a few short steps ahead.
    gc_was_on = gc.isenabled()
    gc.disable()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record(s)
    for i in range(steps):
        step()
        ev[i + 1].record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    if gc_was_on:
        gc.enable()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return ev[0].elapsed_time(ev[steps]) / steps, per, t_wall


def step_stats(per):
    """Median, minimum and maximum of the per-step times (ms)."""
    a = np.asarray(per, dtype=np.float64)
    return {"median": round(float(np.median(a)), 5), "min": round(float(a.min()), 5),
            "max": round(float(a.max()), 5)}


_QUEUE_AHEAD = {}


def time_launches(fn, reps, torch):
    """Average duration of fn() (one kernel launch) over reps, HIP events on the launch stream.

    A few untimed products run first, long enough for the host to enqueue
    every timed launch behind them: a launch shorter than its host-side call
    (argument checks, marshalling) would otherwise be timed at the host's rate.
    """
    s = torch.cuda.current_stream()
    fn()
    if "a" not in _QUEUE_AHEAD:
        _QUEUE_AHEAD["a"] = torch.ones((4096, 4096), dtype=torch.bfloat16, device="cuda")
        _QUEUE_AHEAD["c"] = torch.empty_like(_QUEUE_AHEAD["a"])
    qa, qc = _QUEUE_AHEAD["a"], _QUEUE_AHEAD["c"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    for _ in range(2 + reps // 4):  # about 0.15 ms each
        torch.mm(qa, qa, out=qc)
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            return int(info[0]["num_threads"]), info[0].get("internal_api", "blas")
    except Exception:
        pass
    return len(os.sched_getaffinity(0)), "unknown"


def cpu_baseline(ref_fn, w, target_s, got_out, layers=1):
    """Time the float64 oracle (ref_fn(sequence indices) -> (n, T, D)) on a bounded
    sample of sequences; also check the GPU output's parity there."""
    t0 = time.perf_counter()
    ref0 = ref_fn([0])
    t1 = time.perf_counter() - t0
    n = int(max(1, min(w.N, math.floor(target_s / max(t1, 1e-6)))))
    seqs = sorted(set(np.linspace(0, w.N - 1, n).astype(int).tolist()))
    t0 = time.perf_counter()
    ref = ref_fn(seqs)
    dt = time.perf_counter() - t0
    got = got_out[seqs]
    err = np.abs(got - ref)
    viol = float((err / (1.0 + np.abs(ref))).max())
    threads, api = blas_threads()
    del ref0
    return ({"value": len(seqs) * w.T / dt, "unit": "tokens/s", "cores": threads,
             "kind": "oracle",
             "sample": f"{len(seqs)} of {w.N} sequences ({len(seqs) * w.T} tokens), float64 "
                       f"NumPy ({api} BLAS, {threads} threads), {dt:.1f} s",
             "host_cpus": len(os.sched_getaffinity(0))},
            {"violation": viol, "bar": (3e-2 if w.dtype == "bf16" else 2e-4) * math.sqrt(layers),
             "mean_abs_err": float(err.mean()), "sequences": len(seqs)})


def bench_embed(a, w, torch, vb):
    """The front end alone: images -> tokens (vitblk_patch_embed)."""
    from vision_transformer_encoder_amd.inputs import round_to
    import oracle
    P = 14 if w.name == "vit_h14" else 16
    side = int(round(math.sqrt(w.T - 1))) * P
    B, C, D = w.N, 3, w.D
    K = P * P * C
    rng = np.random.default_rng([a.seed, 3])
    img = round_to(rng.standard_normal((B, C, side, side)), w.dtype)
    wp = round_to(rng.standard_normal((K, D)) / math.sqrt(K), w.dtype)
    bp = round_to(0.1 * rng.standard_normal(D), w.dtype)
    cls = round_to(0.02 * rng.standard_normal(D), w.dtype)
    pos = round_to(0.02 * rng.standard_normal((w.T, D)), w.dtype)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    dev = torch.device("cuda:0")
    to_g = lambda v: torch.from_numpy(v.astype(np.float32)).to(dev, tdt)  # noqa: E731
    gi, gw, gb, gc, gpos = map(to_g, (img, wp, bp, cls, pos))
    out = torch.empty((B, w.T, D), dtype=tdt, device=dev)
    ws = torch.empty(vb.patch_embed_workspace_bytes(B, C, side, side, P, D, tdt),
                     dtype=torch.uint8, device=dev)

    def step():
        vb.patch_embed(gi, gw, P, gb, gc, gpos, out=out, workspace=ws)

    for _ in range(a.warmup):
        step()
    ms, per_step, t_wall = time_steps(step, a.steps, torch)
    got = out.to("cpu", torch.float64).numpy()
    # The embedding GEMM alone, on the same shapes: the dominant kernel.
    Kp = (K + 63) // 64 * 64
    pm = torch.zeros((B * (w.T - 1), Kp), dtype=tdt, device=dev)
    wt = torch.zeros((D, Kp), dtype=tdt, device=dev)
    emb = torch.empty((B * (w.T - 1), D), dtype=tdt, device=dev)
    gemm = lambda: vb.linear(pm, wt, vb.EPI_NONE, bias=gb, out=emb)  # noqa: E731
    gms = time_launches(gemm, a.kernel_reps, torch)
    gflop = 2 * B * (w.T - 1) * Kp * D
    es = 2 if w.dtype == "bf16" else 4
    io_bytes = (B * C * side * side + K * D + B * w.T * D) * es
    ach = gflop / (gms * 1e-3) / 1e12
    res = {
        "metric": f"front-end (patch embedding) tokens/sec, {w.name} shape N={w.N}",
        "value": round(B * w.T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) pixels, N(0,1/fan_in) W_patch)",
        "config": {"workload": w.name, "images": B, "image_side": side, "channels": C,
                   "patch": P, "D": D, "tokens_per_image": w.T, "variant": "embed"},
        "step_ms": step_stats(per_step),
        "wall_s_timed": round(t_wall, 3),
        "io_gbs": round(io_bytes / (ms * 1e-3) / 1e9, 1),
        "kernels": {"embed_gemm": {"ms": round(gms, 5), "bound": "mfma",
                                   "tflops": round(ach, 2)}},
        "roofline": {"kernel": "embed_gemm", "bound": "mfma", "achieved": round(ach, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                     "work_per_launch": f"{gflop / 1e9:.2f} GFLOP"},
    }
    if a.cpu_seconds > 0:
        def ref_fn(seqs):
            return oracle.patch_embed(img[seqs], wp, P, bp, cls, pos)
        cb, par = cpu_baseline(ref_fn, w, a.cpu_seconds, got)
        res["cpu_baseline"] = cb
        res["parity"] = par
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def backward_flops(N, T, D, F):
    """Matmul FLOPs of one block backward with the forward recomputed:
    the forward's N*T*(8 D^2 + 4 D F + 4 T D), then twice the projections'
    (input and weight gradients) and four attention products (dV, dP, dQ, dK)."""
    return N * T * (24 * D * D + 12 * D * F + 12 * T * D)


def bench_backward(a, w, torch, vb):
    """The block backward: x, weights and dL/d(out) -> dx and the six weight gradients."""
    import oracle
    from vision_transformer_encoder_amd.inputs import make_block_inputs, make_dout
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    dev = torch.device("cuda:0")
    WN = ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]
    inp = make_block_inputs(w.N, w.T, w.D, w.F, w.dtype, seed=a.seed)
    dout = make_dout(w.N, w.T, w.D, w.dtype, seed=a.seed)
    to_g = lambda v: torch.from_numpy(v.astype(np.float32)).to(dev, tdt)  # noqa: E731
    g = {k: to_g(v) for k, v in inp.items()}
    gd = to_g(dout)
    ws = torch.empty(vb.backward_workspace_bytes(w.N, w.T, w.D, w.F, w.H, tdt),
                     dtype=torch.uint8, device=dev)
    grads = vb.backward(g["x"], *(g[k] for k in WN), gd, w.H, w.eps, workspace=ws)

    def step():
        vb.backward(g["x"], *(g[k] for k in WN), gd, w.H, w.eps, grads=grads, workspace=ws)

    for _ in range(a.warmup):
        step()
    ms, per_step, t_wall = time_steps(step, a.steps, torch)
    got_dx = grads["dx"].to("cpu", torch.float64).numpy()

    # The backward's steps alone, on the same shapes and realistic operands.
    M, D, F = w.M, w.D, w.F
    es = 2 if w.dtype == "bf16" else 4
    x2, dout2 = g["x"].view(M, D), gd.view(M, D)
    packed = vb.pack_weights(*(g[k] for k in WN))
    wqkv_t, wo_t, w1_t, w2_t = vb.packed_views(packed, D, F, tdt)
    xn = vb.layernorm(x2, w.eps)
    qkv = vb.qkv_projection(xn, wqkv_t)
    att = vb.attention(qkv, w.N, w.T, w.H)
    y = vb.linear(att, wo_t, vb.EPI_RESIDUAL, residual=x2)
    yn = vb.layernorm(y, w.eps)
    z = vb.linear(yn, w1_t, vb.EPI_NONE)
    hid = vb.linear(yn, w1_t, vb.EPI_GELU)
    dz = vb.linear(dout2, g["w_mlp2"], vb.EPI_GELU_GRAD, residual=z)
    dyn = vb.linear(dz, g["w_mlp1"], vb.EPI_NONE)
    dy = vb.layernorm_backward(y, dyn, w.eps, residual=dout2)
    datt = vb.linear(dy, g["w_o"], vb.EPI_NONE)
    dqkv = vb.attention_backward(qkv, datt, w.N, w.T, w.H)
    wcat = torch.cat([g["w_q"], g["w_k"], g["w_v"]], dim=1).contiguous()
    dxn = vb.linear(dqkv, wcat, vb.EPI_NONE)
    outs = {k: torch.empty_like(v) for k, v in (("dz", dz), ("dyn", dyn), ("dy", dy),
                                                ("datt", datt), ("dqkv", dqkv), ("dxn", dxn))}
    wouts = {"dw_mlp2": torch.empty((F, D), dtype=tdt, device=dev),
             "dw_mlp1": torch.empty((D, F), dtype=tdt, device=dev),
             "dw_o": torch.empty((D, D), dtype=tdt, device=dev),
             "dw_qkv": torch.empty((D, 3 * D), dtype=tdt, device=dev)}
    wws = torch.empty(max(vb.weight_grad_workspace_bytes(M, i, j) for i, j in
                          ((F, D), (D, F), (D, D), (D, 3 * D))), dtype=torch.uint8, device=dev)
    aws = torch.empty(vb.attention_backward_workspace_bytes(w.N, w.T, D, w.H), dtype=torch.uint8,
                      device=dev)
    T_ = w.T
    kern = {
        "dw_mlp2": (lambda: vb.weight_grad(hid, dout2, out=wouts["dw_mlp2"], workspace=wws),
                    "mfma", 2 * M * F * D),
        "dz_gemm_gelu_grad": (lambda: vb.linear(dout2, g["w_mlp2"], vb.EPI_GELU_GRAD,
                                                residual=z, out=outs["dz"]), "mfma",
                              2 * M * D * F),
        "dw_mlp1": (lambda: vb.weight_grad(yn, dz, out=wouts["dw_mlp1"], workspace=wws), "mfma",
                    2 * M * D * F),
        "dyn_gemm": (lambda: vb.linear(dz, g["w_mlp1"], vb.EPI_NONE, out=outs["dyn"]), "mfma",
                     2 * M * F * D),
        "ln2_backward": (lambda: vb.layernorm_backward(y, dyn, w.eps, residual=dout2,
                                                       out=outs["dy"]), "hbm", 4 * M * D * es),
        "dw_o": (lambda: vb.weight_grad(att, dy, out=wouts["dw_o"], workspace=wws), "mfma",
                 2 * M * D * D),
        "datt_gemm": (lambda: vb.linear(dy, g["w_o"], vb.EPI_NONE, out=outs["datt"]), "mfma",
                      2 * M * D * D),
        "attention_backward": (lambda: vb.attention_backward(qkv, datt, w.N, T_, w.H,
                                                             out=outs["dqkv"], workspace=aws),
                               "mfma", 8 * w.N * T_ * T_ * D),
        "dw_qkv": (lambda: vb.weight_grad(xn, dqkv, out=wouts["dw_qkv"], workspace=wws), "mfma",
                   2 * M * D * 3 * D),
        "dxn_gemm": (lambda: vb.linear(dqkv, wcat, vb.EPI_NONE, out=outs["dxn"]), "mfma",
                     2 * M * 3 * D * D),
        "ln1_backward": (lambda: vb.layernorm_backward(x2, dxn, w.eps, residual=dy,
                                                       out=outs["dy"]), "hbm", 4 * M * D * es),
    }
    per = {}
    for name, (fn, bound, work) in kern.items():
        kms = time_launches(fn, a.kernel_reps, torch)
        rate = work / (kms * 1e-3)
        per[name] = {"ms": round(kms, 5), "bound": bound,
                     ("tflops" if bound == "mfma" else "gbs"):
                     round(rate / (1e12 if bound == "mfma" else 1e9), 2)}
        if name == "attention":  # both rates: its bound moves with T
            per[name]["tflops"] = round(att_flops / (kms * 1e-3) / 1e12, 2)
            per[name]["gbs"] = round(att_bytes / (kms * 1e-3) / 1e9, 2)
    dom = max(per, key=lambda k: per[k]["ms"])
    fn, bound, work = kern[dom]
    dms = per[dom]["ms"]
    if bound == "mfma":
        ach = work / (dms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": None,
                "work_per_launch": f"{work / 1e9:.2f} GFLOP"}
    else:
        ach = work / (dms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None,
                "work_per_launch": f"{work / 1e6:.1f} MB"}
    flops = backward_flops(w.N, w.T, w.D, w.F)
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": f"encoder-block backward tokens/sec (forward recomputed; dx and the six "
                  f"weight gradients), {w.name} shape N={w.N}",
        "value": round(M / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens and output gradient, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "N": w.N, "T": w.T, "D": w.D, "H": w.H, "F": w.F,
                   "eps": w.eps, "global_batch": w.N, "seq_len": w.T, "parallelism": "none",
                   "variant": "backward"},
        "block_tflops": round(tflops, 2),
        "block_frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "step_ms": step_stats(per_step),
        "wall_s_timed": round(t_wall, 3),
        "kernels": per,
        "roofline": roof,
    }
    if a.cpu_seconds > 0:
        def ref_fn(seqs):
            return oracle.vit_block_backward(inp["x"][seqs], *(inp[k] for k in WN), dout[seqs],
                                             w.H, w.eps, chunk=1)["dx"]
        cb, par = cpu_baseline(ref_fn, w, a.cpu_seconds, got_dx)
        par["checked"] = "dx"
        res["cpu_baseline"] = cb
        res["parity"] = par
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path "
              f"(--gpus {a.gpus} requested). Under data parallelism each GPU would run "
              "this same block on its own share of the sequences.", file=sys.stderr)
        sys.exit(2)
    import torch

    import vision_transformer_encoder_amd as vb
    from vision_transformer_encoder_amd.inputs import (WORKLOADS, make_affine_params,
                                                       make_block_inputs)

    if a.profile_step:  # counters only: one untimed block, then the step alone
        a.warmup, a.steps, a.cpu_seconds = 0, 1, 0
    w = WORKLOADS[a.workload]
    if a.dtype and a.dtype != w.dtype:
        # The same shapes in another element type (fp32: the generic VALU kernels).
        w = w.with_(dtype=a.dtype)
    if a.variant == "embed":
        torch.cuda.set_device(torch.device("cuda:0"))
        return bench_embed(a, w, torch, vb)
    if a.variant == "backward":
        torch.cuda.set_device(torch.device("cuda:0"))
        return bench_backward(a, w, torch, vb)
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16}[w.dtype]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_block_inputs(w.N, w.T, w.D, w.F, w.dtype, seed=a.seed)
    g = {k: torch.from_numpy(v.astype(np.float32)).to(dev, tdt) for k, v in inp.items()}
    out = torch.empty_like(g["x"])
    ws = torch.empty(vb.workspace_bytes(w.N, w.T, w.D, w.F, w.H, tdt), dtype=torch.uint8,
                     device=dev)
    encoder = a.variant == "encoder"
    affine = a.variant in ("affine", "encoder")
    prm = make_affine_params(w.D, w.F, w.dtype, seed=a.seed) if affine else None
    gp = ({k: torch.from_numpy(v.astype(np.float32)).to(dev, tdt) for k, v in prm.items()}
          if affine else {})
    WN = ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]
    L = 1
    if encoder:
        L = a.layers or {"vit_b16": 12, "vit_l16": 24, "vit_h14": 32}.get(w.name, 12)
        # Block 0 uses the block inputs' weights; block l > 0 draws its own.
        layers = [dict({k: inp[k] for k in WN}, params=prm)]
        for l in range(1, L):
            li = make_block_inputs(1, 1, w.D, w.F, w.dtype, seed=a.seed * 1000 + l)
            layers.append(dict({k: li[k] for k in WN},
                               params=make_affine_params(w.D, w.F, w.dtype,
                                                         seed=a.seed * 1000 + l)))
        to_g = lambda v: torch.from_numpy(v.astype(np.float32)).to(dev, tdt)  # noqa: E731
        enc_packed = [vb.pack_weights(*(to_g(lay[k]) for k in WN)) for lay in layers]
        enc_params = [{k: to_g(v) for k, v in lay["params"].items()} for lay in layers]
        frng = np.random.default_rng([a.seed, 2])
        from vision_transformer_encoder_amd.inputs import round_to
        fgb = (round_to(1.0 + 0.1 * frng.standard_normal(w.D), w.dtype),
               round_to(0.1 * frng.standard_normal(w.D), w.dtype))
        fg, fb = to_g(fgb[0]), to_g(fgb[1])
        cls = torch.empty((w.N, w.D), dtype=tdt, device=dev)
        ws_enc = torch.empty(vb.encoder_workspace_bytes(w.N, w.T, w.D, w.F, w.H, tdt),
                             dtype=torch.uint8, device=dev)

    def step():
        if encoder:
            vb.encoder_forward(g["x"], enc_packed, w.F, w.H, w.eps, params=enc_params,
                               final_gamma=fg, final_beta=fb, out=out, cls_out=cls,
                               workspace=ws_enc)
        elif affine:
            vb.forward_affine(g["x"], g["w_q"], g["w_k"], g["w_v"], g["w_o"], g["w_mlp1"],
                              g["w_mlp2"], w.H, w.eps, params=gp, out=out, workspace=ws)
        else:
            vb.forward(g["x"], g["w_q"], g["w_k"], g["w_v"], g["w_o"], g["w_mlp1"],
                       g["w_mlp2"], w.H, w.eps, out=out, workspace=ws)

    for _ in range(a.warmup):
        step()
    ms, per_step, t_wall = time_steps(step, a.steps, torch)
    got = out.to("cpu", torch.float64).numpy()
    cls_only = None
    if encoder:
        # The same stack asked for the class tokens only: its last block then
        # computes just their rows.  Timed only after its output is checked
        # against the class tokens of the full run (the same values to within
        # the stack's bar; its smaller products may sum K in another order).
        cls_full = cls.to("cpu", torch.float64).numpy()
        cls_only_out = torch.empty_like(cls)

        def cls_step():
            vb.encoder_forward(g["x"], enc_packed, w.F, w.H, w.eps, params=enc_params,
                               final_gamma=fg, final_beta=fb, want_tokens=False,
                               cls_out=cls_only_out, workspace=ws_enc)
        cls_step()
        torch.cuda.synchronize()
        got_cls = cls_only_out.to("cpu", torch.float64).numpy()
        dev_ratio = float((np.abs(got_cls - cls_full) / (1.0 + np.abs(cls_full))).max())
        bar = 3e-2 * math.sqrt(L)
        cls_only = {"agrees_with_full_run": dev_ratio, "bar": bar}
        if np.all(np.isfinite(got_cls)) and dev_ratio <= bar:
            cms, cper, _ = time_steps(cls_step, a.steps, torch)
            cls_only.update({"ms_per_step": round(cms, 5), "step_ms": step_stats(cper)})

    # Each step's kernel alone, on the same shapes (separate buffers per step).
    M, D, F = w.M, w.D, w.F
    packed = vb.pack_weights(g["w_q"], g["w_k"], g["w_v"], g["w_o"], g["w_mlp1"], g["w_mlp2"])
    wqkv_t, wo_t, w1_t, w2_t = vb.packed_views(packed, D, F, tdt)
    x2 = g["x"].view(M, D)
    xn = torch.empty_like(x2)
    qkv = torch.empty((M, 3 * D), dtype=tdt, device=dev)
    att = torch.empty_like(x2)
    y = torch.empty_like(x2)
    yn = torch.empty_like(x2)
    hid = torch.empty((M, F), dtype=tdt, device=dev)
    o2 = torch.empty_like(x2)
    # The affine variant's steps: LN with gain/shift, GEMMs with bias (the
    # fused QKV bias as one [3D] vector here, the same values).
    gq = gp.get
    bqkv = torch.cat([gp["b_q"], gp["b_k"], gp["b_v"]]) if affine else None
    es = 2 if w.dtype == "bf16" else 4
    wbytes = (4 * D * D + 2 * D * F) * es
    # The packing step also sums the columns of [w_q | w_k | w_v] and w_mlp1.
    pack_bytes = 2 * wbytes + (3 * D * D + D * F) * es + (3 * D + F) * 4
    kern = {
        "pack_weights": (lambda: vb.pack_weights(g["w_q"], g["w_k"], g["w_v"], g["w_o"],
                                                 g["w_mlp1"], g["w_mlp2"], packed=packed),
                         "hbm", pack_bytes),
    }
    if w.dtype != "bf16":
        kern.update({
            "ln1": (lambda: vb.layernorm(x2, w.eps, gamma=gq("ln1_gamma"), beta=gq("ln1_beta"),
                                         out=xn), "hbm", 2 * M * D * es),
            "qkv_gemm": ((lambda: vb.linear(xn, wqkv_t, vb.EPI_NONE, bias=bqkv, out=qkv))
                         if affine else (lambda: vb.qkv_projection(xn, wqkv_t, out=qkv)),
                         "mfma", 2 * M * D * 3 * D),
        })
    else:
        # bf16: each LayerNorm is folded into the next product (row
        # statistics, then rstd (x @ W - mean colsum) in the product), as the
        # block does; with a gain and shift the product takes the fold's
        # scaled weight copy, its column sums and bias + beta @ W (one launch
        # per call, the fold step below).
        cs_qkv, cs_1 = vb.packed_col_sums(packed, D, F, tdt)
        st1 = torch.empty((M, 2), dtype=torch.float32, device=dev)
        st2 = torch.empty_like(st1)
        kern["ln1_stats"] = (lambda: vb.row_stats(x2, w.eps, out=st1), "hbm", M * D * es + M * 8)
        if affine:
            f1 = vb.affine_fold(wqkv_t, gq("ln1_gamma"), gq("ln1_beta"), bqkv)
            f2 = vb.affine_fold(w1_t, gq("ln2_gamma"), gq("ln2_beta"), gq("b_mlp1"))
            fold_bytes = lambda n: 2 * n * D * es + 2 * D * es + n * (4 + 2 * es)  # noqa: E731
            kern.update({
                "ln1_fold": (lambda: vb.affine_fold(wqkv_t, gq("ln1_gamma"), gq("ln1_beta"), bqkv,
                                                    out=f1), "hbm", fold_bytes(3 * D)),
                "qkv_gemm": (lambda: vb.linear_normed(x2, f1[0], f1[1], st1, vb.EPI_NONE,
                                                      bias=f1[2], out=qkv),
                             "mfma", 2 * M * D * 3 * D),
            })
        else:
            kern["qkv_gemm"] = (lambda: vb.linear_normed(x2, wqkv_t, cs_qkv, st1, vb.EPI_NONE,
                                                         out=qkv), "mfma", 2 * M * D * 3 * D)
    # Attention's bound depends on T: 4 N T^2 D FLOP against 4 M D elements
    # (Q, K, V read, O written), an intensity of about T / es FLOP per byte,
    # below the ridge (peak FLOP/s / peak bytes/s) at ViT sequence lengths.
    att_flops, att_bytes = 4 * w.N * w.T * w.T * D, 4 * M * D * es
    att_peak, att_unit = ((PEAK_BF16_TFLOPS, "mfma") if w.dtype == "bf16"
                          else (PEAK_FP32_TFLOPS, "alu"))
    att_bound = ("hbm" if att_flops / att_bytes < att_peak * 1e12 / (PEAK_HBM_GBS * 1e9)
                 else att_unit)
    kern["attention"] = (lambda: vb.attention(qkv, w.N, w.T, w.H, out=att), att_bound,
                         att_bytes if att_bound == "hbm" else att_flops)
    if w.dtype != "bf16":
        kern.update({
            "oproj_residual": (lambda: vb.linear(att, wo_t, vb.EPI_RESIDUAL, residual=x2,
                                                 bias=gq("b_o"), out=y), "mfma", 2 * M * D * D),
            "ln2": (lambda: vb.layernorm(y, w.eps, gamma=gq("ln2_gamma"), beta=gq("ln2_beta"),
                                         out=yn), "hbm", 2 * M * D * es),
            "mlp1_gelu": (lambda: vb.linear(yn, w1_t, vb.EPI_GELU, bias=gq("b_mlp1"), out=hid),
                          "mfma", 2 * M * D * F),
        })
    else:
        # The output projection writes the LN2 row statistics' partials from
        # its epilogue and one small kernel combines them, as in the block
        # (this step entry takes no bias: the affine block's b_o starts in the
        # accumulators and costs no epilogue work).
        ows = torch.empty(vb.linear_residual_row_stats_workspace_bytes(M, D), dtype=torch.uint8,
                          device=dev)
        kern["oproj_residual_ln2_stats"] = (lambda: vb.linear_residual_row_stats(
            att, wo_t, x2, w.eps, out=y, stats=st2, workspace=ows), "mfma", 2 * M * D * D)
        if affine:
            kern.update({
                "ln2_fold": (lambda: vb.affine_fold(w1_t, gq("ln2_gamma"), gq("ln2_beta"),
                                                    gq("b_mlp1"), out=f2), "hbm", fold_bytes(F)),
                "mlp1_gelu": (lambda: vb.linear_normed(y, f2[0], f2[1], st2, vb.EPI_GELU,
                                                       bias=f2[2], out=hid),
                              "mfma", 2 * M * D * F),
            })
        else:
            kern["mlp1_gelu"] = (lambda: vb.linear_normed(y, w1_t, cs_1, st2, vb.EPI_GELU,
                                                          out=hid), "mfma", 2 * M * D * F)
    kern["mlp2_residual"] = (lambda: vb.linear(hid, w2_t, vb.EPI_RESIDUAL, residual=y,
                                               bias=gq("b_mlp2"), out=o2), "mfma", 2 * M * F * D)
    for name in [k for k in kern if k not in ("pack_weights", "mlp2_residual")]:
        kern[name][0]()  # realistic operands for every step, in block order
    if a.profile_step:
        x_copy = torch.empty(256 * 1024 * 1024, dtype=torch.bfloat16, device=dev).fill_(1.0)
        y_copy = torch.empty_like(x_copy)
        for _ in range(3):
            y_copy.copy_(x_copy)  # 512 MiB read + 512 MiB written, for calibration
        torch.cuda.synchronize()
        fn = kern[a.profile_step][0]
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        print(f"profiled {a.profile_step}", file=sys.stderr)
        return

    if w.dtype == "fp32":
        # fp32 products run on the VALU (generic kernels).
        kern = {k: (fn, "alu" if bound == "mfma" else bound, work)
                for k, (fn, bound, work) in kern.items()}
    per = {}
    for name, (fn, bound, work) in kern.items():
        kms = time_launches(fn, a.kernel_reps, torch)
        rate = work / (kms * 1e-3)
        per[name] = {"ms": round(kms, 5), "bound": bound,
                     ("gbs" if bound == "hbm" else "tflops"):
                     round(rate / (1e9 if bound == "hbm" else 1e12), 2)}
        if name == "attention":  # both rates: its bound moves with T
            per[name]["tflops"] = round(att_flops / (kms * 1e-3) / 1e12, 2)
            per[name]["gbs"] = round(att_bytes / (kms * 1e-3) / 1e9, 2)
    vendor = None
    if w.dtype == "bf16" and not a.no_vendor_ref:
        # Reference only, never on the product path: torch.mm (hipBLASLt) on
        # operands of the four products' shapes, plain products without the
        # fused epilogues -- what the vendor library reaches on these shapes.
        vendor = {}
        for vname, (kk, nn) in {"qkv": (D, 3 * D), "oproj": (D, D), "mlp1": (D, F),
                                "mlp2": (F, D)}.items():
            va = torch.randn(M, kk, device=dev).to(tdt)
            vw = (torch.randn(kk, nn, device=dev) / math.sqrt(kk)).to(tdt).contiguous()
            vo = torch.empty(M, nn, device=dev, dtype=tdt)
            vms = time_launches(lambda: torch.mm(va, vw, out=vo), a.kernel_reps, torch)
            vendor[vname] = {"ms": round(vms, 5),
                             "tflops": round(2 * M * kk * nn / (vms * 1e-3) / 1e12, 2)}
            del va, vw, vo
    dom = max(per, key=lambda k: per[k]["ms"])
    fn, bound, work = kern[dom]
    dms = per[dom]["ms"]
    if bound in ("mfma", "alu"):
        ach = work / (dms * 1e-3) / 1e12
        pk = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_FP32_TFLOPS
        roof = {"kernel": dom, "bound": bound, "achieved": round(ach, 2),
                "peak": pk, "unit": "TFLOP/s",
                "frac": round(ach / pk, 4),
                "traffic": (None if affine or w.dtype != "bf16"
                            else recorded_traffic(dom, w.name)),
                "work_per_launch": f"{work / 1e9:.2f} GFLOP"}
    else:
        ach = work / (dms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4),
                "traffic": None if affine else recorded_traffic(dom, w.name),
                "work_per_launch": f"{work / 1e6:.1f} MB"}

    flops = L * block_flops(w.N, w.T, w.D, w.F)
    tflops = flops / (ms * 1e-3) / 1e12
    res = {
        "metric": (f"encoder-stack fwd tokens/sec ({L} blocks + final LN), {w.name} shape N={w.N}"
                   if encoder else METRIC if w.dtype == "bf16" and w.name == "vit_l16" and
                   not affine else f"encoder-block fwd tokens/sec, {w.name} shape N={w.N}, "
                   f"{w.dtype}{', affine' if affine else ''}"),
        "value": round(w.M / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,1/fan_in) weights)",
        "config": {"workload": w.name, "N": w.N, "T": w.T, "D": w.D, "H": w.H, "F": w.F,
                   "eps": w.eps, "global_batch": w.N, "seq_len": w.T, "parallelism": "none",
                   **({"variant": a.variant} if a.variant != "plain" else {}),
                   **({"layers": L} if encoder else {})},
        "block_tflops": round(tflops, 2),
        "block_frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "step_ms": step_stats(per_step),
        "wall_s_timed": round(t_wall, 3),
        "kernels": per,
        "roofline": roof,
    }
    if w.dtype == "fp32":
        res["block_frac_fp32_vector_peak"] = round(tflops / PEAK_FP32_TFLOPS, 4)
    if cls_only is not None:
        res["cls_only"] = cls_only
    if vendor is not None:
        res["vendor_gemm_ref"] = vendor
    if a.cpu_seconds > 0:
        import oracle
        if encoder:
            ref_fn = lambda seqs: oracle.encoder(inp["x"][seqs], layers, w.H, w.eps,  # noqa: E731
                                                 fgb[0], fgb[1])[0]
        else:
            ref_fn = lambda seqs: oracle.vit_block(  # noqa: E731
                inp["x"][seqs], *(inp[k] for k in WN), w.H, w.eps, params=prm)
        # A stack's bar: the one-block bar times sqrt(L) (independent per-block rounding).
        cb, par = cpu_baseline(ref_fn, w, a.cpu_seconds, got, layers=L)
        res["cpu_baseline"] = cb
        res["parity"] = par
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
