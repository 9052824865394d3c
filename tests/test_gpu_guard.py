"""Guard bands and poisoned workspaces: the entry points write only their outputs
and read only what they wrote.

crackedaicode.com "ViT Encoder Block", "Inputs and output": the block returns a
new tensor and leaves its inputs unchanged.  Each case below runs an entry
point with
* the output (and the workspace) inside a larger buffer whose bands before
  and after hold a canary pattern, which must survive the call;
* the workspace filled first with NaN bit patterns, then with zeros: a
  kernel that read a region nobody wrote (a stale split-K partial, a row
  outside the class-token rows) would carry the NaN into the output, or make
  the two outputs differ; the outputs must be finite and bit-identical;
* copies of the inputs, which must be unchanged afterwards.
The shapes cover the split-K tail of the residual products (N = 85 at
ViT-L/16 width: fp32 partials in workspace regions that are dead at that
point) and the class-token-only last block of the encoder stack, whose
attention output is valid on the class-token rows only.
"""

import numpy as np
import pytest

import oracle
import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd.inputs import (WORKLOADS, make_affine_params,
                                                   make_block_inputs)

from gpu_util import assert_close, stack_scale, to_dev, to_host

pytestmark = pytest.mark.gpu

WEIGHTS = ["w_q", "w_k", "w_v", "w_o", "w_mlp1", "w_mlp2"]
GUARD = 4096          # elements (bf16) or bytes (workspace) per band
CANARY = 0x5A5A       # int16 pattern of the output bands (a finite bf16)
WS_CANARY = 0xA5      # byte pattern of the workspace bands


def _guarded(shape, dtype):
    """(buffer, view): a tensor of `shape` with canary bands of GUARD elements."""
    import torch
    n = int(np.prod(shape))
    buf = torch.empty(GUARD + n + GUARD, dtype=dtype, device="cuda")
    buf.view(torch.int16).fill_(CANARY - 0x10000 if CANARY > 0x7FFF else CANARY)
    return buf, buf[GUARD:GUARD + n].view(*shape)


def _bands_intact(buf, n):
    import torch
    raw = buf.view(torch.int16)
    want = CANARY - 0x10000 if CANARY > 0x7FFF else CANARY
    return bool((raw[:GUARD] == want).all()) and bool((raw[GUARD + n:] == want).all())


def _guarded_ws(nbytes):
    import torch
    buf = torch.empty(GUARD + nbytes + GUARD, dtype=torch.uint8, device="cuda")
    buf.fill_(WS_CANARY)
    return buf, buf[GUARD:GUARD + nbytes]


def _ws_bands_intact(buf, nbytes):
    return bool((buf[:GUARD] == WS_CANARY).all()) and bool((buf[GUARD + nbytes:] == WS_CANARY).all())


def _poison(ws, nan):
    # 0xFF bytes are a NaN in bf16 and fp32 alike.
    ws.fill_(0xFF if nan else 0)


def _run_twice(call, out_shape, ws_bytes, inputs):
    """call(out, ws) with a NaN-filled and then a zero-filled workspace; returns
    the first output after checking bands, finiteness, bit-identity and
    untouched inputs."""
    import torch
    before = [t.clone() for t in inputs]
    outs = []
    for nan in (True, False):
        obuf, out = _guarded(out_shape, torch.bfloat16)
        wbuf, ws = _guarded_ws(ws_bytes)
        _poison(ws, nan)
        call(out, ws)
        torch.cuda.synchronize()
        assert _bands_intact(obuf, out.numel()), "output guard band overwritten"
        assert _ws_bands_intact(wbuf, ws_bytes), "workspace guard band overwritten"
        assert bool(torch.isfinite(out.float()).all()), "non-finite output"
        outs.append(out.clone())
    assert torch.equal(outs[0], outs[1]), "output depends on the workspace's prior contents"
    for a, b in zip(before, inputs):
        assert torch.equal(a, b), "an input was modified"
    return outs[0]


@pytest.mark.parametrize("N,seqs", [(85, [0, 83, 84]), (256, [0, 255])])
@pytest.mark.parametrize("affine", [False, True])
def test_block_guarded_and_poisoned(N, seqs, affine):
    # ViT-L/16 width; N = 85 puts the last 361 rows in the residual products'
    # split-K tail, N = 256 is the full workload.
    w = WORKLOADS["vit_l16"]
    inp = make_block_inputs(N, w.T, w.D, w.F, "bf16", seed=17)
    dev = {k: to_dev(v, "bf16") for k, v in inp.items()}
    prm = make_affine_params(w.D, w.F, "bf16", seed=17) if affine else None
    dp = {k: to_dev(v, "bf16") for k, v in prm.items()} if affine else None
    ws_bytes = vb.workspace_bytes(N, w.T, w.D, w.F, w.H, vb.VITBLK_BF16)

    def call(out, ws):
        if affine:
            vb.forward_affine(dev["x"], *(dev[k] for k in WEIGHTS), w.H, w.eps, params=dp,
                              out=out, workspace=ws)
        else:
            vb.forward(dev["x"], *(dev[k] for k in WEIGHTS), w.H, w.eps, out=out, workspace=ws)

    inputs = list(dev.values()) + (list(dp.values()) if affine else [])
    out = _run_twice(call, (N, w.T, w.D), ws_bytes, inputs)
    ref = oracle.vit_block(inp["x"][seqs], *(inp[k] for k in WEIGHTS), w.H, w.eps, params=prm)
    assert_close(to_host(out)[seqs], ref, "bf16", f"guarded block N={N} affine={affine}")


@pytest.mark.parametrize("affine", [False, True])
def test_encoder_class_tokens_only_guarded_and_poisoned(affine):
    # The class-token-only last block: attention rows past each sequence's
    # first query tile are never written and must never be read.
    N, T, D, H, F, L = 6, 197, 256, 4, 1024, 2
    x = make_block_inputs(N, T, D, F, "bf16", seed=18)["x"]
    layers = []
    for l in range(L):
        li = make_block_inputs(1, 1, D, F, "bf16", seed=1800 + l)
        lay = {k: li[k] for k in WEIGHTS}
        if affine:
            lay["params"] = make_affine_params(D, F, "bf16", seed=1800 + l)
        layers.append(lay)
    dx = to_dev(x, "bf16")
    packed = [vb.pack_weights(*(to_dev(lay[k], "bf16") for k in WEIGHTS)) for lay in layers]
    prm = ([{k: to_dev(v, "bf16") for k, v in lay["params"].items()} for lay in layers]
           if affine else None)
    ws_bytes = vb.encoder_workspace_bytes(N, T, D, F, H, vb.VITBLK_BF16)

    def call(out, ws):
        vb.encoder_forward(dx, packed, F, H, 1e-6, params=prm, want_tokens=False, cls_out=out,
                           workspace=ws)

    inputs = [dx] + packed + ([t for p in prm for t in p.values()] if affine else [])
    cls = _run_twice(call, (N, D), ws_bytes, inputs)
    _, ref = oracle.encoder(x, layers, H, 1e-6)
    assert_close(to_host(cls), ref, "bf16", f"guarded class tokens affine={affine}",
                 scale=stack_scale(L))


def test_encoder_all_tokens_guarded_and_poisoned():
    N, T, D, H, F, L = 3, 197, 256, 4, 1024, 2
    x = make_block_inputs(N, T, D, F, "bf16", seed=19)["x"]
    layers = [{k: v for k, v in make_block_inputs(1, 1, D, F, "bf16", seed=1900 + l).items()
               if k in WEIGHTS} for l in range(L)]
    dx = to_dev(x, "bf16")
    packed = [vb.pack_weights(*(to_dev(lay[k], "bf16") for k in WEIGHTS)) for lay in layers]
    ws_bytes = vb.encoder_workspace_bytes(N, T, D, F, H, vb.VITBLK_BF16)

    def call(out, ws):
        vb.encoder_forward(dx, packed, F, H, 1e-6, want_cls=False, out=out, workspace=ws)

    tok = _run_twice(call, (N, T, D), ws_bytes, [dx] + packed)
    ref, _ = oracle.encoder(x, layers, H, 1e-6)
    assert_close(to_host(tok), ref, "bf16", "guarded encoder tokens", scale=stack_scale(L))


def test_binding_rejects_a_wrong_out_without_launching():
    # A wrong-shaped output never reaches the library: ValueError, and the
    # buffer keeps its contents.
    import torch
    inp = make_block_inputs(2, 65, 128, 512, "bf16", seed=20)
    dev = {k: to_dev(v, "bf16") for k, v in inp.items()}
    bad = torch.full((2, 64, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="out"):
        vb.forward(dev["x"], *(dev[k] for k in WEIGHTS), 2, 1e-6, out=bad)
    torch.cuda.synchronize()
    assert bool((bad == 7.0).all())
    short = torch.zeros(vb.workspace_bytes(2, 65, 128, 512, 2, vb.VITBLK_BF16) - 1,
                        dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        vb.forward(dev["x"], *(dev[k] for k in WEIGHTS), 2, 1e-6, workspace=short)
