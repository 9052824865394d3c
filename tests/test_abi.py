"""C-ABI tests that run without a GPU.

They load libvitblk.so, check that it exports every function include/vitblk.h
declares, and drive every argument-error path with fake (never dereferenced)
device addresses: all checks run on the host before any HIP call, so no
kernel is launched here.
"""

import ctypes
import math
import os
import re

import pytest

import vision_transformer_encoder_amd as vb
from vision_transformer_encoder_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vitblk.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, ALIAS = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def lib():
    return vb.load()


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(vitblk_\w+)\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert names, "no declarations parsed from the header"
    assert sorted(_lib.SIGNATURES) == names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in _lib.STATUS.items():
        assert vb.status_string(code).startswith(name)
    assert "unknown" in vb.status_string(12345)


def test_workspace_bytes():
    # three 256-B aligned regions: [M, max(3D, F)], [M, D], [M, D]
    def expect(N, T, D, F, es):
        r = lambda b: (b + 255) // 256 * 256  # noqa: E731
        M = N * T
        # four weight regions, then the fp32 column sums of Wqkv [3D] and W1 [F]
        packed = (r(3 * D * D * es) + r(D * D * es) + 2 * r(D * F * es) + r(3 * D * 4)
                  + r(F * 4))
        assert vb.packed_weights_bytes(D, F, 1 if es == 2 else 0) == packed
        return packed + r(M * max(3 * D, F) * es) + 2 * r(M * D * es)
    assert vb.workspace_bytes(256, 197, 1024, 4096, 16, vb.VITBLK_BF16) == expect(256, 197, 1024, 4096, 2)
    assert vb.workspace_bytes(4, 5, 16, 32, 2, vb.VITBLK_FP32) == expect(4, 5, 16, 32, 4)
    assert vb.workspace_bytes(2, 3, 8, 8, 2, vb.VITBLK_FP32) == expect(2, 3, 8, 8, 4)  # 3D > F
    assert vb.workspace_bytes(1, 1, 6, 4, 4, vb.VITBLK_BF16) == 0       # H does not divide D
    assert vb.workspace_bytes(0, 1, 8, 8, 1, vb.VITBLK_BF16) == 0       # empty batch
    assert vb.workspace_bytes(1, 1, 8, 8, 1, 7) == 0                    # unknown dtype
    assert vb.workspace_bytes(1, 1, 2048 * 2, 8, 2, vb.VITBLK_BF16) == 0  # head width 2048


# Fake device addresses, 16-byte aligned and far apart (never dereferenced).
GAP = 1 << 36


def _addr(i):
    return ctypes.c_void_p((i + 1) * GAP)


def _fwd(lib, N=2, T=5, D=16, F=32, H=2, eps=1e-6, dtype=1, ptrs=None, ws=None, ws_bytes=None):
    p = [_addr(i) for i in range(8)] if ptrs is None else ptrs
    if ws is None:
        ws = _addr(20)
    if ws_bytes is None:
        ws_bytes = max(vb.workspace_bytes(max(N, 1), max(T, 1), max(D, 1), max(F, 1),
                                          max(H, 1), 1), 1 << 20)
    return lib.vitblk_forward(*p, N, T, D, F, H, eps, dtype, ws, ws_bytes, None)


def test_forward_invalid_args(lib):
    assert _fwd(lib, N=0) == INVALID
    assert _fwd(lib, T=-1) == INVALID
    assert _fwd(lib, D=0) == INVALID
    assert _fwd(lib, F=0) == INVALID
    assert _fwd(lib, H=0) == INVALID
    assert _fwd(lib, D=16, H=3) == INVALID
    assert _fwd(lib, eps=-1e-6) == INVALID
    assert _fwd(lib, eps=math.nan) == INVALID
    assert _fwd(lib, eps=math.inf) == INVALID
    assert _fwd(lib, dtype=2) == INVALID
    for i in range(8):
        p = [_addr(j) for j in range(8)]
        p[i] = None
        assert _fwd(lib, ptrs=p) == INVALID, i
        p[i] = ctypes.c_void_p((i + 1) * GAP + 2)  # misaligned
        assert _fwd(lib, ptrs=p) == INVALID, i


def test_forward_unsupported_sizes(lib):
    assert _fwd(lib, N=1 << 20, T=1 << 12, ws_bytes=1) == UNSUPPORTED  # N*T > 2^31-1
    assert _fwd(lib, D=4096, H=2, F=8) == UNSUPPORTED                   # head width 2048


def test_forward_workspace_errors(lib):
    need = vb.workspace_bytes(2, 5, 16, 32, 2, 1)
    assert _fwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert _fwd(lib, ws=ctypes.c_void_p(0)) == WORKSPACE


def test_forward_alias_errors(lib):
    # out overlapping x
    p = [_addr(i) for i in range(8)]
    p[7] = ctypes.c_void_p(p[0].value + 64)
    assert _fwd(lib, ptrs=p) == ALIAS
    # out overlapping w_mlp2
    p = [_addr(i) for i in range(8)]
    p[7] = ctypes.c_void_p(p[6].value)
    assert _fwd(lib, ptrs=p) == ALIAS
    # workspace overlapping out, and workspace overlapping an input
    assert _fwd(lib, ws=ctypes.c_void_p(_addr(7).value + 16)) == ALIAS
    assert _fwd(lib, ws=ctypes.c_void_p(_addr(3).value)) == ALIAS
    # (Calls whose arguments all pass the checks would launch kernels, so the
    # accepting side of these checks is covered by the GPU tests only.)


def test_step_entry_points_errors(lib):
    a, b, c, d, e = (_addr(i) for i in range(5))
    # layernorm
    assert lib.vitblk_layernorm(None, b, 4, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_layernorm(a, b, 0, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_layernorm(a, b, 4, 8, -1.0, 1, None) == INVALID
    assert lib.vitblk_layernorm(a, b, 4, 8, 1e-5, 9, None) == INVALID
    assert lib.vitblk_layernorm(a, a, 4, 8, 1e-5, 1, None) == ALIAS
    # qkv
    assert lib.vitblk_qkv_projection(a, b, None, 4, 8, 1, None) == INVALID
    assert lib.vitblk_qkv_projection(a, b, a, 4, 8, 1, None) == ALIAS
    assert lib.vitblk_qkv_projection(a, b, e, 4, 0, 1, None) == INVALID
    # pack
    w = [_addr(i) for i in range(6)]
    assert lib.vitblk_pack_weights(*w, None, 16, 32, 1, None) == INVALID
    assert lib.vitblk_pack_weights(*w, _addr(2), 16, 32, 1, None) == ALIAS
    assert lib.vitblk_pack_weights(*w, _addr(9), 0, 32, 1, None) == INVALID
    assert lib.vitblk_pack_weights(*w, _addr(9), 16, 32, 5, None) == INVALID
    assert vb.packed_weights_bytes(0, 8, 1) == 0
    # forward_packed
    ws_need = vb.workspace_bytes(2, 5, 16, 32, 2, 1) - vb.packed_weights_bytes(16, 32, 1)
    fp = lambda *args: lib.vitblk_forward_packed(*args)  # noqa: E731
    assert fp(a, b, c, 2, 5, 16, 32, 2, 1e-6, 1, _addr(9), ws_need - 1, None) == WORKSPACE
    assert fp(a, b, a, 2, 5, 16, 32, 2, 1e-6, 1, _addr(9), ws_need, None) == ALIAS
    assert fp(a, b, c, 2, 5, 16, 32, 3, 1e-6, 1, _addr(9), ws_need, None) == INVALID
    assert fp(a, b, c, 2, 5, 16, 32, 2, -1.0, 1, _addr(9), ws_need, None) == INVALID
    assert fp(a, None, c, 2, 5, 16, 32, 2, 1e-6, 1, _addr(9), ws_need, None) == INVALID
    assert fp(a, b, c, 2, 5, 16, 32, 2, 1e-6, 1, _addr(1), ws_need, None) == ALIAS
    # attention
    assert lib.vitblk_attention(a, b, 2, 3, 8, 3, 1, None) == INVALID   # H does not divide D
    assert lib.vitblk_attention(a, a, 2, 3, 8, 2, 1, None) == ALIAS
    assert lib.vitblk_attention(a, b, 1, 1, 4096, 2, 1, None) == UNSUPPORTED
    # linear
    assert lib.vitblk_linear(a, b, None, c, 4, 8, 8, vb.EPI_RESIDUAL, 1, None) == INVALID
    assert lib.vitblk_linear(a, b, None, c, 4, 8, 8, 7, 1, None) == INVALID
    assert lib.vitblk_linear(a, b, c, c, 4, 8, 8, vb.EPI_RESIDUAL, 1, None) == ALIAS
    assert lib.vitblk_linear(a, b, None, a, 4, 8, 8, vb.EPI_NONE, 1, None) == ALIAS
    assert lib.vitblk_linear(a, b, None, c, 4, -8, 8, vb.EPI_GELU, 1, None) == INVALID
    # row statistics (stats 8-byte aligned, 2 floats per row); every call
    # below fails its checks before any launch
    off = lambda p, k: ctypes.c_void_p(p.value + k)  # noqa: E731
    assert lib.vitblk_row_stats(None, b, 4, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_row_stats(a, None, 4, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_row_stats(a, off(b, 4), 4, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_row_stats(a, b, 0, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_row_stats(a, b, 4, 8, -1.0, 1, None) == INVALID
    assert lib.vitblk_row_stats(a, off(a, 8), 4, 8, 1e-5, 1, None) == ALIAS
    # the LayerNorm-folded product: plain or GELU epilogue, sums 16-byte aligned
    ln = lambda *args: lib.vitblk_linear_normed(*args)  # noqa: E731
    assert ln(a, b, c, d, None, e, 4, 8, 8, vb.EPI_RESIDUAL, 1, None) == INVALID
    assert ln(a, b, None, d, None, e, 4, 8, 8, vb.EPI_GELU, 1, None) == INVALID
    assert ln(a, b, c, None, None, e, 4, 8, 8, vb.EPI_GELU, 1, None) == INVALID
    assert ln(a, b, off(c, 8), d, None, e, 4, 8, 8, vb.EPI_GELU, 1, None) == INVALID
    assert ln(a, b, c, off(d, 4), None, e, 4, 8, 8, vb.EPI_GELU, 1, None) == INVALID
    assert ln(a, b, c, d, None, e, 4, 0, 8, vb.EPI_GELU, 1, None) == INVALID
    assert ln(a, b, c, d, None, c, 4, 8, 8, vb.EPI_GELU, 1, None) == ALIAS
    assert ln(a, b, c, d, None, d, 4, 8, 8, vb.EPI_NONE, 1, None) == ALIAS
    assert ln(a, b, c, d, None, a, 4, 8, 8, vb.EPI_NONE, 1, None) == ALIAS
    # the affine LayerNorm fold: bf16 only, K a multiple of 8, outputs clear
    # of the inputs and of each other (w_t a, gamma b, beta c, bias d;
    # outputs e, col sums at _addr(6), bias_out at _addr(7))
    fo = lambda *args: lib.vitblk_affine_fold(*args)  # noqa: E731
    cs, bo = _addr(6), _addr(7)
    assert fo(None, b, c, d, e, cs, bo, 8, 16, 1, None) == INVALID
    assert fo(a, b, c, d, None, cs, bo, 8, 16, 1, None) == INVALID
    assert fo(a, b, c, d, e, None, bo, 8, 16, 1, None) == INVALID
    assert fo(a, b, c, d, e, cs, None, 8, 16, 1, None) == INVALID
    assert fo(a, off(b, 8), c, d, e, cs, bo, 8, 16, 1, None) == INVALID
    assert fo(a, b, c, d, e, off(cs, 4), bo, 8, 16, 1, None) == INVALID
    assert fo(a, b, c, off(d, 1), e, cs, bo, 8, 16, 1, None) == INVALID
    assert fo(a, b, c, d, e, cs, bo, 0, 16, 1, None) == INVALID
    assert fo(a, b, c, d, e, cs, bo, 8, 16, 9, None) == INVALID
    assert fo(a, b, c, d, e, cs, bo, 8, 16, 0, None) == UNSUPPORTED  # fp32
    assert fo(a, b, c, d, e, cs, bo, 8, 12, 1, None) == UNSUPPORTED  # K % 8
    assert fo(a, b, c, d, off(a, 64), cs, bo, 8, 16, 1, None) == ALIAS
    assert fo(a, b, c, d, e, off(b, 16), bo, 8, 16, 1, None) == ALIAS
    assert fo(a, b, c, d, e, cs, off(d, 2), 8, 16, 1, None) == ALIAS
    assert fo(a, b, c, d, e, cs, off(e, 64), 8, 16, 1, None) == ALIAS
    assert fo(a, None, None, None, e, cs, off(cs, 16), 8, 16, 1, None) == ALIAS
    # the output projection with the next LayerNorm's statistics: residual
    # required, stats 8-byte aligned, a workspace of one pair per 64 columns
    rs = lambda *args: lib.vitblk_linear_residual_row_stats(*args)  # noqa: E731
    need = lib.vitblk_linear_residual_row_stats_workspace_bytes(4, 128)
    assert need == 4 * 2 * 8
    assert lib.vitblk_linear_residual_row_stats_workspace_bytes(4, 130) == 4 * 3 * 8
    assert lib.vitblk_linear_residual_row_stats_workspace_bytes(0, 128) == 0
    ws = _addr(9)
    assert rs(a, b, None, c, d, 4, 8, 128, 1e-6, 1, ws, need, None) == INVALID
    assert rs(a, b, e, c, None, 4, 8, 128, 1e-6, 1, ws, need, None) == INVALID
    assert rs(a, b, e, c, off(d, 4), 4, 8, 128, 1e-6, 1, ws, need, None) == INVALID
    assert rs(a, b, e, c, d, 4, 8, 128, -1.0, 1, ws, need, None) == INVALID
    assert rs(a, b, e, c, d, 4, 8, 128, 1e-6, 1, ws, need - 1, None) == WORKSPACE
    assert rs(a, b, e, c, d, 4, 8, 128, 1e-6, 1, None, need, None) == WORKSPACE
    assert rs(a, b, e, c, c, 4, 8, 128, 1e-6, 1, ws, need, None) == ALIAS
    assert rs(a, b, e, c, d, 4, 8, 128, 1e-6, 1, c, need, None) == ALIAS
    assert rs(a, b, e, c, d, 4, 8, 128, 1e-6, 1, e, need, None) == ALIAS


def test_affine_entry_points_errors(lib):
    AP = vb._lib.AffineParams
    need = vb.workspace_bytes(2, 5, 16, 32, 2, 1)
    w = [_addr(i) for i in range(7)]   # x, w_q .. w_mlp2
    out, ws = _addr(8), _addr(20)

    def fa(prm, out=out, ws_bytes=need):
        ref = None if prm is None else ctypes.byref(prm)
        return lib.vitblk_forward_affine(*w, ref, out, 2, 5, 16, 32, 2, 1e-6, 1, ws, ws_bytes,
                                         None)

    assert fa(None, ws_bytes=need - 1) == WORKSPACE          # plain checks still apply
    assert fa(AP(), out=ctypes.c_void_p(w[0].value)) == ALIAS
    prm = AP(**{k: (30 + i) * GAP for i, k in enumerate(vb.AFFINE_KEYS)})
    assert fa(AP(ln1_gamma=31 * GAP + 8)) == INVALID         # misaligned parameter
    assert fa(AP(b_mlp1=out.value + 64)) == ALIAS            # parameter inside out
    assert fa(AP(b_o=ws.value + 256)) == ALIAS               # parameter inside the workspace
    assert fa(AP(b_q=ws.value + need - 16)) == ALIAS         # ... at its last bytes
    prm_bad = AP(**{k: getattr(prm, k) for k in vb.AFFINE_KEYS})
    prm_bad.b_mlp2 = out.value
    assert fa(prm_bad) == ALIAS
    # packed variant: same parameter checks against the activation workspace
    ws_need = need - vb.packed_weights_bytes(16, 32, 1)
    fpa = lambda prm, n=ws_need: lib.vitblk_forward_packed_affine(  # noqa: E731
        w[0], w[1], ctypes.byref(prm), out, 2, 5, 16, 32, 2, 1e-6, 1, ws, n, None)
    assert fpa(AP(), n=ws_need - 1) == WORKSPACE
    assert fpa(AP(ln2_beta=ws.value)) == ALIAS
    assert fpa(AP(ln2_beta=ws.value + 8)) == INVALID
    # layernorm with gain/shift
    a, b, c = _addr(0), _addr(1), _addr(2)
    assert lib.vitblk_layernorm_affine(a, ctypes.c_void_p(c.value + 4), None, b, 4, 8, 1e-5, 1,
                                       None) == INVALID
    assert lib.vitblk_layernorm_affine(a, None, ctypes.c_void_p(b.value), b, 4, 8, 1e-5, 1,
                                       None) == ALIAS
    assert lib.vitblk_layernorm_affine(a, c, c, a, 4, 8, 1e-5, 1, None) == ALIAS
    # linear with bias
    d = _addr(3)
    assert lib.vitblk_linear_bias(a, b, ctypes.c_void_p(d.value + 2), None, c, 4, 8, 8,
                                  vb.EPI_NONE, 1, None) == INVALID
    assert lib.vitblk_linear_bias(a, b, c, None, c, 4, 8, 8, vb.EPI_GELU, 1, None) == ALIAS
    assert lib.vitblk_linear_bias(a, b, d, None, c, 4, 8, 8, 9, 1, None) == INVALID


def test_encoder_errors(lib):
    N, T, D, F, H = 2, 5, 16, 32, 2
    need = vb.encoder_workspace_bytes(N, T, D, F, H, 1)
    r = lambda b: (b + 255) // 256 * 256  # noqa: E731
    assert need == (vb.workspace_bytes(N, T, D, F, H, 1) - vb.packed_weights_bytes(D, F, 1)
                    + 2 * r(N * T * D * 2))
    assert vb.encoder_workspace_bytes(N, T, D, F, 3, 1) == 0
    x, out, cls, ws = _addr(0), _addr(1), _addr(2), _addr(20)
    pk = (ctypes.c_void_p * 3)(*[_addr(5 + i).value for i in range(3)])

    def enc(L=3, packed=pk, params=None, fg=None, fb=None, out=out, cls=cls, ws_bytes=need,
            eps=1e-6):
        return lib.vitblk_encoder_forward(x, packed, params, L, fg, fb, out, cls, N, T, D, F, H,
                                          eps, 1, ws, ws_bytes, None)

    assert enc(L=0) == INVALID
    assert enc(packed=None) == INVALID
    assert enc(out=None, cls=None) == INVALID
    assert enc(eps=-1.0) == INVALID
    assert enc(ws_bytes=need - 1) == WORKSPACE
    bad = (ctypes.c_void_p * 3)(pk[0], None, pk[2])
    assert enc(packed=bad) == INVALID
    bad = (ctypes.c_void_p * 3)(pk[0], pk[1] + 8, pk[2])
    assert enc(packed=bad) == INVALID
    bad = (ctypes.c_void_p * 3)(pk[0], out.value, pk[2])      # packed weights inside out
    assert enc(packed=bad) == ALIAS
    assert enc(cls=ctypes.c_void_p(out.value + 32)) == ALIAS  # the two outputs overlap
    assert enc(out=ctypes.c_void_p(x.value)) == ALIAS
    assert enc(cls=ctypes.c_void_p(ws.value + 64)) == ALIAS
    assert enc(fg=ctypes.c_void_p(out.value)) == ALIAS
    assert enc(fb=ctypes.c_void_p(_addr(9).value + 4)) == INVALID
    AP = vb._lib.AffineParams
    prm = (AP * 3)(AP(), AP(b_o=cls.value), AP())
    assert enc(params=ctypes.cast(prm, ctypes.POINTER(AP))) == ALIAS


def test_patch_embed_errors(lib):
    B, C, H, W, P, D = 2, 3, 32, 32, 8, 64
    need = vb.patch_embed_workspace_bytes(B, C, H, W, P, D, 1)
    r = lambda b: (b + 255) // 256 * 256  # noqa: E731
    Kp = 192  # 8*8*3 = 192, already a multiple of 64
    assert need == r(D * Kp * 2) + r(B * 16 * Kp * 2) + r(B * 16 * D * 2)
    assert vb.patch_embed_workspace_bytes(B, C, 30, W, P, D, 1) == 0   # 30 % 8 != 0
    # P = 14, C = 3: patch width 588 padded to 640
    assert vb.patch_embed_workspace_bytes(1, 3, 28, 28, 14, 64, 1) == \
        r(64 * 640 * 2) + r(4 * 640 * 2) + r(4 * 64 * 2)
    img, w, out, ws = _addr(0), _addr(1), _addr(2), _addr(20)

    def pe(b=None, cls=None, pos=None, out=out, H=H, ws_bytes=need, dtype=1):
        return lib.vitblk_patch_embed(img, w, b, cls, pos, out, B, C, H, W, P, D, dtype, ws,
                                      ws_bytes, None)

    assert pe(H=30) == INVALID
    assert pe(dtype=4) == INVALID
    assert pe(ws_bytes=need - 1) == WORKSPACE
    assert pe(out=None) == INVALID
    assert pe(b=ctypes.c_void_p(_addr(5).value + 2)) == INVALID
    assert pe(out=ctypes.c_void_p(img.value + 64)) == ALIAS
    assert pe(pos=ctypes.c_void_p(out.value)) == ALIAS
    assert pe(cls=ctypes.c_void_p(ws.value + 512)) == ALIAS
    assert lib.vitblk_patch_embed(img, None, None, None, None, out, B, C, H, W, P, D, 1, ws,
                                  need, None) == INVALID


def test_python_binding_rejects_unknown_affine_parameter():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 8)
    w = torch.zeros(8, 8)
    with pytest.raises(ValueError):
        vb.forward_affine(x, w, w, w, w, w, w, 2, 1e-6, params={"b_qkv": w})


def test_python_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 8)
    w = torch.zeros(8, 8)
    with pytest.raises(ValueError):
        vb.forward(x, w, w, w, w, w, w, 2, 1e-6)


# ------------------------------------------------------------------ backward

def _bwd(lib, N=2, T=5, D=16, F=32, H=2, eps=1e-6, dtype=1, ptrs=None, ws=None, ws_bytes=None):
    """vitblk_backward with fake pointers: 8 inputs (x, six weights, dout), then 7 gradients."""
    p = [_addr(i) for i in range(15)] if ptrs is None else ptrs
    if ws is None:
        ws = _addr(40)
    if ws_bytes is None:
        ws_bytes = max(vb.backward_workspace_bytes(max(N, 1), max(T, 1), max(D, 1), max(F, 1),
                                                   max(H, 1), 1), 1 << 20)
    return lib.vitblk_backward(*p, N, T, D, F, H, eps, dtype, ws, ws_bytes, None)


def _split(M, I, J):
    tiles = -(-I // 256) * -(-J // 256)
    return max(1, min(256 // tiles if tiles < 256 else 1, max(1, M // 512)))


def test_backward_workspace_bytes():
    r = lambda b: (b + 255) // 256 * 256  # noqa: E731

    def expect(N, T, D, F, H, es):
        M = N * T
        packed = (r(3 * D * D * es) + r(D * D * es) + 2 * r(D * F * es) + r(3 * D * 4)
                  + r(F * 4))
        wcat = r(3 * D * D * es)
        # xn, att, y, yn, dy [M, D]; qkv [M, 3D]; z [M, max(F, 3D)]; h [M, F]
        acts = 5 * r(M * D * es) + r(M * 3 * D * es) + r(M * max(F, 3 * D) * es) + r(M * F * es)
        stats = r(M * H * 3 * 4)  # score max, exp sum and rowsum(P * dP) per query and head
        part = max(r(_split(M, i, j) * i * j * 4) for i, j in
                   [(F, D), (D, F), (D, D), (D, 3 * D)])
        return packed + wcat + acts + stats + part

    for (N, T, D, F, H, es) in [(256, 197, 1024, 4096, 16, 2), (4, 5, 16, 32, 2, 4),
                                (2, 3, 8, 8, 2, 4), (64, 197, 768, 3072, 12, 2)]:
        code = 1 if es == 2 else 0
        assert vb.backward_workspace_bytes(N, T, D, F, H, code) == \
            expect(N, T, D, F, H, es), (N, T, D, F, H)
    assert vb.backward_workspace_bytes(1, 1, 6, 4, 4, 1) == 0   # H does not divide D
    assert vb.backward_workspace_bytes(0, 1, 8, 8, 1, 1) == 0   # empty batch
    assert vb.backward_workspace_bytes(1, 1, 8, 8, 1, 5) == 0   # unknown dtype
    # weight gradient: split over token rows into fp32 partials
    assert vb.weight_grad_workspace_bytes(50432, 1024, 1024) == 16 * 1024 * 1024 * 4
    assert vb.weight_grad_workspace_bytes(50432, 1024, 4096) == 4 * 1024 * 4096 * 4
    assert vb.weight_grad_workspace_bytes(50432, 1024, 3072) == 5 * 1024 * 3072 * 4
    assert vb.weight_grad_workspace_bytes(20, 16, 32) == r(16 * 32 * 4)  # few rows: no split
    assert vb.weight_grad_workspace_bytes(0, 16, 32) == 0
    assert vb.attention_backward_workspace_bytes(256, 197, 1024, 16) == r(256 * 197 * 16 * 12)
    assert vb.attention_backward_workspace_bytes(2, 5, 16, 3) == 0


def test_backward_errors(lib):
    assert _bwd(lib, N=0) == INVALID
    assert _bwd(lib, D=16, H=3) == INVALID
    assert _bwd(lib, eps=-1.0) == INVALID
    assert _bwd(lib, eps=math.nan) == INVALID
    assert _bwd(lib, dtype=3) == INVALID
    for i in range(15):
        p = [_addr(j) for j in range(15)]
        p[i] = None
        assert _bwd(lib, ptrs=p) == INVALID, i
        p[i] = ctypes.c_void_p((i + 1) * GAP + 4)  # misaligned
        assert _bwd(lib, ptrs=p) == INVALID, i
    assert _bwd(lib, D=4096, H=2, F=8) == UNSUPPORTED
    need = vb.backward_workspace_bytes(2, 5, 16, 32, 2, 1)
    assert _bwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert _bwd(lib, ws=ctypes.c_void_p(0)) == WORKSPACE
    # a gradient overlapping an input, another gradient, or the workspace
    for gi, other in [(8, 0), (9, 1), (14, 7), (10, 11), (13, 8)]:
        p = [_addr(j) for j in range(15)]
        p[gi] = ctypes.c_void_p(p[other].value)
        assert _bwd(lib, ptrs=p) == ALIAS, (gi, other)
    assert _bwd(lib, ws=ctypes.c_void_p(_addr(12).value)) == ALIAS
    assert _bwd(lib, ws=ctypes.c_void_p(_addr(7).value)) == ALIAS   # dout inside the workspace


def test_backward_step_entry_points_errors(lib):
    a, b, c, d = (_addr(i) for i in range(4))
    big = 1 << 30
    # weight gradient
    assert lib.vitblk_weight_grad(None, b, c, 64, 16, 16, 1, d, big, None) == INVALID
    assert lib.vitblk_weight_grad(a, b, c, 0, 16, 16, 1, d, big, None) == INVALID
    assert lib.vitblk_weight_grad(a, b, c, 64, 16, 16, 9, d, big, None) == INVALID
    assert lib.vitblk_weight_grad(a, b, c, 64, 16, 16, 1, None, big, None) == WORKSPACE
    assert lib.vitblk_weight_grad(a, b, c, 64, 16, 16, 1, d, 16 * 16 * 4 - 1, None) == WORKSPACE
    assert lib.vitblk_weight_grad(a, b, a, 64, 16, 16, 1, d, big, None) == ALIAS
    assert lib.vitblk_weight_grad(a, b, c, 64, 16, 16, 1, ctypes.c_void_p(c.value + 32), big,
                                  None) == ALIAS
    # LayerNorm backward (residual may be NULL: that is not an error by itself)
    assert lib.vitblk_layernorm_backward(None, b, c, d, 4, 8, 1e-5, 1, None) == INVALID
    assert lib.vitblk_layernorm_backward(a, b, c, d, 4, 0, 1e-5, 1, None) == INVALID
    assert lib.vitblk_layernorm_backward(a, b, c, d, 4, 8, -1.0, 1, None) == INVALID
    assert lib.vitblk_layernorm_backward(a, b, None, a, 4, 8, 1e-5, 1, None) == ALIAS
    assert lib.vitblk_layernorm_backward(a, b, c, c, 4, 8, 1e-5, 1, None) == ALIAS
    assert lib.vitblk_layernorm_backward(a, b, c, ctypes.c_void_p(b.value + 16), 4, 8, 1e-5, 1,
                                         None) == ALIAS
    # attention backward
    assert lib.vitblk_attention_backward(a, b, None, 2, 5, 16, 2, 1, d, big, None) == INVALID
    assert lib.vitblk_attention_backward(a, b, c, 2, 5, 16, 3, 1, d, big, None) == INVALID
    assert lib.vitblk_attention_backward(a, b, c, 2, 5, 16, 2, 1, None, big, None) == WORKSPACE
    assert lib.vitblk_attention_backward(a, b, c, 2, 5, 16, 2, 1, d, 2 * 5 * 2 * 12 - 1,
                                         None) == WORKSPACE
    assert lib.vitblk_attention_backward(a, b, a, 2, 5, 16, 2, 1, d, big, None) == ALIAS
    assert lib.vitblk_attention_backward(a, b, c, 2, 5, 16, 2, 1, ctypes.c_void_p(c.value),
                                         big, None) == ALIAS
    # the GELU-derivative epilogue reads z through `residual`, so it must be given
    assert lib.vitblk_linear(a, b, None, c, 64, 64, 64, vb.EPI_GELU_GRAD, 1, None) == INVALID
    assert lib.vitblk_linear(a, b, c, c, 64, 64, 64, vb.EPI_GELU_GRAD, 1, None) == ALIAS
    assert lib.vitblk_linear(a, b, c, d, 64, 64, 64, 4, 1, None) == INVALID
