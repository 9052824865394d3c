"""ctypes binding over ``libvitblk.so`` (declared in ``include/vitblk.h``).

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  PyTorch supplies device memory and the HIP stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libvitblk.so")

VITBLK_FP32, VITBLK_BF16 = 0, 1
EPI_NONE, EPI_RESIDUAL, EPI_GELU, EPI_GELU_GRAD = 0, 1, 2, 3
STATUS = {0: "VITBLK_OK", -1: "VITBLK_ERR_INVALID_ARG", -2: "VITBLK_ERR_UNSUPPORTED",
          -3: "VITBLK_ERR_WORKSPACE", -4: "VITBLK_ERR_ALIAS", -5: "VITBLK_ERR_HIP"}

# Names of the affine variant's optional parameters, in vitblk_affine_params order.
AFFINE_KEYS = ("ln1_gamma", "ln1_beta", "b_q", "b_k", "b_v", "b_o",
               "ln2_gamma", "ln2_beta", "b_mlp1", "b_mlp2")


class AffineParams(ctypes.Structure):
    """vitblk_affine_params: ten nullable device pointers."""
    _fields_ = [(k, ctypes.c_void_p) for k in AFFINE_KEYS]


# Every symbol include/vitblk.h declares, with its ctypes signature.
_P, _I64, _I, _D, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
_AP = ctypes.POINTER(AffineParams)
SIGNATURES = {
    "vitblk_status_string": (ctypes.c_char_p, [_I]),
    "vitblk_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I]),
    "vitblk_packed_weights_bytes": (_SZ, [_I64, _I64, _I]),
    "vitblk_pack_weights": (_I, [_P] * 7 + [_I64, _I64, _I, _P]),
    "vitblk_forward": (_I, [_P] * 8 + [_I64] * 5 + [_D, _I, _P, _SZ, _P]),
    "vitblk_forward_packed": (_I, [_P] * 3 + [_I64] * 5 + [_D, _I, _P, _SZ, _P]),
    "vitblk_forward_packed_noalloc": (_I, [_P] * 3 + [_I64] * 5 + [_D, _I, _P]),
    "vitblk_layernorm": (_I, [_P, _P, _I64, _I64, _D, _I, _P]),
    "vitblk_qkv_projection": (_I, [_P] * 3 + [_I64, _I64, _I, _P]),
    "vitblk_attention": (_I, [_P, _P, _I64, _I64, _I64, _I64, _I, _P]),
    "vitblk_attention_first_queries": (_I, [_P, _P, _I64, _I64, _I64, _I64, _I, _P]),
    "vitblk_linear": (_I, [_P] * 4 + [_I64, _I64, _I64, _I, _I, _P]),
    "vitblk_forward_affine": (_I, [_P] * 7 + [_AP, _P] + [_I64] * 5 + [_D, _I, _P, _SZ, _P]),
    "vitblk_forward_packed_affine": (_I, [_P, _P, _AP, _P] + [_I64] * 5 + [_D, _I, _P, _SZ, _P]),
    "vitblk_layernorm_affine": (_I, [_P] * 4 + [_I64, _I64, _D, _I, _P]),
    "vitblk_linear_bias": (_I, [_P] * 5 + [_I64, _I64, _I64, _I, _I, _P]),
    "vitblk_row_stats": (_I, [_P, _P, _I64, _I64, _D, _I, _P]),
    "vitblk_linear_normed": (_I, [_P] * 6 + [_I64, _I64, _I64, _I, _I, _P]),
    "vitblk_affine_fold": (_I, [_P] * 4 + [_P] * 3 + [_I64, _I64, _I, _P]),
    "vitblk_linear_residual_row_stats_workspace_bytes": (_SZ, [_I64, _I64]),
    "vitblk_linear_residual_row_stats": (_I, [_P] * 5 + [_I64] * 3 + [_D, _I, _P, _SZ, _P]),
    "vitblk_encoder_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I]),
    "vitblk_patch_embed_workspace_bytes": (_SZ, [_I64] * 6 + [_I]),
    "vitblk_patch_embed": (_I, [_P] * 6 + [_I64] * 6 + [_I, _P, _SZ, _P]),
    "vitblk_encoder_forward": (_I, [_P, ctypes.POINTER(ctypes.c_void_p), _AP, _I64, _P, _P, _P,
                                    _P] + [_I64] * 5 + [_D, _I, _P, _SZ, _P]),
    "vitblk_backward_workspace_bytes": (_SZ, [_I64] * 5 + [_I]),
    "vitblk_backward": (_I, [_P] * 15 + [_I64] * 5 + [_D, _I, _P, _SZ, _P]),
    "vitblk_weight_grad_workspace_bytes": (_SZ, [_I64] * 3),
    "vitblk_weight_grad": (_I, [_P] * 3 + [_I64] * 3 + [_I, _P, _SZ, _P]),
    "vitblk_layernorm_backward": (_I, [_P] * 4 + [_I64, _I64, _D, _I, _P]),
    "vitblk_attention_backward_workspace_bytes": (_SZ, [_I64] * 4),
    "vitblk_attention_backward": (_I, [_P] * 3 + [_I64] * 4 + [_I, _P, _SZ, _P]),
}

# Gradients written by vitblk_backward, in argument order.
GRAD_KEYS = ("dx", "dw_q", "dw_k", "dw_v", "dw_o", "dw_mlp1", "dw_mlp2")

_lib = None


class VitblkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def load():
    """Load the library (once); raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m vision_transformer_encoder_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().vitblk_status_string(int(status)).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise VitblkError(fn, status)


# ------------------------------------------------------------ torch plumbing

def _torch():
    import torch
    return torch


def dtype_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.float32:
        return VITBLK_FP32
    if dtype == torch.bfloat16:
        return VITBLK_BF16
    raise TypeError(f"unsupported dtype {dtype}; use torch.float32 or torch.bfloat16")


def _dev(*ts):
    t0 = ts[0]
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("vitblk tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("vitblk tensors must be contiguous")
        if t.dtype != t0.dtype or t.device != t0.device:
            raise ValueError("vitblk tensors must share dtype and device")
    return t0


def _dev_f32(t0, *ts):
    """fp32 side tensors (statistics, sums) on t0's device, contiguous."""
    torch = _torch()
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or t.device != t0.device:
            raise ValueError("vitblk tensors must be on the GPU, on one device")
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("vitblk statistics and sums are contiguous float32 tensors")


def _stream(t, stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


# Shape checks.  The C interface receives bare pointers, so a tensor of the
# wrong size would be read or written out of bounds on the device; every
# entry point below checks the shapes it relies on before anything reaches
# the library.

def _shape(t, shape, name):
    """t (if given) must have exactly this shape."""
    if t is not None and tuple(t.shape) != tuple(int(d) for d in shape):
        raise ValueError(f"{name} must have shape {tuple(int(d) for d in shape)}, "
                         f"got {tuple(t.shape)}")


def _rank(t, ndim, name):
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _buffer(t, ref, need, name):
    """A caller-supplied byte buffer (workspace, packed weights): on ref's
    GPU, contiguous, and at least `need` bytes."""
    if t is None:
        return
    if _nbytes(t) < need:
        raise ValueError(f"{name} holds {_nbytes(t)} bytes, needs at least {need}")
    if ref is None:  # size only
        return
    if not t.is_cuda or t.device != ref.device:
        raise ValueError(f"{name} must be on the same GPU as the inputs")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _params_shapes(params, D, F):
    """Each affine parameter is one value per feature: [F] for b_mlp1, else [D]."""
    if params is None:
        return
    for k, v in params.items():
        _shape(v, (F,) if k == "b_mlp1" else (D,), k)


def _block_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, D):
    """The six (in, out) weights of a block of width D; returns F."""
    _rank(w_mlp1, 2, "w_mlp1")
    F = w_mlp1.shape[1]
    for name, w in (("w_q", w_q), ("w_k", w_k), ("w_v", w_v), ("w_o", w_o)):
        _shape(w, (D, D), name)
    _shape(w_mlp1, (D, F), "w_mlp1")
    _shape(w_mlp2, (F, D), "w_mlp2")
    return F


def workspace_bytes(N, T, D, F, H, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().vitblk_workspace_bytes(N, T, D, F, H, code))


def packed_weights_bytes(D, F, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().vitblk_packed_weights_bytes(D, F, code))


def forward(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, num_heads: int, eps: float,
            out=None, workspace=None, stream=None):
    """out = block(x) for x [N, T, D]; returns out (allocated if not given)."""
    torch = _torch()
    _rank(x, 3, "x")
    N, T, D = x.shape
    F = _block_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, D)
    _shape(out, x.shape, "out")
    code = dtype_code(x.dtype)
    need = workspace_bytes(N, T, D, F, num_heads, code)
    _buffer(workspace, x, need, "workspace")
    _dev(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, out)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = load().vitblk_forward(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o),
                               _ptr(w_mlp1), _ptr(w_mlp2), _ptr(out), N, T, D, F,
                               num_heads, float(eps), code, _ptr(workspace),
                               workspace.numel() * workspace.element_size(),
                               _stream(x, stream))
    _check("vitblk_forward", st)
    return out


def _affine(params, ref, D, F):
    """AffineParams from a {name: tensor or None} dict (None: no parameters)."""
    if params is None:
        return None
    unknown = set(params) - set(AFFINE_KEYS)
    if unknown:
        raise ValueError(f"unknown block parameters: {sorted(unknown)}")
    _params_shapes(params, D, F)
    ts = [params.get(k) for k in AFFINE_KEYS]
    _dev(ref, *ts)
    return AffineParams(*[0 if t is None else t.data_ptr() for t in ts])


def forward_affine(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, num_heads: int, eps: float,
                   params=None, out=None, workspace=None, stream=None):
    """The affine block: params maps AFFINE_KEYS names to [D] (b_mlp1: [F]) tensors."""
    torch = _torch()
    _rank(x, 3, "x")
    N, T, D = x.shape
    F = _block_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, D)
    _shape(out, x.shape, "out")
    _params_shapes(params, D, F)
    code = dtype_code(x.dtype)
    need = workspace_bytes(N, T, D, F, num_heads, code)
    _buffer(workspace, x, need, "workspace")
    _dev(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, out)
    ap = _affine(params, x, D, F)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = load().vitblk_forward_affine(_ptr(x), _ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o),
                                      _ptr(w_mlp1), _ptr(w_mlp2),
                                      None if ap is None else ctypes.byref(ap), _ptr(out), N, T,
                                      D, F, num_heads, float(eps), code, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(x, stream))
    _check("vitblk_forward_affine", st)
    return out


def patch_embed_workspace_bytes(B, C, H, W, P, D, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().vitblk_patch_embed_workspace_bytes(B, C, H, W, P, D, code))


def patch_embed(images, w_patch, patch: int, b_patch=None, cls_token=None, pos_emb=None,
                out=None, workspace=None, stream=None):
    """Tokens [B, N (+1), D] from images [B, C, H, W] (see vitblk_patch_embed)."""
    torch = _torch()
    _rank(images, 4, "images")
    _rank(w_patch, 2, "w_patch")
    B, C, H, W = images.shape
    D = w_patch.shape[1]
    if patch <= 0 or H % patch or W % patch:
        raise ValueError(f"the patch side {patch} must divide the image sides {H} x {W}")
    T = (H // patch) * (W // patch) + (1 if cls_token is not None else 0)
    _shape(w_patch, (patch * patch * C, D), "w_patch")
    _shape(b_patch, (D,), "b_patch")
    _shape(cls_token, (D,), "cls_token")
    _shape(pos_emb, (T, D), "pos_emb")
    _shape(out, (B, T, D), "out")
    code = dtype_code(images.dtype)
    need = patch_embed_workspace_bytes(B, C, H, W, patch, D, code)
    _buffer(workspace, images, need, "workspace")
    _dev(images, w_patch, b_patch, cls_token, pos_emb, out)
    if out is None:
        out = torch.empty((B, T, D), dtype=images.dtype, device=images.device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=images.device)
    st = load().vitblk_patch_embed(_ptr(images), _ptr(w_patch), _ptr(b_patch), _ptr(cls_token),
                                   _ptr(pos_emb), _ptr(out), B, C, H, W, patch, D, code,
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(images, stream))
    _check("vitblk_patch_embed", st)
    return out


def encoder_workspace_bytes(N, T, D, F, H, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().vitblk_encoder_workspace_bytes(N, T, D, F, H, code))


def encoder_forward(x, packed, F: int, num_heads: int, eps: float, params=None,
                    final_gamma=None, final_beta=None, want_tokens=True, want_cls=True,
                    out=None, cls_out=None, workspace=None, stream=None):
    """L blocks (packed: list of pack_weights() buffers) then the final LayerNorm.

    params: None or a list of L dicts (see forward_affine).  Returns
    (tokens [N, T, D] or None, cls [N, D] or None).
    """
    torch = _torch()
    _rank(x, 3, "x")
    N, T, D = x.shape
    L = len(packed)
    _shape(final_gamma, (D,), "final_gamma")
    _shape(final_beta, (D,), "final_beta")
    _shape(out, x.shape, "out")
    _shape(cls_out, (N, D), "cls_out")
    if params is not None:
        for p in params:
            _params_shapes(p, D, F)
    code = dtype_code(x.dtype)
    pw = packed_weights_bytes(D, F, code)
    for i, p in enumerate(packed):  # every size first, then every device
        _buffer(p, None, pw, f"packed[{i}]")
    for i, p in enumerate(packed):
        _buffer(p, x, pw, f"packed[{i}]")
    _buffer(workspace, x, encoder_workspace_bytes(N, T, D, F, num_heads, code), "workspace")
    _dev(x, final_gamma, final_beta, out, cls_out)
    if want_tokens and out is None:
        out = torch.empty_like(x)
    if want_cls and cls_out is None:
        cls_out = torch.empty((N, D), dtype=x.dtype, device=x.device)
    arr = (ctypes.c_void_p * L)(*[p.data_ptr() for p in packed])
    aps = None
    if params is not None:
        if len(params) != L:
            raise ValueError("one parameter dict per block")
        aps = (AffineParams * L)(*[_affine(p, x, D, F) or AffineParams() for p in params])
    need = encoder_workspace_bytes(N, T, D, F, num_heads, code)
    _buffer(workspace, x, need, "workspace")
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = load().vitblk_encoder_forward(
        _ptr(x), arr, None if aps is None else ctypes.cast(aps, _AP), L, _ptr(final_gamma),
        _ptr(final_beta), _ptr(out if want_tokens else None),
        _ptr(cls_out if want_cls else None), N, T, D, F, num_heads, float(eps), code,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(x, stream))
    _check("vitblk_encoder_forward", st)
    return (out if want_tokens else None), (cls_out if want_cls else None)


def pack_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, packed=None, stream=None):
    """Out-major copies of the six weights in one buffer (uint8 tensor)."""
    torch = _torch()
    _rank(w_q, 2, "w_q")
    D = w_q.shape[0]
    F = _block_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, D)
    code = dtype_code(w_q.dtype)
    _buffer(packed, w_q, packed_weights_bytes(D, F, code), "packed")
    _dev(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2)
    if packed is None:
        packed = torch.empty(max(packed_weights_bytes(D, F, code), 1), dtype=torch.uint8,
                             device=w_q.device)
    st = load().vitblk_pack_weights(_ptr(w_q), _ptr(w_k), _ptr(w_v), _ptr(w_o), _ptr(w_mlp1),
                                    _ptr(w_mlp2), _ptr(packed), D, F, code,
                                    _stream(w_q, stream))
    _check("vitblk_pack_weights", st)
    return packed


def packed_views(packed, D: int, F: int, dtype):
    """Views of the four out-major regions of a packed buffer (documented layout).

    Returns (w_qkv_t [3D, D], w_o_t [D, D], w1_t [F, D], w2_t [D, F]).
    """
    torch = _torch()
    es = 2 if dtype == torch.bfloat16 else 4

    def up(b):
        return (b + 255) // 256 * 256

    offs = [0, up(3 * D * D * es)]
    offs.append(offs[1] + up(D * D * es))
    offs.append(offs[2] + up(D * F * es))
    shapes = [(3 * D, D), (D, D), (F, D), (D, F)]
    return tuple(packed[o:o + r * c * es].view(dtype).view(r, c)
                 for o, (r, c) in zip(offs, shapes))


def packed_col_sums(packed, D: int, F: int, dtype):
    """fp32 views of the packed buffer's column sums: (cs_qkv [3D], cs_1 [F])."""
    torch = _torch()
    es = 2 if dtype == torch.bfloat16 else 4

    def up(b):
        return (b + 255) // 256 * 256

    o = up(3 * D * D * es) + up(D * D * es) + 2 * up(D * F * es)
    o1 = o + up(3 * D * 4)
    return (packed[o:o + 3 * D * 4].view(torch.float32),
            packed[o1:o1 + F * 4].view(torch.float32))


def forward_packed(x, packed, F: int, num_heads: int, eps: float, out=None, workspace=None,
                   stream=None):
    """out = block(x) on weights packed by pack_weights()."""
    torch = _torch()
    _rank(x, 3, "x")
    N, T, D = x.shape
    _shape(out, x.shape, "out")
    code = dtype_code(x.dtype)
    _buffer(packed, x, packed_weights_bytes(D, F, code), "packed")
    need = workspace_bytes(N, T, D, F, num_heads, code) - packed_weights_bytes(D, F, code)
    _buffer(workspace, x, need, "workspace")
    _dev(x, out)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = load().vitblk_forward_packed(_ptr(x), _ptr(packed), _ptr(out), N, T, D, F, num_heads,
                                      float(eps), code, _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(x, stream))
    _check("vitblk_forward_packed", st)
    return out


# Bytes of the library's own scratch array (VITBLK_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def forward_packed_noalloc(x, packed, F: int, num_heads: int, eps: float, out, stream=None):
    """forward_packed() with the activations in the library's scratch array:
    no workspace, nothing allocated (out must be given).  Calls that overlap
    on one GPU race (they share that GPU's array)."""
    _rank(x, 3, "x")
    N, T, D = x.shape
    if out is None:
        raise ValueError("out must be given: this entry point allocates nothing")
    _shape(out, x.shape, "out")
    code = dtype_code(x.dtype)
    _buffer(packed, x, packed_weights_bytes(D, F, code), "packed")
    _dev(x, out)
    st = load().vitblk_forward_packed_noalloc(_ptr(x), _ptr(packed), _ptr(out), N, T, D, F,
                                              num_heads, float(eps), code, _stream(x, stream))
    _check("vitblk_forward_packed_noalloc", st)
    return out


def forward_packed_affine(x, packed, F: int, num_heads: int, eps: float, params=None,
                          out=None, workspace=None, stream=None):
    """The affine block on weights packed by pack_weights()."""
    torch = _torch()
    _rank(x, 3, "x")
    N, T, D = x.shape
    _shape(out, x.shape, "out")
    _params_shapes(params, D, F)
    code = dtype_code(x.dtype)
    _buffer(packed, x, packed_weights_bytes(D, F, code), "packed")
    need = workspace_bytes(N, T, D, F, num_heads, code) - packed_weights_bytes(D, F, code)
    _buffer(workspace, x, need, "workspace")
    _dev(x, out)
    ap = _affine(params, x, D, F)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = load().vitblk_forward_packed_affine(_ptr(x), _ptr(packed),
                                             None if ap is None else ctypes.byref(ap), _ptr(out),
                                             N, T, D, F, num_heads, float(eps), code,
                                             _ptr(workspace),
                                             workspace.numel() * workspace.element_size(),
                                             _stream(x, stream))
    _check("vitblk_forward_packed_affine", st)
    return out


def layernorm(x, eps: float, gamma=None, beta=None, out=None, stream=None):
    """Row-wise LN over the last axis of a contiguous tensor, optionally * gamma + beta."""
    torch = _torch()
    D = x.shape[-1]
    rows = x.numel() // D
    _shape(gamma, (D,), "gamma")
    _shape(beta, (D,), "beta")
    _shape(out, x.shape, "out")
    _dev(x, gamma, beta, out)
    if out is None:
        out = torch.empty_like(x)
    if gamma is None and beta is None:
        st = load().vitblk_layernorm(_ptr(x), _ptr(out), rows, D, float(eps),
                                     dtype_code(x.dtype), _stream(x, stream))
        _check("vitblk_layernorm", st)
    else:
        st = load().vitblk_layernorm_affine(_ptr(x), _ptr(gamma), _ptr(beta), _ptr(out), rows, D,
                                            float(eps), dtype_code(x.dtype), _stream(x, stream))
        _check("vitblk_layernorm_affine", st)
    return out


def qkv_projection(xn, w_qkv_t, out=None, stream=None):
    """Packed [M, 3D] = xn [M, D] @ [w_q | w_k | w_v], weight given out-major [3D, D]."""
    torch = _torch()
    D = xn.shape[-1]
    M = xn.numel() // D
    _shape(w_qkv_t, (3 * D, D), "w_qkv_t")
    _shape(out, (M, 3 * D), "out")
    _dev(xn, w_qkv_t, out)
    if out is None:
        out = torch.empty((M, 3 * D), dtype=xn.dtype, device=xn.device)
    st = load().vitblk_qkv_projection(_ptr(xn), _ptr(w_qkv_t), _ptr(out), M, D,
                                      dtype_code(xn.dtype), _stream(xn, stream))
    _check("vitblk_qkv_projection", st)
    return out


def attention(qkv, N: int, T: int, num_heads: int, out=None, stream=None):
    """Concatenated head outputs [N*T, D] from packed qkv [N*T, 3D]."""
    torch = _torch()
    _rank(qkv, 2, "qkv")
    D = qkv.shape[-1] // 3
    _shape(qkv, (N * T, 3 * D), "qkv")
    _shape(out, (N * T, D), "out")
    _dev(qkv, out)
    if out is None:
        out = torch.empty((N * T, D), dtype=qkv.dtype, device=qkv.device)
    st = load().vitblk_attention(_ptr(qkv), _ptr(out), N, T, D, num_heads,
                                 dtype_code(qkv.dtype), _stream(qkv, stream))
    _check("vitblk_attention", st)
    return out


def attention_first_queries(qkv, N: int, T: int, num_heads: int, out=None, stream=None):
    """attention() for the first min(T, 32) queries of each sequence (all keys):
    those rows of out [N*T, D] are written, the others may not be."""
    torch = _torch()
    _rank(qkv, 2, "qkv")
    D = qkv.shape[-1] // 3
    _shape(qkv, (N * T, 3 * D), "qkv")
    _shape(out, (N * T, D), "out")
    _dev(qkv, out)
    if out is None:
        out = torch.empty((N * T, D), dtype=qkv.dtype, device=qkv.device)
    st = load().vitblk_attention_first_queries(_ptr(qkv), _ptr(out), N, T, D, num_heads,
                                               dtype_code(qkv.dtype), _stream(qkv, stream))
    _check("vitblk_attention_first_queries", st)
    return out


def linear(a, w_t, epilogue: int = EPI_NONE, residual=None, out=None, stream=None,
           bias=None):
    """out = epilogue(a [M, K] @ W + bias) (+ residual), W given out-major, w_t [Nout, K]."""
    torch = _torch()
    K = a.shape[-1]
    M = a.numel() // K
    _rank(w_t, 2, "w_t")
    Nout = w_t.shape[0]
    _shape(w_t, (Nout, K), "w_t")
    _shape(residual, (M, Nout), "residual")
    _shape(bias, (Nout,), "bias")
    _shape(out, (M, Nout), "out")
    if epilogue == EPI_RESIDUAL and residual is None:
        raise ValueError("the residual epilogue needs a residual")
    _dev(a, w_t, residual, bias, out)
    if out is None:
        out = torch.empty((M, Nout), dtype=a.dtype, device=a.device)
    if bias is None:
        st = load().vitblk_linear(_ptr(a), _ptr(w_t), _ptr(residual), _ptr(out), M, K, Nout,
                                  int(epilogue), dtype_code(a.dtype), _stream(a, stream))
        _check("vitblk_linear", st)
    else:
        st = load().vitblk_linear_bias(_ptr(a), _ptr(w_t), _ptr(bias), _ptr(residual), _ptr(out),
                                       M, K, Nout, int(epilogue), dtype_code(a.dtype),
                                       _stream(a, stream))
        _check("vitblk_linear_bias", st)
    return out


def row_stats(x, eps: float, out=None, stream=None):
    """fp32 [rows, 2]: each row's mean and 1 / sqrt(var + eps) (x [..., D])."""
    torch = _torch()
    _dev(x)
    _dev_f32(x, out)
    D = x.shape[-1]
    rows = x.numel() // D
    if out is None:
        out = torch.empty((rows, 2), dtype=torch.float32, device=x.device)
    if out.numel() != 2 * rows:
        raise ValueError(f"stats must hold 2 floats per row ({2 * rows}), got {out.numel()}")
    st = load().vitblk_row_stats(_ptr(x), _ptr(out), rows, D, float(eps), dtype_code(x.dtype),
                                 _stream(x, stream))
    _check("vitblk_row_stats", st)
    return out


def linear_normed(a, w_t, col_sums, stats, epilogue: int = EPI_NONE, bias=None, out=None,
                  stream=None):
    """out = epilogue(LN(a) @ W + bias) with the LayerNorm folded into the product:
    a [M, K] raw rows, stats = row_stats(a), col_sums fp32 [Nout] (W's column sums),
    W given out-major, w_t [Nout, K]."""
    torch = _torch()
    K = a.shape[-1]
    M = a.numel() // K
    _rank(w_t, 2, "w_t")
    Nout = w_t.shape[0]
    _shape(w_t, (Nout, K), "w_t")
    _shape(bias, (Nout,), "bias")
    _shape(out, (M, Nout), "out")
    if col_sums.numel() != Nout or stats.numel() != 2 * M:
        raise ValueError("col_sums must hold Nout floats and stats 2 per row of a")
    _dev(a, w_t, bias, out)
    _dev_f32(a, col_sums, stats)
    if out is None:
        out = torch.empty((M, Nout), dtype=a.dtype, device=a.device)
    st = load().vitblk_linear_normed(_ptr(a), _ptr(w_t), _ptr(col_sums), _ptr(stats), _ptr(bias),
                                     _ptr(out), M, K, Nout, int(epilogue), dtype_code(a.dtype),
                                     _stream(a, stream))
    _check("vitblk_linear_normed", st)
    return out


def affine_fold(w_t, gamma=None, beta=None, bias=None, out=None, stream=None):
    """The affine LayerNorm folded into the product after it (bf16):
    (w_scaled [Nout, K], col_sums fp32 [Nout], bias_out [Nout]) with
    w_scaled = gamma * w_t (per column k), col_sums its row sums and
    bias_out = bias + w_t @ beta, the operands vitblk_linear_normed takes for
    (LN(a) * gamma + beta) @ W + bias.  w_t [Nout, K] is W out-major.
    out: optional preallocated triple."""
    torch = _torch()
    _rank(w_t, 2, "w_t")
    Nout, K = w_t.shape
    _shape(gamma, (K,), "gamma")
    _shape(beta, (K,), "beta")
    _shape(bias, (Nout,), "bias")
    _dev(w_t, gamma, beta, bias)
    if out is None:
        out = (torch.empty_like(w_t), torch.empty(Nout, dtype=torch.float32, device=w_t.device),
               torch.empty(Nout, dtype=w_t.dtype, device=w_t.device))
    ws, cs, bo = out
    _shape(ws, (Nout, K), "w_scaled")
    _shape(bo, (Nout,), "bias_out")
    _dev(w_t, ws, bo)
    _dev_f32(w_t, cs)
    if cs.numel() != Nout:
        raise ValueError("col_sums must hold Nout floats")
    st = load().vitblk_affine_fold(_ptr(w_t), _ptr(gamma), _ptr(beta), _ptr(bias), _ptr(ws),
                                   _ptr(cs), _ptr(bo), Nout, K, dtype_code(w_t.dtype),
                                   _stream(w_t, stream))
    _check("vitblk_affine_fold", st)
    return ws, cs, bo


def linear_residual_row_stats_workspace_bytes(M, Nout) -> int:
    return int(load().vitblk_linear_residual_row_stats_workspace_bytes(M, Nout))


def linear_residual_row_stats(a, w_t, residual, eps: float, out=None, stats=None,
                              workspace=None, stream=None):
    """(out, stats): out = residual + a @ W (W out-major, w_t [Nout, K]) and each
    row's (mean, 1 / sqrt(var + eps)) of out as stored, fp32 [M, 2]."""
    torch = _torch()
    K = a.shape[-1]
    M = a.numel() // K
    _rank(w_t, 2, "w_t")
    Nout = w_t.shape[0]
    _shape(w_t, (Nout, K), "w_t")
    _shape(residual, (M, Nout), "residual")
    _shape(out, (M, Nout), "out")
    _shape(stats, (M, 2), "stats")
    need = linear_residual_row_stats_workspace_bytes(M, Nout)
    _buffer(workspace, a, need, "workspace")
    _dev(a, w_t, residual, out)
    _dev_f32(a, stats)
    if out is None:
        out = torch.empty((M, Nout), dtype=a.dtype, device=a.device)
    if stats is None:
        stats = torch.empty((M, 2), dtype=torch.float32, device=a.device)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=a.device)
    st = load().vitblk_linear_residual_row_stats(
        _ptr(a), _ptr(w_t), _ptr(residual), _ptr(out), _ptr(stats), M, K, Nout, float(eps),
        dtype_code(a.dtype), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(a, stream))
    _check("vitblk_linear_residual_row_stats", st)
    return out, stats


# ------------------------------------------------------------------ backward

def backward_workspace_bytes(N, T, D, F, H, dtype) -> int:
    code = dtype if isinstance(dtype, int) else dtype_code(dtype)
    return int(load().vitblk_backward_workspace_bytes(N, T, D, F, H, code))


def backward(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, dout, num_heads: int, eps: float,
             grads=None, workspace=None, stream=None):
    """Gradients of sum(dout * block(x)): dict keyed by GRAD_KEYS (allocated if not given)."""
    torch = _torch()
    ws_ = (w_q, w_k, w_v, w_o, w_mlp1, w_mlp2)
    _rank(x, 3, "x")
    N, T, D = x.shape
    F = _block_weights(*ws_, D)
    _shape(dout, x.shape, "dout")
    if grads is not None:
        missing = set(GRAD_KEYS) - set(grads)
        if missing:
            raise ValueError(f"grads lacks {sorted(missing)}")
        _shape(grads["dx"], x.shape, "dx")
        for k, w in zip(GRAD_KEYS[1:], ws_):
            _shape(grads[k], w.shape, k)
    code = dtype_code(x.dtype)
    need = backward_workspace_bytes(N, T, D, F, num_heads, code)
    _buffer(workspace, x, need, "workspace")
    _dev(x, dout, *ws_)
    if grads is None:
        grads = {"dx": torch.empty_like(x)}
        for k, w in zip(GRAD_KEYS[1:], ws_):
            grads[k] = torch.empty_like(w)
    _dev(x, *(grads[k] for k in GRAD_KEYS))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    st = load().vitblk_backward(_ptr(x), *[_ptr(w) for w in ws_], _ptr(dout),
                                *[_ptr(grads[k]) for k in GRAD_KEYS], N, T, D, F, num_heads,
                                float(eps), code, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(x, stream))
    _check("vitblk_backward", st)
    return grads


def weight_grad_workspace_bytes(M, I, J) -> int:
    return int(load().vitblk_weight_grad_workspace_bytes(M, I, J))


def weight_grad(a, b, out=None, workspace=None, stream=None):
    """out [I, J] = a^T b for a [M, I], b [M, J] (sum over the M token rows)."""
    torch = _torch()
    I, J = a.shape[-1], b.shape[-1]
    M = a.numel() // I
    if b.numel() // J != M:
        raise ValueError("a and b must have the same number of rows")
    _shape(out, (I, J), "out")
    _buffer(workspace, a, weight_grad_workspace_bytes(M, I, J), "workspace")
    _dev(a, b, out)
    if out is None:
        out = torch.empty((I, J), dtype=a.dtype, device=a.device)
    if workspace is None:
        workspace = torch.empty(max(weight_grad_workspace_bytes(M, I, J), 1), dtype=torch.uint8,
                                device=a.device)
    st = load().vitblk_weight_grad(_ptr(a), _ptr(b), _ptr(out), M, I, J, dtype_code(a.dtype),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(),
                                   _stream(a, stream))
    _check("vitblk_weight_grad", st)
    return out


def layernorm_backward(x, g, eps: float, residual=None, out=None, stream=None):
    """dx = residual + LN'(x)^T g, row by row over the last axis."""
    torch = _torch()
    D = x.shape[-1]
    rows = x.numel() // D
    _shape(g, x.shape, "g")
    _shape(residual, x.shape, "residual")
    _shape(out, x.shape, "out")
    _dev(x, g, residual, out)
    if out is None:
        out = torch.empty_like(x)
    st = load().vitblk_layernorm_backward(_ptr(x), _ptr(g), _ptr(residual), _ptr(out), rows, D,
                                          float(eps), dtype_code(x.dtype), _stream(x, stream))
    _check("vitblk_layernorm_backward", st)
    return out


def attention_backward_workspace_bytes(N, T, D, H) -> int:
    return int(load().vitblk_attention_backward_workspace_bytes(N, T, D, H))


def attention_backward(qkv, datt, N: int, T: int, num_heads: int, out=None, workspace=None,
                       stream=None):
    """dqkv [N*T, 3D] from the forward's qkv [N*T, 3D] and datt [N*T, D]."""
    torch = _torch()
    D = datt.shape[-1]
    _shape(qkv, (N * T, 3 * D), "qkv")
    _shape(datt, (N * T, D), "datt")
    _shape(out, (N * T, 3 * D), "out")
    _buffer(workspace, qkv, attention_backward_workspace_bytes(N, T, D, num_heads), "workspace")
    _dev(qkv, datt, out)
    if out is None:
        out = torch.empty((N * T, 3 * D), dtype=qkv.dtype, device=qkv.device)
    if workspace is None:
        workspace = torch.empty(max(attention_backward_workspace_bytes(N, T, D, num_heads), 1),
                                dtype=torch.uint8, device=qkv.device)
    st = load().vitblk_attention_backward(_ptr(qkv), _ptr(datt), _ptr(out), N, T, D, num_heads,
                                          dtype_code(qkv.dtype), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(qkv, stream))
    _check("vitblk_attention_backward", st)
    return out
