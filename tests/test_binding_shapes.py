"""The Python binding checks every shape the C interface relies on (CPU).

The C entry points receive bare device pointers, so a tensor of the wrong
size would be read or written out of bounds on the GPU.  The binding checks
the shapes of weights, parameters, outputs, packed-weight buffers and
workspaces before anything reaches the library; these checks run before
the device check, so they can be driven here with CPU tensors (nothing is
launched: a CPU tensor with the right shapes stops at "must be on the GPU").
"""

import pytest
import torch

import vision_transformer_encoder_amd as vb

N, T, D, F, H = 2, 5, 16, 32, 2
bf = torch.bfloat16


def _t(*shape):
    return torch.zeros(shape, dtype=bf)


def _weights(**over):
    w = dict(w_q=_t(D, D), w_k=_t(D, D), w_v=_t(D, D), w_o=_t(D, D), w_mlp1=_t(D, F),
             w_mlp2=_t(F, D))
    w.update(over)
    return w


def _fwd(x=None, out=None, workspace=None, **over):
    w = _weights(**over)
    return vb.forward(_t(N, T, D) if x is None else x, w["w_q"], w["w_k"], w["w_v"], w["w_o"],
                      w["w_mlp1"], w["w_mlp2"], H, 1e-6, out=out, workspace=workspace)


def test_forward_right_shapes_reach_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _fwd()


@pytest.mark.parametrize("name,bad", [("w_q", (D, D + 8)), ("w_k", (D + 8, D)), ("w_v", (D,)),
                                      ("w_o", (D, F)), ("w_mlp2", (F, D + 8)),
                                      ("w_mlp2", (F + 8, D))])
def test_forward_rejects_a_wrong_weight(name, bad):
    with pytest.raises(ValueError, match=name):
        _fwd(**{name: _t(*bad)})


def test_forward_rejects_w_mlp1_of_another_width():
    with pytest.raises(ValueError, match="w_mlp1"):
        _fwd(w_mlp1=_t(D + 8, F))


@pytest.mark.parametrize("bad", [(N, T, D + 8), (N, T + 1, D), (N * T, D)])
def test_forward_rejects_a_wrong_out(bad):
    with pytest.raises(ValueError, match="out"):
        _fwd(out=_t(*bad))


def test_forward_rejects_a_short_workspace():
    need = vb.workspace_bytes(N, T, D, F, H, vb.VITBLK_BF16)
    with pytest.raises(ValueError, match="workspace"):
        _fwd(workspace=torch.empty(need - 1, dtype=torch.uint8))


def test_forward_rejects_a_workspace_off_the_gpu():
    # Right size but on the host: its address must never reach a kernel.
    need = vb.workspace_bytes(N, T, D, F, H, vb.VITBLK_BF16)
    with pytest.raises(ValueError, match="GPU"):
        _fwd(workspace=torch.empty(need, dtype=torch.uint8))


@pytest.mark.parametrize("key,bad", [("ln1_gamma", (D + 1,)), ("b_q", (F,)), ("b_mlp1", (D,)),
                                     ("b_mlp2", (F,)), ("ln2_beta", (1, D))])
def test_forward_affine_rejects_a_wrong_parameter(key, bad):
    w = _weights()
    with pytest.raises(ValueError, match=key):
        vb.forward_affine(_t(N, T, D), w["w_q"], w["w_k"], w["w_v"], w["w_o"], w["w_mlp1"],
                          w["w_mlp2"], H, 1e-6, params={key: _t(*bad)})


def test_packed_buffers_are_checked():
    need = vb.packed_weights_bytes(D, F, vb.VITBLK_BF16)
    short = torch.empty(need - 256, dtype=torch.uint8)
    with pytest.raises(ValueError, match="packed"):
        vb.forward_packed(_t(N, T, D), short, F, H, 1e-6)
    with pytest.raises(ValueError, match="packed"):
        vb.forward_packed_affine(_t(N, T, D), short, F, H, 1e-6)
    with pytest.raises(ValueError, match=r"packed\[1\]"):
        vb.encoder_forward(_t(N, T, D), [torch.empty(need, dtype=torch.uint8), short], F, H,
                           1e-6)
    w = _weights()
    with pytest.raises(ValueError, match="packed"):
        vb.pack_weights(*w.values(), packed=short)


def test_encoder_outputs_and_final_ln_are_checked():
    need = vb.packed_weights_bytes(D, F, vb.VITBLK_BF16)
    pk = [torch.empty(need, dtype=torch.uint8)]
    with pytest.raises(ValueError, match="cls_out"):
        vb.encoder_forward(_t(N, T, D), pk, F, H, 1e-6, cls_out=_t(N + 1, D))
    with pytest.raises(ValueError, match="out"):
        vb.encoder_forward(_t(N, T, D), pk, F, H, 1e-6, out=_t(N, T - 1, D))
    with pytest.raises(ValueError, match="final_gamma"):
        vb.encoder_forward(_t(N, T, D), pk, F, H, 1e-6, final_gamma=_t(F))
    with pytest.raises(ValueError, match="b_mlp1"):
        vb.encoder_forward(_t(N, T, D), pk, F, H, 1e-6, params=[{"b_mlp1": _t(D)}])


def test_step_entries_check_their_shapes():
    M = N * T
    with pytest.raises(ValueError, match="w_qkv_t"):
        vb.qkv_projection(_t(M, D), _t(2 * D, D))
    with pytest.raises(ValueError, match="out"):
        vb.qkv_projection(_t(M, D), _t(3 * D, D), out=_t(M, 2 * D))
    with pytest.raises(ValueError, match="qkv"):
        vb.attention(_t(M + 1, 3 * D), N, T, H)
    with pytest.raises(ValueError, match="out"):
        vb.attention(_t(M, 3 * D), N, T, H, out=_t(M, 3 * D))
    with pytest.raises(ValueError, match="w_t"):
        vb.linear(_t(M, D), _t(F, D + 8))
    with pytest.raises(ValueError, match="residual"):
        vb.linear(_t(M, D), _t(F, D), vb.EPI_RESIDUAL, residual=_t(M, D))
    with pytest.raises(ValueError, match="residual"):
        vb.linear(_t(M, D), _t(F, D), vb.EPI_RESIDUAL)
    with pytest.raises(ValueError, match="bias"):
        vb.linear(_t(M, D), _t(F, D), bias=_t(D))
    with pytest.raises(ValueError, match="out"):
        vb.linear(_t(M, D), _t(F, D), out=_t(M, D))
    with pytest.raises(ValueError, match="gamma"):
        vb.layernorm(_t(M, D), 1e-6, gamma=_t(F))
    with pytest.raises(ValueError, match="out"):
        vb.layernorm(_t(M, D), 1e-6, out=_t(M, F))
    f32 = torch.float32
    with pytest.raises(ValueError, match="bias"):
        vb.linear_normed(_t(M, D), _t(F, D), torch.zeros(F, dtype=f32),
                         torch.zeros(M, 2, dtype=f32), bias=_t(D))
    with pytest.raises(ValueError, match="out"):
        vb.linear_normed(_t(M, D), _t(F, D), torch.zeros(F, dtype=f32),
                         torch.zeros(M, 2, dtype=f32), out=_t(M, D))


def test_front_end_checks_its_shapes():
    imgs = _t(2, 3, 8, 8)
    with pytest.raises(ValueError, match="w_patch"):
        vb.patch_embed(imgs, _t(4 * 4 * 3 + 1, D), 4)
    with pytest.raises(ValueError, match="pos_emb"):
        vb.patch_embed(imgs, _t(48, D), 4, cls_token=_t(D), pos_emb=_t(4, D))
    with pytest.raises(ValueError, match="out"):
        vb.patch_embed(imgs, _t(48, D), 4, out=_t(2, 5, D))
    with pytest.raises(ValueError, match="patch side"):
        vb.patch_embed(imgs, _t(27, D), 3)


def test_backward_checks_its_shapes():
    w = _weights()
    with pytest.raises(ValueError, match="dout"):
        vb.backward(_t(N, T, D), *w.values(), _t(N, T, F), H, 1e-6)
    grads = {"dx": _t(N, T, D), "dw_q": _t(D, D), "dw_k": _t(D, D), "dw_v": _t(D, D),
             "dw_o": _t(D, D), "dw_mlp1": _t(F, D), "dw_mlp2": _t(F, D)}
    with pytest.raises(ValueError, match="dw_mlp1"):
        vb.backward(_t(N, T, D), *w.values(), _t(N, T, D), H, 1e-6, grads=grads)
    with pytest.raises(ValueError, match="out"):
        vb.weight_grad(_t(10, D), _t(10, F), out=_t(F, D))
    with pytest.raises(ValueError, match="g"):
        vb.layernorm_backward(_t(10, D), _t(10, F), 1e-6)
    with pytest.raises(ValueError, match="datt"):
        vb.attention_backward(_t(N * T, 3 * D), _t(N * T + 1, D), N, T, H)
