// Host-side argument validation and workspace planning for the vitblk C ABI.
// HIP-free: this interface and validate.cpp build with a plain C++ compiler,
// so every error path can be exercised on a machine without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "vitblk.h"

namespace vitblk {

constexpr size_t kRegionAlign = 256;
constexpr int64_t kMaxDim = 2147483647;   // every dim and N*T fit in int32
constexpr int64_t kMaxHeadDim = 1024;

size_t elem_size(int dtype);  // 0 for an unknown dtype

// Out-major weight copies written by vitblk_pack_weights (element offsets
// rounded to kRegionAlign bytes): Wqkv^T [3D, D], Wo^T [D, D], W1^T [F, D],
// W2^T [D, F].
struct PackedPlan {
  size_t off_qkv, off_o, off_1, off_2;
  size_t off_cs_qkv, off_cs_1;  // fp32 column sums of [w_q | w_k | w_v] and of w_mlp1
  size_t total;
};

// Activation regions of the forward pass, relative to `base`.
struct WorkspacePlan {
  PackedPlan packed;   // at the start of the vitblk_forward workspace
  size_t act_base;     // first activation byte (0 for vitblk_forward_packed)
  size_t off_big;      // [M, max(3D, F)]: packed qkv, later the MLP hidden
  size_t off_act;      // [M, D]: LN(x) or its row statistics, then the concatenated
                       // heads, then LN(y) or its row statistics
  size_t off_y;        // [M, D]: first residual output
  size_t act_total;    // bytes of the three activation regions
  size_t total;        // vitblk_forward workspace: packed.total + act_total
};

// Encoder stack workspace: one block's activations, then two [M, D] token
// buffers that the blocks alternate between.
struct EncoderPlan {
  WorkspacePlan block;  // activations at block.act_base (packed weights are the caller's)
  size_t off_tok0, off_tok1;
  size_t total;
};

// Front-end workspace: packed W_patch^T [D, Kp], the patch matrix [B*N, Kp]
// and the embedded patches [B*N, D] (Kp = P*P*C rounded up to 64).
struct EmbedPlan {
  int64_t N, Kp;  // patches per image, padded patch width
  size_t off_wt, off_patches, off_embedded;
  size_t total;
};

int plan_embed(int64_t B, int64_t C, int64_t H, int64_t W, int64_t P, int64_t D, int dtype,
               EmbedPlan* plan);

int validate_patch_embed(const void* images, const void* w_patch, const void* b_patch,
                         const void* cls_token, const void* pos_emb, const void* tokens,
                         int64_t B, int64_t C, int64_t H, int64_t W, int64_t P, int64_t D,
                         int dtype, const void* workspace, size_t workspace_bytes,
                         EmbedPlan* plan);

int plan_packed(int64_t D, int64_t F, int dtype, PackedPlan* plan);

int plan_encoder(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                 EncoderPlan* plan);

// Returns VITBLK_OK and fills *plan, or an error status.
int plan_workspace(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                   WorkspacePlan* plan);

int validate_forward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                     const void* w_o, const void* w_mlp1, const void* w_mlp2,
                     const void* out, int64_t N, int64_t T, int64_t D, int64_t F,
                     int64_t H, double eps, int dtype, const void* workspace,
                     size_t workspace_bytes, WorkspacePlan* plan);

int validate_forward_packed(const void* x, const void* packed, const void* out, int64_t N,
                            int64_t T, int64_t D, int64_t F, int64_t H, double eps, int dtype,
                            const void* workspace, size_t workspace_bytes,
                            WorkspacePlan* plan);

int validate_pack(const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                  const void* w_mlp1, const void* w_mlp2, const void* packed, int64_t D,
                  int64_t F, int dtype, PackedPlan* plan);

// gamma and beta may be null.
int validate_layernorm(const void* x, const void* gamma, const void* beta, const void* out,
                       int64_t rows, int64_t D, double eps, int dtype);

int validate_qkv(const void* xn, const void* w_qkv_t, const void* qkv, int64_t M, int64_t D,
                 int dtype);

int validate_attention(const void* qkv, const void* att, int64_t N, int64_t T, int64_t D,
                       int64_t H, int dtype);

// bias may be null.
int validate_row_stats(const void* x, const float* stats, int64_t rows, int64_t D, double eps,
                       int dtype);
int validate_linear_normed(const void* a, const void* w, const float* col_sums,
                           const float* row_stats, const void* bias, const void* out, int64_t M,
                           int64_t K, int64_t Nout, int epilogue, int dtype);
// gamma, beta and bias may be null.
int validate_affine_fold(const void* w_t, const void* gamma, const void* beta, const void* bias,
                         const void* w_scaled, const float* col_sums, const void* bias_out,
                         int64_t Nout, int64_t K, int dtype);
// Workspace of vitblk_linear_residual_row_stats: one (mean, M2) pair per row
// and 64 columns.  0 for invalid sizes.
size_t linear_stats_workspace_bytes(int64_t M, int64_t Nout);

int validate_linear_residual_stats(const void* a, const void* w, const void* residual,
                                   const void* out, const float* stats, int64_t M, int64_t K,
                                   int64_t Nout, double eps, int dtype, const void* workspace,
                                   size_t workspace_bytes);

int validate_linear(const void* a, const void* w, const void* bias, const void* residual,
                    const void* out, int64_t M, int64_t K, int64_t Nout, int epilogue,
                    int dtype);

// The encoder stack: L >= 1 packed weight buffers (host array of device
// pointers), optional per-block parameters (host array of L) and final
// gain/shift; at least one of out and cls_out.
int validate_encoder(const void* x, const void* const* packed, const vitblk_affine_params* params,
                     int64_t L, const void* final_gamma, const void* final_beta,
                     const void* out, const void* cls_out, int64_t N, int64_t T, int64_t D,
                     int64_t F, int64_t H, double eps, int dtype, const void* workspace,
                     size_t workspace_bytes, EncoderPlan* plan);

// The affine variant's parameters (params may be null; so may every member):
// each present one 16-byte aligned and clear of out ([rows, D]) and of the
// workspace's first workspace_bytes bytes.
int validate_affine_params(const vitblk_affine_params* params, const void* out, int64_t rows,
                           int64_t D, int64_t F, int dtype, const void* workspace,
                           size_t workspace_bytes);

// Weight gradients (out = a^T b over M token rows, out [I, J]): the token
// rows are split into `wgrad_split` ranges, each reduced into an fp32
// partial [I, J]; a second kernel sums the partials in order and rounds.
// The split fills about one round of 256x256 output tiles on 256 compute
// units and keeps at least 512 token rows per range.
int wgrad_split(int64_t M, int64_t I, int64_t J);
size_t wgrad_partial_bytes(int64_t M, int64_t I, int64_t J);  // 0: invalid or overflow

// Per-query softmax statistics of the attention backward: the score maximum,
// the sum of exponentials and rowsum(P * dP) for every (sequence, head,
// query), fp32.
size_t attention_stats_bytes(int64_t N, int64_t T, int64_t H);

// vitblk_backward workspace: the forward's packed weights, the concatenated
// [w_q | w_k | w_v] ([D, 3D], the B operand of the input gradient of the
// fused projection), the recomputed forward activations, the gradient
// buffers, the softmax statistics and the weight-gradient partials.  The
// gradient steps reuse activation regions once these are dead: dz -> h,
// dyn -> yn, datt -> y, dqkv -> z, dxn -> att.
struct BackwardPlan {
  PackedPlan packed;  // at offset 0
  size_t off_wcat;
  size_t off_xn, off_qkv, off_att, off_y, off_yn, off_z, off_h, off_dy;
  size_t off_stats, off_partial;
  size_t partial_bytes;
  size_t total;
};

int plan_backward(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                  BackwardPlan* plan);

// grads: dx, dw_q, dw_k, dw_v, dw_o, dw_mlp1, dw_mlp2 (all non-null).
int validate_backward(const void* x, const void* const* w, const void* dout,
                      void* const* grads, int64_t N, int64_t T, int64_t D, int64_t F,
                      int64_t H, double eps, int dtype, const void* workspace,
                      size_t workspace_bytes, BackwardPlan* plan);

int validate_weight_grad(const void* a, const void* b, const void* out, int64_t M, int64_t I,
                         int64_t J, int dtype, const void* workspace, size_t workspace_bytes);

// residual may be null.
int validate_layernorm_backward(const void* x, const void* g, const void* residual,
                                const void* dx, int64_t rows, int64_t D, double eps, int dtype);

int validate_attention_backward(const void* qkv, const void* datt, const void* dqkv, int64_t N,
                                int64_t T, int64_t D, int64_t H, int dtype,
                                const void* workspace, size_t workspace_bytes);

}  // namespace vitblk
