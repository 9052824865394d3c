/*
 * vitblk -- forward pass of one pre-LayerNorm Vision Transformer encoder block
 * on AMD Instinct MI355X (gfx950), as a C ABI over hand-written HIP kernels.
 *
 * The block (crackedaicode.com "ViT Encoder Block", sections "Normalize before
 * each stage", "Multi-head attention" and "Feed-forward stage"; the same
 * block appears as "Key Equations" steps 1-6 on ai-engineer-exhaustive.pages.dev
 * "ViT Encoder Block"):
 *
 *   xn  = LN(x)                      LN: per token over D features, population
 *                                    variance, eps inside the square root, no
 *                                    learned scale or shift
 *   Q, K, V = xn @ w_q, xn @ w_k, xn @ w_v
 *   att = concat_h softmax(Q_h K_h^T / sqrt(D/H)) V_h
 *                                    head h = features [h*D/H, (h+1)*D/H),
 *                                    no mask, stable softmax over keys
 *   y   = x + att @ w_o
 *   out = y + GELU_tanh(LN(y) @ w_mlp1) @ w_mlp2
 *   GELU_tanh(z) = 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3)))
 *
 * There are no biases.  Weights are stored (in_features, out_features) and
 * applied as x @ W.  vitblk_forward_affine() adds the optional LayerNorm
 * gains and shifts and projection biases of the affine variant (see there).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, w_*, out, qkv, ... are DEVICE pointers (HIP global
 *   memory) on the current device, owned by the caller.  The library never
 *   allocates or frees memory and keeps no caller data between calls; the
 *   only exception to "no device memory of its own" is the scratch array of
 *   vitblk_forward_packed_noalloc() (see there).  Its only host state is
 *   per-process launch configuration computed on first use (each kernel's
 *   resident workgroup count and dynamic-LDS attribute, the scratch array's
 *   address per device): written once with the same value by whichever call
 *   comes first, so concurrent calls from several threads are safe.  Calls
 *   enqueue on `stream` (0 = the null stream) and return without
 *   synchronising; the caller synchronises before reading results.
 * - All tensors are dense, row-major and contiguous in the element type given
 *   by `dtype` (VITBLK_FP32: IEEE float; VITBLK_BF16: bfloat16 stored as its
 *   16-bit pattern).  Device pointers must be aligned to 16 bytes.
 * - Arithmetic: bf16 operands, fp32 accumulation, fp32 softmax and LayerNorm
 *   statistics; every tensor written to memory (outputs and intermediates)
 *   is rounded to `dtype` with round-to-nearest-even.
 * - Errors: every argument check runs before any kernel is launched; on any
 *   error the outputs are left untouched.  Return values are vitblk_status
 *   codes; vitblk_status_string() names them.  Nothing is thrown across the
 *   ABI.  VITBLK_ERR_HIP reports a launch failure (hipGetLastError) after
 *   work may already have been enqueued.
 */
#ifndef VITBLK_H
#define VITBLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* vitblk_stream_t; /* the same type as hipStream_t */

typedef enum {
  VITBLK_FP32 = 0,
  VITBLK_BF16 = 1
} vitblk_dtype;

typedef enum {
  VITBLK_OK = 0,
  VITBLK_ERR_INVALID_ARG = -1, /* null pointer, dim <= 0, H not dividing D,
                                  unknown dtype or epilogue, eps < 0 or not
                                  finite, misaligned pointer */
  VITBLK_ERR_UNSUPPORTED = -2, /* valid but beyond the kernels' limits:
                                  a dimension or N*T above 2^31-1, or
                                  D/H above 1024 */
  VITBLK_ERR_WORKSPACE = -3,   /* workspace null or smaller than
                                  vitblk_workspace_bytes() */
  VITBLK_ERR_ALIAS = -4,       /* an output overlaps an input or the
                                  workspace, or the workspace overlaps an
                                  input */
  VITBLK_ERR_HIP = -5          /* a kernel launch failed */
} vitblk_status;

typedef enum {
  VITBLK_EPI_NONE = 0,     /* out = a @ w                      */
  VITBLK_EPI_RESIDUAL = 1, /* out = residual + a @ w           */
  VITBLK_EPI_GELU = 2,     /* out = GELU_tanh(a @ w)           */
  VITBLK_EPI_GELU_GRAD = 3 /* out = (a @ w) * GELU_tanh'(residual): the
                              MLP's backward through the activation */
} vitblk_epilogue;

/* Human-readable name of a vitblk_status value (static storage; never NULL). */
const char* vitblk_status_string(int status);

/*
 * Bytes of device workspace vitblk_forward() needs for these sizes, or 0 if
 * the arguments are invalid.  Pure host function: no HIP call.
 *
 * Layout (each region starts on a 256-byte boundary), es = element size,
 * M = N*T:
 *   packed weights, vitblk_packed_weights_bytes(D, F, dtype) bytes
 *   activations:
 *     region 0: M x max(3D, F) elements: packed Q|K|V [M, 3D], later the
 *               MLP hidden activations [M, F]
 *     region 1: M x D elements: LN(x) (or, folded, its row statistics),
 *               later the concatenated heads, later LN(y) (or its statistics)
 *     region 2: M x D elements: y = x + att @ w_o
 *   Regions 0 and 1 also hold fp32 partial sums of the residual products'
 *   last rows while they are otherwise unused.
 * (ViT-L/16, N = 256, bf16: about 645 MB.)  vitblk_forward_packed() needs
 * only the activations: vitblk_workspace_bytes() minus
 * vitblk_packed_weights_bytes().
 */
size_t vitblk_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                              int dtype);

/*
 * Out-major ("packed") copies of the six weights, the layout the GEMM kernels
 * read: both operands of every product contiguous along the reduction axis.
 * Regions, each on a 256-byte boundary, in this order:
 *   Wqkv^T [3D, D]  row n < D is column n of w_q, rows D..2D-1 columns of
 *                   w_k, rows 2D..3D-1 columns of w_v
 *   Wo^T   [D, D]
 *   W1^T   [F, D]   (w_mlp1 is [D, F])
 *   W2^T   [D, F]   (w_mlp2 is [F, D])
 *   cs_qkv [3D]     fp32: cs_qkv[n] = sum_k Wqkv[k, n], the column sums of
 *                   [w_q | w_k | w_v] (row sums of Wqkv^T), summed in fp32
 *   cs_1   [F]      fp32: the column sums of w_mlp1
 * The column sums serve the products that fold a LayerNorm in (see
 * vitblk_linear_normed()).  vitblk_packed_weights_bytes() returns the size
 * (0 for invalid arguments; host only).  vitblk_pack_weights() writes it on
 * `stream` (bf16 with every side a multiple of 8 and 16-byte aligned
 * weights: one launch, the sums taken from the source weights; otherwise two:
 * the transposes, then the packed copies' row sums); the buffer must
 * not overlap a weight.  Callers that run many blocks with the same weights
 * pack once and call vitblk_forward_packed().
 */
size_t vitblk_packed_weights_bytes(int64_t D, int64_t F, int dtype);

int vitblk_pack_weights(const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                        const void* w_mlp1, const void* w_mlp2, void* packed, int64_t D,
                        int64_t F, int dtype, vitblk_stream_t stream);

/*
 * One encoder block forward: out = block(x).
 *
 *   x      [N, T, D]  N independent sequences of T tokens of width D
 *   w_q, w_k, w_v, w_o  [D, D]
 *   w_mlp1 [D, F],  w_mlp2 [F, D]
 *   out    [N, T, D]  must not overlap any input or the workspace
 *   H      number of heads; must divide D (head width D/H <= 1024)
 *   eps    LayerNorm epsilon, finite and >= 0 (eps = 0 gives NaN for a
 *          constant token, as the formula does)
 *   dtype  VITBLK_FP32 or VITBLK_BF16, the type of every tensor
 *   workspace, workspace_bytes  caller-owned device scratch of at least
 *          vitblk_workspace_bytes(N, T, D, F, H, dtype) bytes; its contents
 *          on entry are ignored and on return are unspecified
 *
 * Kernels run in order on `stream`: weight packing (and the column sums),
 * LN, fused QKV projection, attention, output projection + residual, LN,
 * MLP1 + GELU, MLP2 + residual.  In bf16 each LN (no gain or shift) is
 * folded into the product that follows it: only the rows' mean and
 * 1/sqrt(var + eps) are computed, and the product's epilogue forms
 * rstd * (x @ W - mean * colsum(W)) = LN(x) @ W (see vitblk_linear_normed());
 * the first LN's statistics are computed in the weight-packing launch when
 * that launch is a single one (see vitblk_pack_weights()).
 * When the last rows of a residual product would leave most of the device
 * idle, their K range is split and a second kernel adds the partial sums
 * (fp32, in the workspace) to the residual.
 */
int vitblk_forward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                   const void* w_o, const void* w_mlp1, const void* w_mlp2, void* out,
                   int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                   int dtype, void* workspace, size_t workspace_bytes,
                   vitblk_stream_t stream);

/*
 * Optional parameters of the affine block variant
 * (ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "Key Equations":
 * step 1 and step 4, a LayerNorm with a per-feature gain gamma and shift beta,
 * each LayerNorm with its own; step 5, the MLP's biases b_1 and b_2; the
 * nn.Linear projections of the nipunbatra.github.io vision1 transcript,
 * Pages 24-26, give Q, K, V and the output projection a bias too):
 *
 *   xn  = LN(x) * ln1_gamma + ln1_beta
 *   Q, K, V = xn @ w_q + b_q, xn @ w_k + b_k, xn @ w_v + b_v
 *   y   = x + att @ w_o + b_o
 *   yn  = LN(y) * ln2_gamma + ln2_beta
 *   out = y + GELU_tanh(yn @ w_mlp1 + b_mlp1) @ w_mlp2 + b_mlp2
 *
 * Every member is a device pointer to a vector in the block's dtype, 16-byte
 * aligned, or NULL for "absent" (gain 1, shift 0, bias 0).  Lengths: D for
 * all of them except b_mlp1, which has F.  A NULL parameter set is the plain
 * block.  The parameters are read directly by the kernels (no copy); they
 * must not overlap out or the workspace (VITBLK_ERR_ALIAS).
 */
typedef struct {
  const void* ln1_gamma;
  const void* ln1_beta;
  const void* b_q;
  const void* b_k;
  const void* b_v;
  const void* b_o;
  const void* ln2_gamma;
  const void* ln2_beta;
  const void* b_mlp1;
  const void* b_mlp2;
} vitblk_affine_params;

/*
 * vitblk_forward() with the affine variant's parameters (may be NULL).  The
 * biases enter the products in fp32 (before GELU and before the residual
 * add).  In bf16 each LayerNorm with a gain or shift is folded into the
 * product after it as the plain block's are (vitblk_affine_fold()'s scaled
 * weight copy, column sums and bias, per call, in workspace regions that are
 * dead at that point) when those regions hold the copy (N T >= 3 D and
 * about N T >= F); otherwise, and in fp32, the LayerNorm kernel applies the
 * gain and shift.  Same workspace and errors as vitblk_forward().
 */
int vitblk_forward_affine(const void* x, const void* w_q, const void* w_k, const void* w_v,
                          const void* w_o, const void* w_mlp1, const void* w_mlp2,
                          const vitblk_affine_params* params, void* out, int64_t N, int64_t T,
                          int64_t D, int64_t F, int64_t H, double eps, int dtype,
                          void* workspace, size_t workspace_bytes, vitblk_stream_t stream);

/*
 * The same block on weights already packed by vitblk_pack_weights() (the
 * seven kernels after packing).  workspace must hold at least
 * vitblk_workspace_bytes() - vitblk_packed_weights_bytes() bytes and must not
 * overlap x, packed or out.
 */
int vitblk_forward_packed(const void* x, const void* packed, void* out, int64_t N, int64_t T,
                          int64_t D, int64_t F, int64_t H, double eps, int dtype,
                          void* workspace, size_t workspace_bytes, vitblk_stream_t stream);

/*
 * vitblk_forward_packed() for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the activations live in a scratch array inside the library (a
 * file-scope __device__ array of VITBLK_NOALLOC_SCRATCH_BYTES bytes, one per
 * GPU the library runs on, held until the process ends) instead of a caller
 * workspace.  The call allocates nothing.  The caller still owns x, packed
 * and out (device pointers on the GPU that `stream` belongs to).
 *
 * Limit: vitblk_workspace_bytes(N, T, D, F, H, dtype) -
 * vitblk_packed_weights_bytes(D, F, dtype) must not exceed
 * VITBLK_NOALLOC_SCRATCH_BYTES (e.g. ViT-L/16 width: up to 27 sequences of
 * 197 tokens); larger sizes return VITBLK_ERR_WORKSPACE and launch nothing.
 * Every call on one GPU uses that GPU's single scratch array, which keeps
 * the last call's contents (nothing in it needs to start at zero): calls
 * that overlap in time on one GPU (other host threads, or streams that run
 * concurrently) race, and the caller must order them.  The results are
 * those of vitblk_forward_packed() on the same inputs, bit for bit.
 * Other errors as vitblk_forward_packed(); VITBLK_ERR_HIP if the scratch
 * array's address cannot be resolved on the stream's device.
 */
#define VITBLK_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int vitblk_forward_packed_noalloc(const void* x, const void* packed, void* out, int64_t N,
                                  int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                                  int dtype, vitblk_stream_t stream);

/* vitblk_forward_packed() with the affine variant's parameters (may be NULL). */
int vitblk_forward_packed_affine(const void* x, const void* packed,
                                 const vitblk_affine_params* params, void* out, int64_t N,
                                 int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                                 int dtype, void* workspace, size_t workspace_bytes,
                                 vitblk_stream_t stream);

/*
 * The front end: images to the tokens the encoder takes (mlgrind.dev "E2E:
 * Tiny Vision Transformer", "Architecture": patchify, @ W_patch + b_patch,
 * prepend the class token, add position embeddings; "Details": patches in
 * row-major order over the (H/P, W/P) grid, each flattened as (p1, p2, c),
 * the same map as a stride-P convolution):
 *
 *   patches[b, i*(W/P) + j, (p1*P + p2)*C + c] = images[b, c, i*P + p1, j*P + p2]
 *   tokens[b] = [cls_token ; patches[b] @ w_patch + b_patch] + pos_emb
 *
 *   images     [B, C, H, W]; H and W multiples of P
 *   w_patch    [P*P*C, D] (x @ W orientation)
 *   b_patch    [D] or NULL; cls_token [D] or NULL (no class token: T = N);
 *   pos_emb    [T, D] or NULL, T = N + (cls_token != NULL), N = (H/P)(W/P)
 *   tokens     [B, T, D]; must not overlap an input or the workspace
 *   workspace  at least vitblk_patch_embed_workspace_bytes() bytes
 *
 * Five kernels: W_patch transposed into the workspace (and its padding
 * zeroed: the patch width is padded to a multiple of 64), the patch matrix,
 * the embedding GEMM with its bias, the token rows.
 */
size_t vitblk_patch_embed_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W,
                                          int64_t P, int64_t D, int dtype);

int vitblk_patch_embed(const void* images, const void* w_patch, const void* b_patch,
                       const void* cls_token, const void* pos_emb, void* tokens, int64_t B,
                       int64_t C, int64_t H, int64_t W, int64_t P, int64_t D, int dtype,
                       void* workspace, size_t workspace_bytes, vitblk_stream_t stream);

/*
 * The encoder stack: L blocks in sequence, each with its own packed weights
 * (and, optionally, its own affine parameters), then a final LayerNorm with
 * its own gain and shift (ai-engineer-exhaustive.pages.dev "ViT Encoder
 * Block", "What It Is": L identical blocks with their own weights, L = 12,
 * 24, 32 for ViT-B/L/H; mlgrind.dev "E2E: Tiny Vision Transformer",
 * "Architecture": cls = LN_f(t[:, 0]) after the last block):
 *
 *   t_0 = x;  t_l = block_l(t_{l-1}), l = 1..L
 *   out     = LN(t_L) * final_gamma + final_beta          [N, T, D]
 *   cls_out = LN(t_L[:, 0, :]) * final_gamma + final_beta [N, D]
 *
 *   packed  HOST array of L device pointers, each a buffer written by
 *           vitblk_pack_weights() (the block's six weights, out-major)
 *   params  HOST array of L vitblk_affine_params, or NULL for plain blocks
 *   final_gamma, final_beta  [D] device vectors, each may be NULL (1, 0)
 *   out, cls_out  either may be NULL, not both; neither may overlap an
 *           input, the other output or the workspace
 *   workspace  at least vitblk_encoder_workspace_bytes() bytes: one block's
 *           activations plus two [N*T, D] token buffers the blocks alternate
 *           between (x itself is never written)
 *
 * With out NULL only the class tokens leave the stack (nipunbatra.github.io
 * "Vision Transformer - optional labs and references", page 55 "Follow the
 * CLS row from scores to weights": a CLS-only readout needs just the class
 * query's row from the last block, with all its keys and values): the last block
 * then computes every token's Q, K and V but attention for the first 32
 * queries of each sequence only, and its output projection, second
 * LayerNorm and MLP for the N class-token rows.  The values are those of the
 * full stack up to rounding (its products' K sums may run in another order).
 *
 * 7 L + 1 or 2 kernels on `stream`.
 */
size_t vitblk_encoder_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                                      int dtype);

int vitblk_encoder_forward(const void* x, const void* const* packed,
                           const vitblk_affine_params* params, int64_t L,
                           const void* final_gamma, const void* final_beta, void* out,
                           void* cls_out, int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                           double eps, int dtype, void* workspace, size_t workspace_bytes,
                           vitblk_stream_t stream);

/*
 * The steps of the block, one call each, on the same kernels vitblk_forward
 * uses.  They exist so that each step can be checked and timed alone and so
 * that callers can compose blocks of their own.
 */

/* out[r, :] = LN(x[r, :]) for r < rows; x, out [rows, D].  LN as above
 * (crackedaicode.com "ViT Encoder Block", "Normalize before each stage").
 * out must not overlap x. */
int vitblk_layernorm(const void* x, void* out, int64_t rows, int64_t D, double eps,
                     int dtype, vitblk_stream_t stream);

/* out[r, :] = LN(x[r, :]) * gamma + beta: the affine LayerNorm of
 * ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "Key Equations"
 * step 1.  gamma and beta ([D], 16-byte aligned) may each be NULL (1, 0);
 * out must not overlap x, gamma or beta. */
int vitblk_layernorm_affine(const void* x, const void* gamma, const void* beta, void* out,
                            int64_t rows, int64_t D, double eps, int dtype,
                            vitblk_stream_t stream);

/* LayerNorm statistics of each row of x [rows, D]: stats[2r] = mean,
 * stats[2r + 1] = 1 / sqrt(var + eps) (population variance; fp32, the values
 * vitblk_layernorm() normalises with).  stats (2 * rows floats, 8-byte
 * aligned) must not overlap x. */
int vitblk_row_stats(const void* x, float* stats, int64_t rows, int64_t D, double eps,
                     int dtype, vitblk_stream_t stream);

/* A product whose left operand is the LayerNorm (no gain or shift) of a,
 * with the normalisation folded into the epilogue:
 *
 *   out = epilogue(LN(a) @ W + bias),  LN(a) @ W = rstd_m (a @ W - mean_m c_n)
 *
 * (the LayerNorm of crackedaicode.com "ViT Encoder Block", "Normalize before
 * each stage", is (a - mean) * rstd per row; multiplied out, the mean term
 * is the row's mean times W's column sum).  a [M, K] is the raw input (not
 * normalised), row_stats its statistics from vitblk_row_stats(), col_sums
 * [Nout] fp32 the column sums of W (16-byte aligned; the packed weights
 * hold them for the QKV and MLP1 products), w_t, bias and out as for
 * vitblk_linear_bias().  epilogue: VITBLK_EPI_NONE or VITBLK_EPI_GELU.  The
 * difference from normalising first is rounding only: a is used as given
 * (no rounding of LN(a) to the dtype); the fp32 subtraction adds an error
 * of about 2^-24 sqrt(K) |mean| / std relative to the output. */
int vitblk_linear_normed(const void* a, const void* w_t, const float* col_sums,
                         const float* row_stats, const void* bias, void* out, int64_t M,
                         int64_t K, int64_t Nout, int epilogue, int dtype,
                         vitblk_stream_t stream);

/* The affine LayerNorm folded into the product after it (bf16 only).  For
 * the LayerNorm gain gamma [K] and shift beta [K]
 * (ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "Key Equations",
 * steps 1 and 4), W given out-major (w_t [Nout, K]) and the product's bias
 * [Nout]:
 *
 *   w_scaled[n, k] = bf16(gamma_k * w_t[n, k])
 *   col_sums[n]    = sum_k w_scaled[n, k]              (fp32, fixed order)
 *   bias_out[n]    = bf16(bias_n + sum_k beta_k * w_t[n, k])
 *
 * so that vitblk_linear_normed(a, w_scaled, col_sums, row_stats(a), bias_out)
 * is (LN(a) * gamma + beta) @ W + bias up to rounding (LN(a) * gamma @ W =
 * rstd (a @ diag(gamma) W - mean colsum(diag(gamma) W))).  gamma, beta and
 * bias may each be NULL (ones, zeros, zeros).  K a multiple of 8; w_t,
 * w_scaled, gamma, beta and col_sums 16-byte aligned; the three outputs must
 * not overlap the inputs or each other.  Other dtypes: VITBLK_ERR_UNSUPPORTED. */
int vitblk_affine_fold(const void* w_t, const void* gamma, const void* beta, const void* bias,
                       void* w_scaled, float* col_sums, void* bias_out, int64_t Nout, int64_t K,
                       int dtype, vitblk_stream_t stream);

/* The output projection with the first residual and the second LayerNorm's
 * statistics: out = residual + a @ W (a [M, K], w_t [Nout, K] out-major as
 * for vitblk_linear(), residual and out [M, Nout]), then row_stats[2m],
 * row_stats[2m + 1] = mean and 1 / sqrt(var + eps) of row m of out as stored
 * (population variance), the pair vitblk_linear_normed() takes.
 * crackedaicode.com "ViT Encoder Block", "Multi-head attention" (y = x +
 * attention @ w_o) and "Feed-forward stage" (LN of y).  In bf16 with Nout a
 * multiple of 64 the product's epilogue writes each row's (mean, M2) over
 * every 64 columns into the workspace and one small kernel combines them
 * (the raw second moment of 32 values per lane: relative error of the
 * variance about 2^-19 (1 + mean^2 / var)); otherwise the plain product is
 * followed by vitblk_row_stats()'s kernel.  workspace: at least
 * vitblk_linear_residual_row_stats_workspace_bytes(M, Nout) bytes, 16-byte
 * aligned, its contents clobbered.  row_stats is fp32, 8-byte aligned; no
 * output may overlap an input, the other output or the workspace. */
size_t vitblk_linear_residual_row_stats_workspace_bytes(int64_t M, int64_t Nout);

int vitblk_linear_residual_row_stats(const void* a, const void* w_t, const void* residual,
                                     void* out, float* row_stats, int64_t M, int64_t K,
                                     int64_t Nout, double eps, int dtype, void* workspace,
                                     size_t workspace_bytes, vitblk_stream_t stream);

/* qkv = xn @ [w_q | w_k | w_v]: xn [M, D], w_qkv_t [3D, D] (the first
 * region of the packed weights), qkv [M, 3D] (one row holds a token's Q, K
 * and V, each as H consecutive head chunks).  crackedaicode.com "ViT Encoder
 * Block", "Multi-head attention" (the three projections); mlgrind.dev "E2E:
 * Tiny Vision Transformer", "Details" (one product with a concatenated
 * weight).  qkv must not overlap an input. */
int vitblk_qkv_projection(const void* xn, const void* w_qkv_t, void* qkv, int64_t M,
                          int64_t D, int dtype, vitblk_stream_t stream);

/* Bidirectional multi-head attention over packed qkv [N*T, 3D] (as written
 * by vitblk_qkv_projection): for every sequence n and head h,
 * att[n, :, h*dh:(h+1)*dh] = softmax(Q_h K_h^T / sqrt(dh)) V_h with dh = D/H,
 * no mask.  att is [N*T, D] (heads concatenated in order) and must not
 * overlap qkv.  crackedaicode.com "ViT Encoder Block", "Multi-head
 * attention". */
int vitblk_attention(const void* qkv, void* att, int64_t N, int64_t T, int64_t D,
                     int64_t H, int dtype, vitblk_stream_t stream);

/* The same attention for the first queries of each sequence only, every key
 * entering their softmax: rows n*T + t of att with t < min(T, 32) are
 * written exactly as vitblk_attention() writes them; the other rows may or
 * may not be written.  It serves a readout that needs only the class token
 * (query 0): mlgrind.dev "E2E: Tiny Vision Transformer", "Architecture" (the
 * class token's final state is the image's representation), with the same
 * kernels as the class-token-only last block of vitblk_encoder_forward().
 * Same arguments and errors as vitblk_attention(). */
int vitblk_attention_first_queries(const void* qkv, void* att, int64_t N, int64_t T, int64_t D,
                                   int64_t H, int dtype, vitblk_stream_t stream);

/* out = epilogue(a @ W) with the weight given out-major: a [M, K],
 * w_t [Nout, K] (row n = column n of the (in, out) weight W, as in the
 * packed regions), out [M, Nout]; residual [M, Nout] is read only for
 * VITBLK_EPI_RESIDUAL and VITBLK_EPI_GELU_GRAD (there it holds the GELU's
 * input z; may be NULL otherwise).  Covers the output projection
 * + first residual, MLP1 + GELU and MLP2 + second residual
 * (crackedaicode.com "ViT Encoder Block", "Multi-head attention" and
 * "Feed-forward stage").  out must not overlap a, w_t or residual. */
int vitblk_linear(const void* a, const void* w_t, const void* residual, void* out,
                  int64_t M, int64_t K, int64_t Nout, int epilogue, int dtype,
                  vitblk_stream_t stream);

/* vitblk_linear() with a bias ([Nout], 16-byte aligned, or NULL) added to
 * a @ W in fp32 before the epilogue: out = epilogue(a @ W + bias), i.e.
 * GELU_tanh(a @ W + bias) or residual + a @ W + bias
 * (ai-engineer-exhaustive.pages.dev "ViT Encoder Block", "Key Equations"
 * step 5).  out must not overlap the bias either. */
int vitblk_linear_bias(const void* a, const void* w_t, const void* bias, const void* residual,
                       void* out, int64_t M, int64_t K, int64_t Nout, int epilogue, int dtype,
                       vitblk_stream_t stream);

/*
 * ------------------------------------------------------------------------
 * Backward pass of the plain block (training; the gradients autograd would
 * produce: nipunbatra.github.io vision1 transcript, Page 88 -- backward()
 * fills dL/dtheta for every block -- and Page 113, one training step;
 * mlgrind.dev "E2E: Tiny Vision Transformer", "Method contract": every
 * parameter is trained).
 *
 * Given dout = dL/d(out) for out = block(x) (the plain block above), write
 *   dx      = dL/dx                                  [N, T, D]
 *   dw_q, dw_k, dw_v, dw_o = dL/dw_*                 [D, D]
 *   dw_mlp1 = dL/dw_mlp1 [D, F],  dw_mlp2 = dL/dw_mlp2 [F, D]
 * i.e. the exact derivative of the forward definition (the vector-Jacobian
 * product with dout).  The weight gradients are written, not accumulated:
 * each is the sum over all N*T tokens of the call.
 *
 * The forward activations are recomputed inside the call (x and the weights
 * are all it needs), then the steps are walked in reverse:
 *   dW2 = h^T dout;  dz = (dout W2^T) * GELU'(z);  dW1 = yn^T dz;
 *   dy  = dout + LN'(y)^T (dz W1^T);  dWo = att^T dy;  datt = dy Wo^T;
 *   dq, dk, dv = attention backward (softmax gradient per head);
 *   dWq|dWk|dWv = xn^T [dq|dk|dv];  dx = dy + LN'(x)^T ([dq|dk|dv] [Wq|Wk|Wv]^T)
 * with h = GELU(z), z = yn W1, yn = LN(y), att the concatenated heads.
 *
 * Precision: as in the forward (bf16 operands and stored intermediates, fp32
 * accumulation and statistics); the weight gradients are reduced in fp32 and
 * rounded once.  Arguments: as vitblk_forward, plus dout [N, T, D] (input)
 * and the seven outputs, which must not overlap each other, an input or the
 * workspace.  workspace: at least vitblk_backward_workspace_bytes() bytes
 * (the forward's packed weights and activations, the concatenated
 * [w_q | w_k | w_v], the gradient buffers and the fp32 partial sums of the
 * weight gradients; about 1.8 GB for ViT-L/16 with N = 256 in bf16).
 */
size_t vitblk_backward_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                                       int dtype);

int vitblk_backward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                    const void* w_o, const void* w_mlp1, const void* w_mlp2, const void* dout,
                    void* dx, void* dw_q, void* dw_k, void* dw_v, void* dw_o, void* dw_mlp1,
                    void* dw_mlp2, int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                    double eps, int dtype, void* workspace, size_t workspace_bytes,
                    vitblk_stream_t stream);

/* The backward's steps, one call each (same kernels as vitblk_backward). */

/* Weight gradient of a projection: out[i, j] = sum_m a[m, i] * b[m, j] over
 * the M token rows, i.e. out = a^T b with a [M, I] (the projection's input)
 * and b [M, J] (the gradient of its output); out [I, J].  Reduced in fp32
 * (split over the token rows into fp32 partial sums held in the workspace,
 * then summed in a fixed order: deterministic) and rounded once.  workspace:
 * at least vitblk_weight_grad_workspace_bytes(M, I, J) bytes.  out must not
 * overlap a, b or the workspace. */
size_t vitblk_weight_grad_workspace_bytes(int64_t M, int64_t I, int64_t J);

int vitblk_weight_grad(const void* a, const void* b, void* out, int64_t M, int64_t I, int64_t J,
                       int dtype, void* workspace, size_t workspace_bytes,
                       vitblk_stream_t stream);

/* Backward of LN (as in vitblk_layernorm: no gain or shift) plus a residual
 * gradient: dx[r, :] = residual[r, :] + J_r^T g[r, :], where J_r is the
 * Jacobian of LN at x[r, :], i.e.
 *   dx = residual + rstd * (g - mean(g) - xhat * mean(g * xhat)),
 *   xhat = (x - mean(x)) * rstd, rstd = 1 / sqrt(var(x) + eps).
 * x, g, dx [rows, D]; residual [rows, D] or NULL (zero).  dx must not
 * overlap x, g or residual. */
int vitblk_layernorm_backward(const void* x, const void* g, const void* residual, void* dx,
                              int64_t rows, int64_t D, double eps, int dtype,
                              vitblk_stream_t stream);

/* Backward of vitblk_attention: given qkv [N*T, 3D] (the forward's input)
 * and datt = dL/d(att) [N*T, D], write dqkv [N*T, 3D] = [dQ | dK | dV] with,
 * per sequence and head, P = softmax(Q_h K_h^T / sqrt(dh)),
 *   dV_h = P^T dO_h,  dS = P * (dO_h V_h^T - rowsum(P * dO_h V_h^T)),
 *   dQ_h = dS K_h / sqrt(dh),  dK_h = dS^T Q_h / sqrt(dh).
 * workspace: at least vitblk_attention_backward_workspace_bytes() bytes
 * (per-query softmax statistics).  dqkv must not overlap qkv, datt or the
 * workspace. */
size_t vitblk_attention_backward_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t H);

int vitblk_attention_backward(const void* qkv, const void* datt, void* dqkv, int64_t N, int64_t T,
                              int64_t D, int64_t H, int dtype, void* workspace,
                              size_t workspace_bytes, vitblk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VITBLK_H */
