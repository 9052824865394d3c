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
 * applied as x @ W.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers named x, w_*, out, qkv, ... are DEVICE pointers (HIP global
 *   memory) on the current device, owned by the caller.  The library never
 *   allocates, frees or retains memory, holds no state between calls, and is
 *   re-entrant.  Calls enqueue on `stream` (0 = the null stream) and return
 *   without synchronising; the caller synchronises before reading results.
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
  VITBLK_EPI_GELU = 2      /* out = GELU_tanh(a @ w)           */
} vitblk_epilogue;

/* Human-readable name of a vitblk_status value (static storage; never NULL). */
const char* vitblk_status_string(int status);

/*
 * Bytes of device workspace vitblk_forward() needs for these sizes, or 0 if
 * the arguments are invalid.  Pure host function: no HIP call.
 *
 * Layout (each region starts on a 256-byte boundary), es = element size:
 *   region 0: M x max(3D, F) elements: packed Q|K|V [M, 3D], later the
 *             MLP hidden activations [M, F]
 *   region 1: M x D elements: LN(x), later the concatenated heads, later LN(y)
 *   region 2: M x D elements: y = x + att @ w_o
 * with M = N*T.  (ViT-L/16, N = 256, bf16: about 620 MB.)
 */
size_t vitblk_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                              int dtype);

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
 * Seven kernels run in order on `stream`: LN, fused QKV projection,
 * attention, output projection + residual, LN, MLP1 + GELU, MLP2 + residual.
 */
int vitblk_forward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                   const void* w_o, const void* w_mlp1, const void* w_mlp2, void* out,
                   int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                   int dtype, void* workspace, size_t workspace_bytes,
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

/* qkv[:, 0:D] = xn @ w_q, qkv[:, D:2D] = xn @ w_k, qkv[:, 2D:3D] = xn @ w_v;
 * xn [M, D], w_* [D, D], qkv [M, 3D] (one row holds a token's Q, K and V,
 * each as H consecutive head chunks).  crackedaicode.com "ViT Encoder Block",
 * "Multi-head attention" (the three projections); mlgrind.dev "E2E: Tiny
 * Vision Transformer", "Details" (one product with a concatenated weight).
 * qkv must not overlap an input. */
int vitblk_qkv_projection(const void* xn, const void* w_q, const void* w_k,
                          const void* w_v, void* qkv, int64_t M, int64_t D, int dtype,
                          vitblk_stream_t stream);

/* Bidirectional multi-head attention over packed qkv [N*T, 3D] (as written
 * by vitblk_qkv_projection): for every sequence n and head h,
 * att[n, :, h*dh:(h+1)*dh] = softmax(Q_h K_h^T / sqrt(dh)) V_h with dh = D/H,
 * no mask.  att is [N*T, D] (heads concatenated in order) and must not
 * overlap qkv.  crackedaicode.com "ViT Encoder Block", "Multi-head
 * attention". */
int vitblk_attention(const void* qkv, void* att, int64_t N, int64_t T, int64_t D,
                     int64_t H, int dtype, vitblk_stream_t stream);

/* out = epilogue(a @ w): a [M, K], w [K, Nout], out [M, Nout]; residual
 * [M, Nout] is read only for VITBLK_EPI_RESIDUAL (may be NULL otherwise).
 * Covers the output projection + first residual, MLP1 + GELU and
 * MLP2 + second residual (crackedaicode.com "ViT Encoder Block",
 * "Multi-head attention" and "Feed-forward stage").  out must not overlap
 * a, w or residual. */
int vitblk_linear(const void* a, const void* w, const void* residual, void* out,
                  int64_t M, int64_t K, int64_t Nout, int epilogue, int dtype,
                  vitblk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* VITBLK_H */
