// Internal launch interface of the vitblk kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vitblk {

// C[m, n] = epi(sum_k A[m, k] * Wt[n, k] + b[n]) (+ R[m, n]) for m < M, n < N.
// A [M, K] with row stride lda; the weight is given out-major, Wt [N, K] with
// row stride ldb (row n = column n of the (in, out) weight); C and R have row
// strides ldc and ldr.  All strides in elements.  The bias is optional and
// given in segments of bias_seg columns: b[n] = bias[n / bias_seg][n %
// bias_seg] (one segment per Q, K, V in the fused projection); a null
// segment is zero, and all three null means no bias.
struct GemmProblem {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C;
  int64_t ldc;
  const void* R;
  int64_t ldr;
  int epi;    // vitblk_epilogue
  int dtype;  // vitblk_dtype
  const void* bias[3];
  int64_t bias_seg;
};

__host__ __device__ inline bool has_bias(const GemmProblem& p) {
  return p.bias[0] != nullptr || p.bias[1] != nullptr || p.bias[2] != nullptr;
}

// One (in, out) weight to write out-major: dst[c * ldd + r] = src[r * cols + c].
struct PackJob {
  const void* src;
  int64_t rows, cols;
  void* dst;
  int64_t ldd;
};

// y = LN(x) * gamma + beta per row; gamma and beta ([D]) may be null (1, 0).
// Input row r starts at x + r * ld_in elements (ld_in >= D); y is [rows, D].
hipError_t launch_layernorm(const void* x, int64_t ld_in, const void* gamma, const void* beta,
                            void* y, int64_t rows, int64_t D, float eps, int dtype,
                            hipStream_t stream);

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);

// The front end: images [B, C, H, W] -> tokens [B, N (+1), D] (patch matrix,
// embedding GEMM, token assembly); w_t, patches and embedded are workspace.
struct PatchEmbedArgs {
  const void* images;
  const void* w_patch;  // [P*P*C, D]
  const void* b_patch;  // [D] or null
  const void* cls;      // [D] or null
  const void* pos;      // [N (+1), D] or null
  void* tokens;         // [B, N (+1), D]
  void* w_t;            // [D, Kp]
  void* patches;        // [B*N, Kp]
  void* embedded;       // [B*N, D]
  int64_t B, C, H, W, P, D, Kp;
  int dtype;
};

hipError_t launch_patch_embed(const PatchEmbedArgs& p, hipStream_t stream);

// Transpose up to 6 weights in one launch.
hipError_t launch_pack(const PackJob* jobs, int njobs, int dtype, hipStream_t stream);

// O[n*T + t, h*dh + c] = sum_j softmax_j(Q_h K_h^T / sqrt(dh))[t, j] V[n*T + j, h*dh + c]
// with Q, K, V row strides ld (elements) and O row stride ldo.
hipError_t launch_attention(const void* q, const void* k, const void* v, int64_t ld,
                            void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                            int64_t dh, int dtype, hipStream_t stream);

// Whole-sequence-in-LDS variant (bf16); hipErrorNotSupported when it does not
// apply (sequence too long for LDS, head width without an instantiation).
hipError_t launch_attention_resident(const void* q, const void* k, const void* v, int64_t ld,
                                     void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                     int64_t dh, hipStream_t stream);

// Generic (any-shape, VALU, fp32 arithmetic) kernels; the fast kernels fall
// back to these for shapes they do not tile and for fp32 tensors.
hipError_t launch_layernorm_generic(const void* x, int64_t ld_in, const void* gamma,
                                    const void* beta, void* y, int64_t rows, int64_t D,
                                    float eps, int dtype, hipStream_t stream);
hipError_t launch_gemm_generic(const GemmProblem& p, hipStream_t stream);
hipError_t launch_attention_generic(const void* q, const void* k, const void* v, int64_t ld,
                                    void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                    int64_t dh, int dtype, hipStream_t stream);

}  // namespace vitblk
