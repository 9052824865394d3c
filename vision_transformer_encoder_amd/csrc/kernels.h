// Internal launch interface of the vitblk kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vitblk {

// C[m, col_off[p] + n] = epi(sum_k A[m, k] * B[p][k, n]) (+ R[m, col_off[p] + n])
// for problem p < nprob, m < M, n < N.  A [M, K] with row stride lda,
// B[p] [K, N] with row stride ldb, C and R with row strides ldc, ldr.
// One launch covers all problems (the three Q/K/V projections share A).
struct GemmProblem {
  int64_t M, N, K;
  const void* A;
  int64_t lda;
  int nprob;
  const void* B[3];
  int64_t ldb;
  void* C;
  int64_t ldc;
  int64_t col_off[3];
  const void* R;
  int64_t ldr;
  int epi;    // vitblk_epilogue
  int dtype;  // vitblk_dtype
};

hipError_t launch_layernorm(const void* x, void* y, int64_t rows, int64_t D, float eps,
                            int dtype, hipStream_t stream);

hipError_t launch_gemm(const GemmProblem& p, hipStream_t stream);

// O[n*T + t, h*dh + c] = sum_j softmax_j(Q_h K_h^T / sqrt(dh))[t, j] V[n*T + j, h*dh + c]
// with Q, K, V row strides ld (elements) and O row stride ldo.
hipError_t launch_attention(const void* q, const void* k, const void* v, int64_t ld,
                            void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                            int64_t dh, int dtype, hipStream_t stream);

// Generic (any-shape, VALU, fp32 arithmetic) kernels; the fast kernels fall
// back to these for shapes they do not tile and for fp32 tensors.
hipError_t launch_layernorm_generic(const void* x, void* y, int64_t rows, int64_t D,
                                    float eps, int dtype, hipStream_t stream);
hipError_t launch_gemm_generic(const GemmProblem& p, hipStream_t stream);
hipError_t launch_attention_generic(const void* q, const void* k, const void* v, int64_t ld,
                                    void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                    int64_t dh, int dtype, hipStream_t stream);

}  // namespace vitblk
