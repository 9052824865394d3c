// Internal launch interface of the vitblk kernels (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitblk.h"

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
  void* C2;  // second output of kEpiGeluDual (same layout as C), else unused
  // LayerNorm folded into a product whose left operand is LN(A) (no gain or
  // shift): the product becomes rstd_m * (A @ W - mean_m * colsum_n), added
  // before the bias and the epilogue, with (mean_m, rstd_m) = row_stats[2m],
  // row_stats[2m + 1] (row m of A) and colsum_n = col_sums[n] = sum_k W[k, n]
  // (of the operand as stored).  Both null: a plain product.  Epilogues NONE
  // and GELU only.
  const float* row_stats;
  const float* col_sums;
  // kEpiPartial only: the number of k-ranges (>= 1).
  int ksplit;
  // Free fp32 device memory launch_gemm may use for split-K partial sums of
  // a residual product (null: none).  Its contents are clobbered.
  float* scratch;
  int64_t scratch_floats;
  // kEpiResidualStats only: row_partials[m * (N / 64) + n / 64] = (mean, M2)
  // of the stored (rounded) outputs of row m over columns [n, n + 64), n a
  // multiple of 64 (M2 = the sum of squared deviations from that mean).
  float2* row_partials;
  // kEpiEmbed only: product row g = row_base + m (m the row within this
  // launch) is token cell = g % row_group of image g / row_group; it goes to
  // C row g + row_skip * (g / row_group + 1) and adds R row row_skip + cell
  // (C and R are not offset by row_base).
  int64_t row_group, row_base;
  int64_t row_skip;
};

// Internal epilogues of the backward (not part of the C interface):
// kEpiGeluDual: C = GELU_tanh(acc), C2 = GELU_tanh'(acc) (the recomputed MLP
// hidden layer and its derivative, from one product); kEpiMul: C = acc * R.
constexpr int kEpiGeluDual = 16;
constexpr int kEpiMul = 17;
// kEpiPartial: split K.  Tile (m, n) of k-range s of ksplit equal ranges is
// written, unrounded, to ((float*)C)[s * M * ldc + m * ldc + n]; no bias.
constexpr int kEpiPartial = 18;
// kEpiResidualStats: the residual epilogue, plus the row partials above (the
// next LayerNorm's statistics, combined by launch_row_stats_from_partials).
constexpr int kEpiResidualStats = 19;
// kEpiEmbed: the patch-embedding product written straight into the token
// rows with the position embedding added (fields row_group, row_base,
// row_skip above; bf16 MFMA kernel only).
constexpr int kEpiEmbed = 20;
// Columns per row partial of kEpiResidualStats (every tile's wave strip).
constexpr int kStatsStrip = 64;

__host__ __device__ inline bool has_bias(const GemmProblem& p) {
  return p.bias[0] != nullptr || p.bias[1] != nullptr || p.bias[2] != nullptr;
}

// Epilogues that read R (the residual, or GELU's input for its derivative).
__host__ __device__ inline bool reads_r(const GemmProblem& p) {
  return p.epi == VITBLK_EPI_RESIDUAL || p.epi == VITBLK_EPI_GELU_GRAD || p.epi == kEpiMul ||
         p.epi == kEpiResidualStats || p.epi == kEpiEmbed;
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

// Whether the residual product p can also write its rows' partial statistics
// (kEpiResidualStats) on the matrix-core kernel.
bool gemm_row_partials_ok(const GemmProblem& p);

// stats[2r], stats[2r + 1] = mean and 1 / sqrt(M2 / D + eps) of row r from its
// nstrips = D / kStatsStrip partials (kEpiResidualStats), combined in order.
hipError_t launch_row_stats_from_partials(const float2* partials, int64_t nstrips, float* stats,
                                          int64_t rows, int64_t D, float eps, hipStream_t stream);

// Whether the matrix-core kernels take p (otherwise the generic kernel does).
bool gemm_fast_ok(const GemmProblem& p);

// stats[2r], stats[2r + 1] = mean and 1 / sqrt(var + eps) of row r of x
// (population variance, fp32, the same arithmetic as launch_layernorm's);
// row r starts at x + r * ld_in elements.
hipError_t launch_row_stats(const void* x, int64_t ld_in, float* stats, int64_t rows, int64_t D,
                            float eps, int dtype, hipStream_t stream);

// sums[r] = sum_c src[r * cols + c] in fp32, in a fixed order (the same
// result on every call); up to two jobs in one launch.
struct RowSumJob {
  const void* src;
  int64_t rows, cols;
  float* sums;
};
hipError_t launch_row_sums(const RowSumJob* jobs, int njobs, int dtype, hipStream_t stream);

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

// sums[c] = sum_r src[r * cols + c] in fp32, in a fixed order: the column sums
// of an (in, out) weight.
struct ColSumJob {
  const void* src;
  int64_t rows, cols;
  float* sums;
};
// Row statistics to compute alongside (launch_row_stats's job).
struct StatsJob {
  const void* x;
  int64_t ld, rows, D;
  float* stats;
  float eps;
};
// One launch for the work at the start of a block call: up to 6 transposes,
// up to 4 column sums and optionally one set of row statistics (null: none),
// all bf16.  Returns hipErrorNotSupported, having launched nothing, when a job
// does not meet the fused kernel's layout (then launch them one by one).
hipError_t launch_prologue(const PackJob* jobs, int njobs, const ColSumJob* cs, int ncs,
                           const StatsJob* stats, int dtype, hipStream_t stream);

// The affine LayerNorm's fold into the product after it (bf16): for the
// out-major weight w_t [N, K], w_scaled[n, k] = bf16(gamma_k w_t[n, k]),
// col_sums[n] = sum_k w_scaled[n, k] (fp32, fixed order) and bias_out[n] =
// bf16(b_n + sum_k beta_k w_t[n, k]), b in segments of bias_seg columns (each
// null: zeros).  gamma, beta null: ones, zeros.  K a multiple of 8, w_t,
// w_scaled, gamma and beta 16-byte aligned.
struct AffineFoldJob {
  const void* w_t;
  const void* gamma;
  const void* beta;
  const void* bias[3];
  int64_t bias_seg;
  int64_t N, K;
  void* w_scaled;
  float* col_sums;
  void* bias_out;
};
// Row statistics computed in the same launch (the product's other operand):
// stats[2r], stats[2r + 1] = mean and rstd of row r, from the bf16 rows x
// (row stride ld; launch_row_stats's job) or, with partials non-null, from
// nstrips = D / kStatsStrip row partials (launch_row_stats_from_partials's).
struct FoldSide {
  const void* x;
  int64_t ld;
  const float2* partials;
  int64_t nstrips;
  float* stats;
  int64_t rows, D;
  float eps;
};
// side may be null.  hipErrorNotSupported, with nothing launched: the side
// job does not meet the kernel's layout (launch it on its own instead).
hipError_t launch_affine_fold(const AffineFoldJob& job, const FoldSide* side, hipStream_t stream);

// O[n*T + t, h*dh + c] = sum_j softmax_j(Q_h K_h^T / sqrt(dh))[t, j] V[n*T + j, h*dh + c]
// with Q, K, V row strides ld (elements) and O row stride ldo.
hipError_t launch_attention(const void* q, const void* k, const void* v, int64_t ld,
                            void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                            int64_t dh, int dtype, hipStream_t stream);
// The same for at least the first 32 queries of each sequence (every key): O
// rows n*T + t for t < min(T, 32) are written, others may not be.  For a
// readout that needs only the class token (query 0).
hipError_t launch_attention_first_queries(const void* q, const void* k, const void* v,
                                          int64_t ld, void* o, int64_t ldo, int64_t N, int64_t T,
                                          int64_t H, int64_t dh, int dtype, hipStream_t stream);

// fp32 on the matrix cores (attention_f32.hip) for head widths 32, 64, 80, 96,
// 128 and 16-byte-aligned rows; hipErrorNotSupported (nothing launched)
// otherwise.
hipError_t launch_attention_f32_mfma(const void* q, const void* k, const void* v, int64_t ld,
                                     void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                     int64_t dh, hipStream_t stream);

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
// fp32 on the matrix cores (gemm_f32.hip); hipErrorNotSupported (nothing
// launched) for shapes, alignments or epilogues it does not take.
hipError_t launch_gemm_f32_mfma(const GemmProblem& p, hipStream_t stream);
hipError_t launch_row_stats_generic(const void* x, int64_t ld_in, float* stats, int64_t rows,
                                    int64_t D, float eps, int dtype, hipStream_t stream);
hipError_t launch_attention_generic(const void* q, const void* k, const void* v, int64_t ld,
                                    void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                    int64_t dh, int dtype, hipStream_t stream);

// ------------------------------------------------------------------ backward

// Weight gradient: C[i, j] = sum_m A[m, i] * B[m, j] over the M token rows.
// A [M, I] (row stride lda), B [M, J] (row stride ldb); output column j goes
// to C[j / seg] at column j % seg (row stride ldc), so the fused Q|K|V
// gradient lands in three separate [D, D] outputs.  The token rows are split
// into `split` ranges, each reduced into partial[s] ([I, J] fp32), and a
// second kernel sums the partials in order and rounds to the dtype.
struct WgradProblem {
  int64_t M, I, J;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* C[3];
  int64_t ldc, seg;
  int dtype;
};

hipError_t launch_wgrad(const WgradProblem& p, float* partial, int split, hipStream_t stream);

// The matrix-core weight gradient over the first wgrad_mfma_rows() token rows
// (0: the problem does not qualify), in at most `split` ranges; *used gets
// the number of partials written.  hipErrorNotSupported: nothing launched.
int64_t wgrad_mfma_rows(const WgradProblem& p, int split);
hipError_t launch_wgrad_mfma(const WgradProblem& p, float* partial, int split, int* used,
                             hipStream_t stream);

// dx[r, :] = res[r, :] + J^T g[r, :] for the Jacobian J of LN (no gain or
// shift) at x[r, :]; res may be null.  All [rows, D].
hipError_t launch_layernorm_backward(const void* x, const void* g, const void* res, void* dx,
                                     int64_t rows, int64_t D, float eps, int dtype,
                                     hipStream_t stream);

// Any-D version (one workgroup per row); the fast kernel falls back to it.
hipError_t launch_layernorm_backward_generic(const void* x, const void* g, const void* res,
                                             void* dx, int64_t rows, int64_t D, float eps,
                                             int dtype, hipStream_t stream);

// Attention backward: dQ, dK, dV (row stride ldd) from Q, K, V (row stride
// ld) and dO (row stride ldo).  stats: 3 * N * H * T floats of workspace
// (each query's score maximum, exponential sum and rowsum(P * dP)).
// Matrix-core attention backward (bf16, the head resident in LDS);
// hipErrorNotSupported when the shape does not qualify (nothing launched).
hipError_t launch_attention_backward_mfma(const void* q, const void* k, const void* v,
                                          int64_t ld, const void* d_o, int64_t ldo, void* dq,
                                          void* dk, void* dv, int64_t ldd, int64_t N, int64_t T,
                                          int64_t H, int64_t dh, float* stats,
                                          hipStream_t stream);

hipError_t launch_attention_backward(const void* q, const void* k, const void* v, int64_t ld,
                                     const void* d_o, int64_t ldo, void* dq, void* dk, void* dv,
                                     int64_t ldd, int64_t N, int64_t T, int64_t H, int64_t dh,
                                     int dtype, float* stats, hipStream_t stream);

}  // namespace vitblk
