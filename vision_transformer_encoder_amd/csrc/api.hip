// C ABI of vitblk: argument checks (validate.cpp), workspace carving and the
// launch sequence of one pre-LN encoder block forward.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"
#include "plan.h"
#include "vitblk.h"

using namespace vitblk;

namespace {

// Launch-failure check after each kernel; the first failure ends the call.
#define VITBLK_LAUNCH(expr)                          \
  do {                                               \
    if ((expr) != hipSuccess) return VITBLK_ERR_HIP; \
  } while (0)

GemmProblem linear_problem(const void* a, const void* w_t, void* c, const void* r, int64_t M,
                           int64_t K, int64_t N, int epi, int dtype, const void* b0 = nullptr,
                           const void* b1 = nullptr, const void* b2 = nullptr,
                           int64_t bias_seg = 0) {
  GemmProblem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.A = a;
  p.lda = K;
  p.B = w_t;
  p.ldb = K;
  p.C = c;
  p.ldc = N;
  p.R = r;
  p.ldr = N;
  p.epi = epi;
  p.dtype = dtype;
  p.bias[0] = b0;
  p.bias[1] = b1;
  p.bias[2] = b2;
  p.bias_seg = bias_seg > 0 ? bias_seg : N;
  return p;
}

// The packed weights and, with stats non-null, a set of row statistics
// (launch_row_stats's job) in the same launch when the layouts allow.
int pack_weights(const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                 const void* w_mlp1, const void* w_mlp2, void* packed, int64_t D, int64_t F,
                 int dtype, const PackedPlan& pl, hipStream_t s,
                 const StatsJob* stats = nullptr) {
  char* base = static_cast<char*>(packed);
  const size_t es = elem_size(dtype);
  char* qkv = base + pl.off_qkv;
  const PackJob jobs[6] = {
      {w_q, D, D, qkv, D},
      {w_k, D, D, qkv + static_cast<size_t>(D) * D * es, D},
      {w_v, D, D, qkv + 2 * static_cast<size_t>(D) * D * es, D},
      {w_o, D, D, base + pl.off_o, D},
      {w_mlp1, D, F, base + pl.off_1, D},
      {w_mlp2, F, D, base + pl.off_2, F},
  };
  // Column sums of [w_q | w_k | w_v] and of w_mlp1 for the products that
  // fold in the LayerNorm: from the source weights in the fused launch, else
  // as the row sums of the packed copies.
  float* cs_qkv = reinterpret_cast<float*>(base + pl.off_cs_qkv);
  const ColSumJob cols[4] = {
      {w_q, D, D, cs_qkv},
      {w_k, D, D, cs_qkv + D},
      {w_v, D, D, cs_qkv + 2 * D},
      {w_mlp1, D, F, reinterpret_cast<float*>(base + pl.off_cs_1)},
  };
  const hipError_t fused = launch_prologue(jobs, 6, cols, 4, stats, dtype, s);
  if (fused != hipErrorNotSupported) {
    VITBLK_LAUNCH(fused);
    return VITBLK_OK;
  }
  VITBLK_LAUNCH(launch_pack(jobs, 6, dtype, s));
  const RowSumJob sums[2] = {
      {qkv, 3 * D, D, reinterpret_cast<float*>(base + pl.off_cs_qkv)},
      {base + pl.off_1, F, D, reinterpret_cast<float*>(base + pl.off_cs_1)},
  };
  VITBLK_LAUNCH(launch_row_sums(sums, 2, dtype, s));
  if (stats != nullptr)
    VITBLK_LAUNCH(launch_row_stats(stats->x, stats->ld, stats->stats, stats->rows, stats->D,
                                   stats->eps, dtype, s));
  return VITBLK_OK;
}

// Where an affine LayerNorm (gain and/or shift) folds into the product after
// it (bf16): the gain-scaled weight copy, its column sums and the folded bias
// (launch_affine_fold) go to a region that is dead while that product runs,
// at these offsets from the region's start: LN1's into region y (written only
// by the output projection, after the fused Q|K|V product), LN2's into region
// act after the row statistics (its concatenated heads are dead once the
// output projection has run).  The block writes such a LayerNorm out where
// the copy does not fit (M < 3D or about M < F) or an operand is misaligned.
struct FoldCopy {
  size_t w, cs, b, end;
};

FoldCopy fold_copy(size_t start, int64_t nout, int64_t K) {
  const auto up = [](size_t v) { return (v + kRegionAlign - 1) / kRegionAlign * kRegionAlign; };
  FoldCopy f;
  f.w = up(start);
  f.cs = up(f.w + static_cast<size_t>(nout) * static_cast<size_t>(K) * 2);
  f.b = up(f.cs + static_cast<size_t>(nout) * 4);
  f.end = f.b + static_cast<size_t>(nout) * 2;
  return f;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Which LayerNorms the block folds.  fold: the product applies the row
// statistics; affine: with the gain/shift fold's copy (region offsets f).
struct FoldPlan {
  bool fold1, affine1, fold2, affine2;
  FoldCopy f1, f2;
};

FoldPlan plan_folds(const vitblk_affine_params& q, const char* pk, const char* act,
                    const WorkspacePlan& pl, int64_t Mo, int64_t D, int64_t F, int dtype) {
  FoldPlan fp{};
  if (dtype != VITBLK_BF16) return fp;
  const bool has1 = q.ln1_gamma != nullptr || q.ln1_beta != nullptr;
  const bool has2 = q.ln2_gamma != nullptr || q.ln2_beta != nullptr;
  const char* a = act + pl.off_act;
  const char* y = act + pl.off_y;
  fp.f1 = fold_copy(0, 3 * D, D);
  fp.f2 = fold_copy(static_cast<size_t>(Mo) * 8, F, D);  // after Mo rows' (mean, rstd)
  const bool ok = D % 8 == 0 && aligned16(a) && aligned16(y);
  fp.affine1 = has1 && ok && aligned16(pk + pl.packed.off_qkv) &&
               fp.f1.end <= pl.act_total - pl.off_y;
  fp.affine2 = has2 && ok && aligned16(pk + pl.packed.off_1) &&
               fp.f2.end <= pl.off_y - pl.off_act;
  fp.fold1 = !has1 || fp.affine1;
  fp.fold2 = !has2 || fp.affine2;
  return fp;
}

// The seven steps of the block on packed (out-major) weights.  prm: the
// affine variant's optional gains, shifts and biases (null: none).
// stats1_ready: the first LayerNorm's row statistics are already in place
// (written with the packed weights; only where the block folds that
// LayerNorm).  cls_only: only each sequence's first token (the class token)
// leaves the block; out is then [N, D].  Every token's K and V still enter
// attention, but only the first query tile is computed, and the output
// projection, LN2 and the MLP run on the N class-token rows (row stride T*D
// into the attention output and x).
int run_block(const void* x, const void* packed, const vitblk_affine_params* prm, void* out,
              int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, double eps, int dtype,
              char* act, const WorkspacePlan& pl, hipStream_t s, bool stats1_ready = false,
              bool cls_only = false) {
  const vitblk_affine_params none{};
  const vitblk_affine_params& q = prm != nullptr ? *prm : none;
  const int64_t M = N * T;
  const size_t es = elem_size(dtype);
  const char* pk = static_cast<const char*>(packed);
  char* big = act + pl.off_big;  // qkv [M, 3D], later hidden [M, F]
  char* a = act + pl.off_act;    // xn, then att, then yn: [M, D]
  char* y = act + pl.off_y;      // [M, D]
  const float feps = static_cast<float>(eps);

  // A LayerNorm folds into the product that follows it (bf16): LN(x) @ W =
  // rstd (x @ W - mean 1^T W), so only the rows' statistics are computed
  // (into region act) and the product applies them with W's column sums from
  // the packed weights.  With a gain and shift the product takes the
  // launch_affine_fold copy instead (diag(gamma) W, its column sums, the bias
  // plus beta @ W).  fp32, and an affine LayerNorm whose copy has no room,
  // are written out.
  float* stats = reinterpret_cast<float*>(a);
  const int64_t Mo = cls_only ? N : M;  // rows after attention
  const FoldPlan fp = plan_folds(q, pk, act, pl, Mo, D, F, dtype);

  // LN1: xn = gamma_1 LN(x) + beta_1, then Q | K | V = xn @ [w_q | w_k | w_v] + [b_q | b_k | b_v]
  GemmProblem pq = linear_problem(a, pk + pl.packed.off_qkv, big, nullptr, M, D, 3 * D,
                                  VITBLK_EPI_NONE, dtype, q.b_q, q.b_k, q.b_v, D);
  if (fp.fold1) {
    bool stats_done = stats1_ready;
    pq.A = x;
    pq.row_stats = stats;
    pq.col_sums = reinterpret_cast<const float*>(pk + pl.packed.off_cs_qkv);
    if (fp.affine1) {
      const AffineFoldJob j{pk + pl.packed.off_qkv, q.ln1_gamma, q.ln1_beta,
                            {q.b_q, q.b_k, q.b_v}, D, 3 * D, D, y + fp.f1.w,
                            reinterpret_cast<float*>(y + fp.f1.cs), y + fp.f1.b};
      const FoldSide side{x, D, nullptr, 0, stats, M, D, feps};
      const hipError_t e = launch_affine_fold(j, stats_done ? nullptr : &side, s);
      if (e != hipErrorNotSupported) {
        VITBLK_LAUNCH(e);
        stats_done = true;
      } else {
        VITBLK_LAUNCH(launch_affine_fold(j, nullptr, s));
      }
      pq.B = y + fp.f1.w;
      pq.col_sums = reinterpret_cast<const float*>(y + fp.f1.cs);
      pq.bias[0] = y + fp.f1.b;
      pq.bias[1] = pq.bias[2] = nullptr;
      pq.bias_seg = 3 * D;
    }
    if (!stats_done) VITBLK_LAUNCH(launch_row_stats(x, D, stats, M, D, feps, dtype, s));
  } else {
    VITBLK_LAUNCH(launch_layernorm(x, D, q.ln1_gamma, q.ln1_beta, a, M, D, feps, dtype, s));
  }
  VITBLK_LAUNCH(launch_gemm(pq, s));
  // att = concat_h softmax(Q_h K_h^T / sqrt(dh)) V_h   (overwrites xn)
  if (cls_only)
    VITBLK_LAUNCH(launch_attention_first_queries(big, big + D * es, big + 2 * D * es, 3 * D, a,
                                                 D, N, T, H, D / H, dtype, s));
  else
    VITBLK_LAUNCH(launch_attention(big, big + D * es, big + 2 * D * es, 3 * D, a, D, N, T, H,
                                   D / H, dtype, s));
  // y = x + att @ w_o + b_o   (qkv's region is free again: split-K scratch)
  GemmProblem po = linear_problem(a, pk + pl.packed.off_o, y, x, Mo, D, D, VITBLK_EPI_RESIDUAL,
                                  dtype, q.b_o);
  if (cls_only) po.lda = po.ldr = T * D;  // the class-token rows of att and x
  po.scratch = reinterpret_cast<float*>(big);
  po.scratch_floats = static_cast<int64_t>(pl.off_act - pl.off_big) / 4;
  // With LN2 folded, the product's epilogue also writes each row's partial
  // statistics over every 64 columns of y (into qkv's region, dead now) and
  // a small kernel combines them: y is not read again for its statistics.
  if (fp.fold2) {
    po.row_partials = reinterpret_cast<float2*>(big);
    if (gemm_row_partials_ok(po)) {
      po.epi = kEpiResidualStats;
      po.scratch = nullptr;
    } else {
      po.row_partials = nullptr;
    }
  }
  VITBLK_LAUNCH(launch_gemm(po, s));
  // LN2: yn = gamma_2 LN(y) + beta_2 (overwrites att), then
  // hidden = GELU(yn @ w_mlp1 + b_mlp1)   (overwrites qkv)
  GemmProblem p1 = linear_problem(a, pk + pl.packed.off_1, big, nullptr, Mo, D, F,
                                  VITBLK_EPI_GELU, dtype, q.b_mlp1);
  if (fp.fold2) {
    // The statistics from the row partials ride in the fold's launch.
    bool stats_done = false;
    p1.A = y;
    p1.row_stats = stats;
    p1.col_sums = reinterpret_cast<const float*>(pk + pl.packed.off_cs_1);
    if (fp.affine2) {
      const AffineFoldJob j{pk + pl.packed.off_1, q.ln2_gamma, q.ln2_beta,
                            {q.b_mlp1, nullptr, nullptr}, F, F, D, a + fp.f2.w,
                            reinterpret_cast<float*>(a + fp.f2.cs), a + fp.f2.b};
      const FoldSide side{nullptr, 0, po.row_partials, D / kStatsStrip, stats, Mo, D, feps};
      const hipError_t e =
          launch_affine_fold(j, po.row_partials != nullptr ? &side : nullptr, s);
      if (e != hipErrorNotSupported) {
        VITBLK_LAUNCH(e);
        stats_done = po.row_partials != nullptr;
      } else {
        VITBLK_LAUNCH(launch_affine_fold(j, nullptr, s));
      }
      p1.B = a + fp.f2.w;
      p1.col_sums = reinterpret_cast<const float*>(a + fp.f2.cs);
      p1.bias[0] = a + fp.f2.b;
      p1.bias_seg = F;
    }
    if (!stats_done) {
      if (po.row_partials != nullptr)
        VITBLK_LAUNCH(launch_row_stats_from_partials(po.row_partials, D / kStatsStrip, stats, Mo,
                                                     D, feps, s));
      else
        VITBLK_LAUNCH(launch_row_stats(y, D, stats, Mo, D, feps, dtype, s));
    }
  } else {
    VITBLK_LAUNCH(launch_layernorm(y, D, q.ln2_gamma, q.ln2_beta, a, Mo, D, feps, dtype, s));
  }
  VITBLK_LAUNCH(launch_gemm(p1, s));
  // out = y + hidden @ w_mlp2 + b_mlp2   (yn's region is free again: split-K scratch)
  GemmProblem p2 = linear_problem(big, pk + pl.packed.off_2, out, y, Mo, F, D,
                                  VITBLK_EPI_RESIDUAL, dtype, q.b_mlp2);
  p2.scratch = reinterpret_cast<float*>(a);
  p2.scratch_floats = static_cast<int64_t>(pl.off_y - pl.off_act) / 4;
  VITBLK_LAUNCH(launch_gemm(p2, s));
  return VITBLK_OK;
}

// L blocks in sequence through two token buffers, then the final LayerNorm
// of every token (out) and/or of each sequence's first token (cls).
int run_encoder(const void* x, const void* const* packed, const vitblk_affine_params* params,
                int64_t L, const void* fg, const void* fb, void* out, void* cls, int64_t N,
                int64_t T, int64_t D, int64_t F, int64_t H, double eps, int dtype, char* ws,
                const EncoderPlan& pl, hipStream_t s) {
  char* tok[2] = {ws + pl.off_tok0, ws + pl.off_tok1};
  const void* cur = x;
  // Only the class tokens leave the stack: the last block computes just their
  // rows (every token's K and V still enter its attention) and writes [N, D].
  const bool cls_last = out == nullptr && cls != nullptr && L > 0;
  for (int64_t l = 0; l < L; ++l) {
    char* dst = tok[l & 1];
    const int st = run_block(cur, packed[l], params != nullptr ? &params[l] : nullptr, dst, N, T,
                             D, F, H, eps, dtype, ws + pl.block.act_base, pl.block, s, false,
                             cls_last && l == L - 1);
    if (st != VITBLK_OK) return st;
    cur = dst;
  }
  const float feps = static_cast<float>(eps);
  if (out != nullptr)
    VITBLK_LAUNCH(launch_layernorm(cur, D, fg, fb, out, N * T, D, feps, dtype, s));
  if (cls != nullptr)  // rows n*T (stride T*D), or the last block's [N, D]
    VITBLK_LAUNCH(launch_layernorm(cur, cls_last ? D : T * D, fg, fb, cls, N, D, feps, dtype, s));
  return VITBLK_OK;
}

WgradProblem wgrad_problem(const void* a, int64_t lda, const void* b, int64_t ldb, void* c,
                           int64_t M, int64_t I, int64_t J, int dtype) {
  WgradProblem p{};
  p.M = M;
  p.I = I;
  p.J = J;
  p.A = a;
  p.lda = lda;
  p.B = b;
  p.ldb = ldb;
  p.C[0] = c;
  p.ldc = J;
  p.seg = J;
  p.dtype = dtype;
  return p;
}

// The backward of the plain block: recompute the forward's activations, then
// walk its steps in reverse (each gradient step names the forward step it
// differentiates).  w: w_q, w_k, w_v, w_o, w_mlp1, w_mlp2; g: dx, dw_q, dw_k,
// dw_v, dw_o, dw_mlp1, dw_mlp2.
int run_backward(const void* x, const void* const* w, const void* dout, void* const* g,
                 int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, double eps, int dtype,
                 char* ws, const BackwardPlan& pl, hipStream_t s) {
  const int64_t M = N * T;
  const size_t es = elem_size(dtype);
  const float feps = static_cast<float>(eps);
  char* pk = ws;  // forward packed weights at offset 0
  char* wcat = ws + pl.off_wcat;
  char* xn = ws + pl.off_xn;
  char* qkv = ws + pl.off_qkv;
  char* att = ws + pl.off_att;
  char* y = ws + pl.off_y;
  char* yn = ws + pl.off_yn;
  char* z = ws + pl.off_z;
  char* h = ws + pl.off_h;
  char* dy = ws + pl.off_dy;
  float* stats = reinterpret_cast<float*>(ws + pl.off_stats);
  float* partial = reinterpret_cast<float*>(ws + pl.off_partial);

  // Weights: the forward's out-major copies, and [w_q | w_k | w_v] row by row.
  int st = pack_weights(w[0], w[1], w[2], w[3], w[4], w[5], pk, D, F, dtype, pl.packed, s);
  if (st != VITBLK_OK) return st;
  for (int i = 0; i < 3; ++i)
    VITBLK_LAUNCH(hipMemcpy2DAsync(wcat + i * D * es, 3 * D * es, w[i], D * es, D * es, D,
                                   hipMemcpyDeviceToDevice, s));

  // ---- forward, keeping every activation the gradients need
  VITBLK_LAUNCH(launch_layernorm(x, D, nullptr, nullptr, xn, M, D, feps, dtype, s));
  VITBLK_LAUNCH(launch_gemm(linear_problem(xn, pk + pl.packed.off_qkv, qkv, nullptr, M, D, 3 * D,
                                           VITBLK_EPI_NONE, dtype),
                            s));
  VITBLK_LAUNCH(launch_attention(qkv, qkv + D * es, qkv + 2 * D * es, 3 * D, att, D, N, T, H,
                                 D / H, dtype, s));
  VITBLK_LAUNCH(launch_gemm(
      linear_problem(att, pk + pl.packed.off_o, y, x, M, D, D, VITBLK_EPI_RESIDUAL, dtype), s));
  VITBLK_LAUNCH(launch_layernorm(y, D, nullptr, nullptr, yn, M, D, feps, dtype, s));
  // h = GELU(yn @ w_mlp1) and, from the same product, GELU'(yn @ w_mlp1) (into z's region)
  GemmProblem p1 = linear_problem(yn, pk + pl.packed.off_1, h, nullptr, M, D, F, kEpiGeluDual,
                                  dtype);
  p1.C2 = z;
  VITBLK_LAUNCH(launch_gemm(p1, s));

  // ---- out = y + h @ w_mlp2
  VITBLK_LAUNCH(launch_wgrad(wgrad_problem(h, F, dout, D, g[6], M, F, D, dtype), partial,
                             wgrad_split(M, F, D), s));
  // h = GELU(z):  dz = (dout @ w_mlp2^T) * GELU'(z)   (into h's region)
  VITBLK_LAUNCH(launch_gemm(linear_problem(dout, w[5], h, z, M, D, F, kEpiMul, dtype), s));
  // z = yn @ w_mlp1
  VITBLK_LAUNCH(launch_wgrad(wgrad_problem(yn, D, h, F, g[5], M, D, F, dtype), partial,
                             wgrad_split(M, D, F), s));
  VITBLK_LAUNCH(launch_gemm(
      linear_problem(h, w[4], yn, nullptr, M, F, D, VITBLK_EPI_NONE, dtype), s));  // dyn
  // yn = LN(y); y also feeds out directly:  dy = dout + LN'(y)^T dyn
  VITBLK_LAUNCH(launch_layernorm_backward(y, yn, dout, dy, M, D, feps, dtype, s));
  // y = x + att @ w_o
  VITBLK_LAUNCH(launch_wgrad(wgrad_problem(att, D, dy, D, g[4], M, D, D, dtype), partial,
                             wgrad_split(M, D, D), s));
  VITBLK_LAUNCH(launch_gemm(
      linear_problem(dy, w[3], y, nullptr, M, D, D, VITBLK_EPI_NONE, dtype), s));  // datt
  // att = heads of softmax(q k^T / sqrt(dh)) v:  dqkv into z's region
  VITBLK_LAUNCH(launch_attention_backward(qkv, qkv + D * es, qkv + 2 * D * es, 3 * D, y, D, z,
                                          z + D * es, z + 2 * D * es, 3 * D, N, T, H, D / H,
                                          dtype, stats, s));
  // q | k | v = xn @ [w_q | w_k | w_v]
  WgradProblem pq = wgrad_problem(xn, D, z, 3 * D, g[1], M, D, 3 * D, dtype);
  pq.C[1] = g[2];
  pq.C[2] = g[3];
  pq.ldc = D;
  pq.seg = D;
  VITBLK_LAUNCH(launch_wgrad(pq, partial, wgrad_split(M, D, 3 * D), s));
  // dxn = dqkv @ [w_q | w_k | w_v]^T   (into att's region)
  GemmProblem px = linear_problem(z, wcat, att, nullptr, M, 3 * D, D, VITBLK_EPI_NONE, dtype);
  VITBLK_LAUNCH(launch_gemm(px, s));
  // xn = LN(x); x also feeds y directly:  dx = dy + LN'(x)^T dxn
  VITBLK_LAUNCH(launch_layernorm_backward(x, att, dy, g[0], M, D, feps, dtype, s));
  return VITBLK_OK;
}

}  // namespace

extern "C" {

size_t vitblk_backward_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                                       int dtype) {
  BackwardPlan p;
  if (plan_backward(N, T, D, F, H, dtype, &p) != VITBLK_OK) return 0;
  return p.total;
}

int vitblk_backward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                    const void* w_o, const void* w_mlp1, const void* w_mlp2, const void* dout,
                    void* dx, void* dw_q, void* dw_k, void* dw_v, void* dw_o, void* dw_mlp1,
                    void* dw_mlp2, int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                    double eps, int dtype, void* workspace, size_t workspace_bytes,
                    vitblk_stream_t stream) {
  const void* w[6] = {w_q, w_k, w_v, w_o, w_mlp1, w_mlp2};
  void* g[7] = {dx, dw_q, dw_k, dw_v, dw_o, dw_mlp1, dw_mlp2};
  BackwardPlan pl;
  const int st = validate_backward(x, w, dout, g, N, T, D, F, H, eps, dtype, workspace,
                                   workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  return run_backward(x, w, dout, g, N, T, D, F, H, eps, dtype, static_cast<char*>(workspace),
                      pl, reinterpret_cast<hipStream_t>(stream));
}

size_t vitblk_weight_grad_workspace_bytes(int64_t M, int64_t I, int64_t J) {
  return wgrad_partial_bytes(M, I, J);
}

int vitblk_weight_grad(const void* a, const void* b, void* out, int64_t M, int64_t I, int64_t J,
                       int dtype, void* workspace, size_t workspace_bytes,
                       vitblk_stream_t stream) {
  const int st = validate_weight_grad(a, b, out, M, I, J, dtype, workspace, workspace_bytes);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_wgrad(wgrad_problem(a, I, b, J, out, M, I, J, dtype),
                             static_cast<float*>(workspace), wgrad_split(M, I, J),
                             reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_layernorm_backward(const void* x, const void* g, const void* residual, void* dx,
                              int64_t rows, int64_t D, double eps, int dtype,
                              vitblk_stream_t stream) {
  const int st = validate_layernorm_backward(x, g, residual, dx, rows, D, eps, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_layernorm_backward(x, g, residual, dx, rows, D, static_cast<float>(eps),
                                          dtype, reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

size_t vitblk_attention_backward_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t H) {
  if (D <= 0 || H <= 0 || D % H != 0) return 0;
  return attention_stats_bytes(N, T, H);
}

int vitblk_attention_backward(const void* qkv, const void* datt, void* dqkv, int64_t N, int64_t T,
                              int64_t D, int64_t H, int dtype, void* workspace,
                              size_t workspace_bytes, vitblk_stream_t stream) {
  const int st = validate_attention_backward(qkv, datt, dqkv, N, T, D, H, dtype, workspace,
                                             workspace_bytes);
  if (st != VITBLK_OK) return st;
  const size_t es = elem_size(dtype);
  const char* q = static_cast<const char*>(qkv);
  char* d = static_cast<char*>(dqkv);
  VITBLK_LAUNCH(launch_attention_backward(q, q + D * es, q + 2 * D * es, 3 * D, datt, D, d,
                                          d + D * es, d + 2 * D * es, 3 * D, N, T, H, D / H,
                                          dtype, static_cast<float*>(workspace),
                                          reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

size_t vitblk_patch_embed_workspace_bytes(int64_t B, int64_t C, int64_t H, int64_t W,
                                          int64_t P, int64_t D, int dtype) {
  EmbedPlan p;
  if (plan_embed(B, C, H, W, P, D, dtype, &p) != VITBLK_OK) return 0;
  return p.total;
}

int vitblk_patch_embed(const void* images, const void* w_patch, const void* b_patch,
                       const void* cls_token, const void* pos_emb, void* tokens, int64_t B,
                       int64_t C, int64_t H, int64_t W, int64_t P, int64_t D, int dtype,
                       void* workspace, size_t workspace_bytes, vitblk_stream_t stream) {
  EmbedPlan pl;
  const int st = validate_patch_embed(images, w_patch, b_patch, cls_token, pos_emb, tokens, B, C,
                                      H, W, P, D, dtype, workspace, workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  char* ws = static_cast<char*>(workspace);
  PatchEmbedArgs a{};
  a.images = images;
  a.w_patch = w_patch;
  a.b_patch = b_patch;
  a.cls = cls_token;
  a.pos = pos_emb;
  a.tokens = tokens;
  a.w_t = ws + pl.off_wt;
  a.patches = ws + pl.off_patches;
  a.embedded = ws + pl.off_embedded;
  a.B = B;
  a.C = C;
  a.H = H;
  a.W = W;
  a.P = P;
  a.D = D;
  a.Kp = pl.Kp;
  a.dtype = dtype;
  VITBLK_LAUNCH(launch_patch_embed(a, reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

size_t vitblk_encoder_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                                      int dtype) {
  EncoderPlan p;
  if (plan_encoder(N, T, D, F, H, dtype, &p) != VITBLK_OK) return 0;
  return p.total;
}

int vitblk_encoder_forward(const void* x, const void* const* packed,
                           const vitblk_affine_params* params, int64_t L,
                           const void* final_gamma, const void* final_beta, void* out,
                           void* cls_out, int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                           double eps, int dtype, void* workspace, size_t workspace_bytes,
                           vitblk_stream_t stream) {
  EncoderPlan pl;
  const int st = validate_encoder(x, packed, params, L, final_gamma, final_beta, out, cls_out, N,
                                  T, D, F, H, eps, dtype, workspace, workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  return run_encoder(x, packed, params, L, final_gamma, final_beta, out, cls_out, N, T, D, F, H,
                     eps, dtype, static_cast<char*>(workspace), pl,
                     reinterpret_cast<hipStream_t>(stream));
}

const char* vitblk_status_string(int status) {
  switch (status) {
    case VITBLK_OK: return "VITBLK_OK";
    case VITBLK_ERR_INVALID_ARG: return "VITBLK_ERR_INVALID_ARG: invalid argument";
    case VITBLK_ERR_UNSUPPORTED: return "VITBLK_ERR_UNSUPPORTED: sizes beyond the kernels' limits";
    case VITBLK_ERR_WORKSPACE: return "VITBLK_ERR_WORKSPACE: workspace missing or too small";
    case VITBLK_ERR_ALIAS: return "VITBLK_ERR_ALIAS: an output overlaps an input or the workspace";
    case VITBLK_ERR_HIP: return "VITBLK_ERR_HIP: a kernel launch failed";
    default: return "unknown vitblk status";
  }
}

size_t vitblk_workspace_bytes(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H,
                              int dtype) {
  WorkspacePlan p;
  if (plan_workspace(N, T, D, F, H, dtype, &p) != VITBLK_OK) return 0;
  return p.total;
}

size_t vitblk_packed_weights_bytes(int64_t D, int64_t F, int dtype) {
  PackedPlan p;
  if (plan_packed(D, F, dtype, &p) != VITBLK_OK) return 0;
  return p.total;
}

int vitblk_pack_weights(const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                        const void* w_mlp1, const void* w_mlp2, void* packed, int64_t D,
                        int64_t F, int dtype, vitblk_stream_t stream) {
  PackedPlan pl;
  const int st = validate_pack(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, packed, D, F, dtype, &pl);
  if (st != VITBLK_OK) return st;
  return pack_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, packed, D, F, dtype, pl,
                      reinterpret_cast<hipStream_t>(stream));
}

int vitblk_forward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                   const void* w_o, const void* w_mlp1, const void* w_mlp2, void* out,
                   int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                   int dtype, void* workspace, size_t workspace_bytes, vitblk_stream_t stream) {
  WorkspacePlan pl;
  int st = validate_forward(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, out, N, T, D, F, H, eps,
                            dtype, workspace, workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  // The block folds its first LayerNorm (bf16): its statistics are computed
  // in the weights' launch, where run_block reads them (region act).
  const bool fold1 = dtype == VITBLK_BF16;
  const StatsJob stats1{x, D, N * T, D,
                        reinterpret_cast<float*>(ws + pl.act_base + pl.off_act),
                        static_cast<float>(eps)};
  st = pack_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, ws, D, F, dtype, pl.packed, s,
                    fold1 ? &stats1 : nullptr);
  if (st != VITBLK_OK) return st;
  return run_block(x, ws, nullptr, out, N, T, D, F, H, eps, dtype, ws + pl.act_base, pl, s,
                   fold1);
}

int vitblk_forward_affine(const void* x, const void* w_q, const void* w_k, const void* w_v,
                          const void* w_o, const void* w_mlp1, const void* w_mlp2,
                          const vitblk_affine_params* params, void* out, int64_t N, int64_t T,
                          int64_t D, int64_t F, int64_t H, double eps, int dtype,
                          void* workspace, size_t workspace_bytes, vitblk_stream_t stream) {
  WorkspacePlan pl;
  int st = validate_forward(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, out, N, T, D, F, H, eps,
                            dtype, workspace, workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  st = validate_affine_params(params, out, N * T, D, F, dtype, workspace, pl.total);
  if (st != VITBLK_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const vitblk_affine_params none{};
  const bool fold1 = plan_folds(params != nullptr ? *params : none, ws, ws + pl.act_base, pl,
                                N * T, D, F, dtype)
                         .fold1;
  const StatsJob stats1{x, D, N * T, D,
                        reinterpret_cast<float*>(ws + pl.act_base + pl.off_act),
                        static_cast<float>(eps)};
  st = pack_weights(w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, ws, D, F, dtype, pl.packed, s,
                    fold1 ? &stats1 : nullptr);
  if (st != VITBLK_OK) return st;
  return run_block(x, ws, params, out, N, T, D, F, H, eps, dtype, ws + pl.act_base, pl, s,
                   fold1);
}

int vitblk_forward_packed(const void* x, const void* packed, void* out, int64_t N, int64_t T,
                          int64_t D, int64_t F, int64_t H, double eps, int dtype,
                          void* workspace, size_t workspace_bytes, vitblk_stream_t stream) {
  WorkspacePlan pl;
  const int st = validate_forward_packed(x, packed, out, N, T, D, F, H, eps, dtype, workspace,
                                         workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  return run_block(x, packed, nullptr, out, N, T, D, F, H, eps, dtype,
                   static_cast<char*>(workspace) + pl.act_base, pl,
                   reinterpret_cast<hipStream_t>(stream));
}

// ---------------------------------------------------------------- no-allocation entry

namespace {

// The activations of vitblk_forward_packed_noalloc: one array per GPU (the
// code object's global), never allocated or freed by the library.  In host
// code `scratch` names a host-side stand-in, not device memory; its device
// address on each GPU comes from hipGetSymbolAddress (scratch_ptr) and only
// that address is ever passed to kernels.
__device__ __align__(256) char scratch[VITBLK_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices] = {};

// scratch's address on the device `stream` runs on, resolved once per device
// with that device current (the caller's current device is restored).
int scratch_ptr(hipStream_t stream, void** out) {
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return VITBLK_ERR_HIP;
  int dev = cur;
  if (stream != nullptr && hipStreamGetDevice(stream, &dev) != hipSuccess) {
    (void)hipGetLastError();
    return VITBLK_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return VITBLK_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_addr[dev] == nullptr) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return VITBLK_ERR_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) (void)hipSetDevice(cur);
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return VITBLK_ERR_HIP;
    }
    scratch_addr[dev] = p;
  }
  *out = scratch_addr[dev];
  return VITBLK_OK;
}

}  // namespace

int vitblk_forward_packed_noalloc(const void* x, const void* packed, void* out, int64_t N,
                                  int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                                  int dtype, vitblk_stream_t stream) {
  // Sizes first (host only): a block whose activations exceed the scratch
  // array is rejected before any HIP call.
  WorkspacePlan pl;
  int st = plan_workspace(N, T, D, F, H, dtype, &pl);
  if (st != VITBLK_OK) return st;
  if (pl.act_total > VITBLK_NOALLOC_SCRATCH_BYTES) return VITBLK_ERR_WORKSPACE;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  st = scratch_ptr(s, &ws);
  if (st != VITBLK_OK) return st;
  st = validate_forward_packed(x, packed, out, N, T, D, F, H, eps, dtype, ws,
                               VITBLK_NOALLOC_SCRATCH_BYTES, &pl);
  if (st != VITBLK_OK) return st;
  return run_block(x, packed, nullptr, out, N, T, D, F, H, eps, dtype,
                   static_cast<char*>(ws) + pl.act_base, pl, s);
}

int vitblk_forward_packed_affine(const void* x, const void* packed,
                                 const vitblk_affine_params* params, void* out, int64_t N,
                                 int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                                 int dtype, void* workspace, size_t workspace_bytes,
                                 vitblk_stream_t stream) {
  WorkspacePlan pl;
  int st = validate_forward_packed(x, packed, out, N, T, D, F, H, eps, dtype, workspace,
                                   workspace_bytes, &pl);
  if (st != VITBLK_OK) return st;
  st = validate_affine_params(params, out, N * T, D, F, dtype, workspace, pl.act_total);
  if (st != VITBLK_OK) return st;
  return run_block(x, packed, params, out, N, T, D, F, H, eps, dtype,
                   static_cast<char*>(workspace) + pl.act_base, pl,
                   reinterpret_cast<hipStream_t>(stream));
}

int vitblk_layernorm(const void* x, void* out, int64_t rows, int64_t D, double eps, int dtype,
                     vitblk_stream_t stream) {
  return vitblk_layernorm_affine(x, nullptr, nullptr, out, rows, D, eps, dtype, stream);
}

int vitblk_layernorm_affine(const void* x, const void* gamma, const void* beta, void* out,
                            int64_t rows, int64_t D, double eps, int dtype,
                            vitblk_stream_t stream) {
  const int st = validate_layernorm(x, gamma, beta, out, rows, D, eps, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_layernorm(x, D, gamma, beta, out, rows, D, static_cast<float>(eps), dtype,
                                 reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_row_stats(const void* x, float* stats, int64_t rows, int64_t D, double eps,
                     int dtype, vitblk_stream_t stream) {
  const int st = validate_row_stats(x, stats, rows, D, eps, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_row_stats(x, D, stats, rows, D, static_cast<float>(eps), dtype,
                                 reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_linear_normed(const void* a, const void* w_t, const float* col_sums,
                         const float* row_stats, const void* bias, void* out, int64_t M,
                         int64_t K, int64_t Nout, int epilogue, int dtype,
                         vitblk_stream_t stream) {
  const int st = validate_linear_normed(a, w_t, col_sums, row_stats, bias, out, M, K, Nout,
                                        epilogue, dtype);
  if (st != VITBLK_OK) return st;
  GemmProblem p = linear_problem(a, w_t, out, nullptr, M, K, Nout, epilogue, dtype, bias);
  p.row_stats = row_stats;
  p.col_sums = col_sums;
  VITBLK_LAUNCH(launch_gemm(p, reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_affine_fold(const void* w_t, const void* gamma, const void* beta, const void* bias,
                       void* w_scaled, float* col_sums, void* bias_out, int64_t Nout, int64_t K,
                       int dtype, vitblk_stream_t stream) {
  const int st = validate_affine_fold(w_t, gamma, beta, bias, w_scaled, col_sums, bias_out, Nout,
                                      K, dtype);
  if (st != VITBLK_OK) return st;
  const AffineFoldJob j{w_t, gamma, beta, {bias, nullptr, nullptr}, Nout, Nout, K,
                        w_scaled, col_sums, bias_out};
  VITBLK_LAUNCH(launch_affine_fold(j, nullptr, reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

size_t vitblk_linear_residual_row_stats_workspace_bytes(int64_t M, int64_t Nout) {
  return linear_stats_workspace_bytes(M, Nout);
}

int vitblk_linear_residual_row_stats(const void* a, const void* w_t, const void* residual,
                                     void* out, float* row_stats, int64_t M, int64_t K,
                                     int64_t Nout, double eps, int dtype, void* workspace,
                                     size_t workspace_bytes, vitblk_stream_t stream) {
  const int st = validate_linear_residual_stats(a, w_t, residual, out, row_stats, M, K, Nout, eps,
                                                dtype, workspace, workspace_bytes);
  if (st != VITBLK_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const float feps = static_cast<float>(eps);
  GemmProblem p = linear_problem(a, w_t, out, residual, M, K, Nout, VITBLK_EPI_RESIDUAL, dtype);
  p.row_partials = static_cast<float2*>(workspace);
  if (gemm_row_partials_ok(p)) {
    p.epi = kEpiResidualStats;
    VITBLK_LAUNCH(launch_gemm(p, s));
    VITBLK_LAUNCH(launch_row_stats_from_partials(p.row_partials, Nout / kStatsStrip, row_stats, M,
                                                 Nout, feps, s));
    return VITBLK_OK;
  }
  p.row_partials = nullptr;
  VITBLK_LAUNCH(launch_gemm(p, s));
  VITBLK_LAUNCH(launch_row_stats(out, Nout, row_stats, M, Nout, feps, dtype, s));
  return VITBLK_OK;
}

int vitblk_qkv_projection(const void* xn, const void* w_qkv_t, void* qkv, int64_t M, int64_t D,
                          int dtype, vitblk_stream_t stream) {
  const int st = validate_qkv(xn, w_qkv_t, qkv, M, D, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_gemm(
      linear_problem(xn, w_qkv_t, qkv, nullptr, M, D, 3 * D, VITBLK_EPI_NONE, dtype),
      reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_attention(const void* qkv, void* att, int64_t N, int64_t T, int64_t D, int64_t H,
                     int dtype, vitblk_stream_t stream) {
  const int st = validate_attention(qkv, att, N, T, D, H, dtype);
  if (st != VITBLK_OK) return st;
  const char* base = static_cast<const char*>(qkv);
  const size_t es = elem_size(dtype);
  VITBLK_LAUNCH(launch_attention(base, base + D * es, base + 2 * D * es, 3 * D, att, D, N, T, H,
                                 D / H, dtype, reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_attention_first_queries(const void* qkv, void* att, int64_t N, int64_t T, int64_t D,
                                   int64_t H, int dtype, vitblk_stream_t stream) {
  const int st = validate_attention(qkv, att, N, T, D, H, dtype);
  if (st != VITBLK_OK) return st;
  const char* base = static_cast<const char*>(qkv);
  const size_t es = elem_size(dtype);
  VITBLK_LAUNCH(launch_attention_first_queries(base, base + D * es, base + 2 * D * es, 3 * D, att,
                                               D, N, T, H, D / H, dtype,
                                               reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_linear(const void* a, const void* w_t, const void* residual, void* out, int64_t M,
                  int64_t K, int64_t Nout, int epilogue, int dtype, vitblk_stream_t stream) {
  return vitblk_linear_bias(a, w_t, nullptr, residual, out, M, K, Nout, epilogue, dtype, stream);
}

int vitblk_linear_bias(const void* a, const void* w_t, const void* bias, const void* residual,
                       void* out, int64_t M, int64_t K, int64_t Nout, int epilogue, int dtype,
                       vitblk_stream_t stream) {
  const int st = validate_linear(a, w_t, bias, residual, out, M, K, Nout, epilogue, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_gemm(
      linear_problem(a, w_t, out,
                     (epilogue == VITBLK_EPI_RESIDUAL || epilogue == VITBLK_EPI_GELU_GRAD)
                         ? residual
                         : nullptr,
                     M, K, Nout, epilogue, dtype, bias),
      reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

}  // extern "C"
