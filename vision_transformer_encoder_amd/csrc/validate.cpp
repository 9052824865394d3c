// Host-only argument checks for the vitblk C ABI (no HIP headers, no GPU).
#include <cmath>
#include <cstdint>

#include "plan.h"
#include "vitblk.h"

namespace vitblk {
namespace {

struct Span {
  uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Span{a, a + bytes};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int64_t v) { return v > 0; }

// Product of non-negative factors with overflow detection (false on overflow).
bool mul_ok(size_t a, size_t b, size_t* r) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *r = a * b;
  return true;
}

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int check_eps(double eps) {
  return (std::isfinite(eps) && eps >= 0.0) ? VITBLK_OK : VITBLK_ERR_INVALID_ARG;
}

// Shape checks shared by the block-level entry points.
int check_block_dims(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype) {
  if (!dim_ok(N) || !dim_ok(T) || !dim_ok(D) || !dim_ok(F) || !dim_ok(H))
    return VITBLK_ERR_INVALID_ARG;
  if (D % H != 0) return VITBLK_ERR_INVALID_ARG;
  if (elem_size(dtype) == 0) return VITBLK_ERR_INVALID_ARG;
  if (N > kMaxDim || T > kMaxDim || D > kMaxDim / 3 || F > kMaxDim || N * T > kMaxDim)
    return VITBLK_ERR_UNSUPPORTED;
  if (D / H > kMaxHeadDim) return VITBLK_ERR_UNSUPPORTED;
  return VITBLK_OK;
}

// out and workspace against each other and against the read-only inputs.
int check_aliases(const void* const* ins, const size_t* in_bytes, int nin, Span out, Span ws) {
  if (overlap(out, ws)) return VITBLK_ERR_ALIAS;
  for (int i = 0; i < nin; ++i) {
    const Span s = span(ins[i], in_bytes[i]);
    if (overlap(out, s) || overlap(ws, s)) return VITBLK_ERR_ALIAS;
  }
  return VITBLK_OK;
}

}  // namespace

size_t elem_size(int dtype) {
  switch (dtype) {
    case VITBLK_FP32: return 4;
    case VITBLK_BF16: return 2;
    default: return 0;
  }
}

int plan_packed(int64_t D, int64_t F, int dtype, PackedPlan* plan) {
  if (!dim_ok(D) || !dim_ok(F)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (D > kMaxDim / 3 || F > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t d = static_cast<size_t>(D), f = static_cast<size_t>(F);
  size_t dd, df;
  if (!mul_ok(d, d, &dd) || !mul_ok(dd, 3 * es, &dd)) return VITBLK_ERR_UNSUPPORTED;
  if (!mul_ok(d, f, &df) || !mul_ok(df, es, &df)) return VITBLK_ERR_UNSUPPORTED;
  PackedPlan p;
  p.off_qkv = 0;
  p.off_o = round_up(dd, kRegionAlign);             // 3 D^2 elements before
  p.off_1 = p.off_o + round_up(dd / 3, kRegionAlign);
  p.off_2 = p.off_1 + round_up(df, kRegionAlign);
  p.off_cs_qkv = p.off_2 + round_up(df, kRegionAlign);
  p.off_cs_1 = p.off_cs_qkv + round_up(3 * d * sizeof(float), kRegionAlign);
  p.total = p.off_cs_1 + round_up(f * sizeof(float), kRegionAlign);
  *plan = p;
  return VITBLK_OK;
}

int plan_workspace(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                   WorkspacePlan* plan) {
  int st = check_block_dims(N, T, D, F, H, dtype);
  if (st != VITBLK_OK) return st;
  WorkspacePlan p;
  st = plan_packed(D, F, dtype, &p.packed);
  if (st != VITBLK_OK) return st;
  const size_t es = elem_size(dtype);
  const size_t M = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t wide = static_cast<size_t>(F > 3 * D ? F : 3 * D);
  size_t big, act;
  if (!mul_ok(M, wide, &big) || !mul_ok(big, es, &big)) return VITBLK_ERR_UNSUPPORTED;
  if (!mul_ok(M, static_cast<size_t>(D), &act) || !mul_ok(act, es, &act))
    return VITBLK_ERR_UNSUPPORTED;
  p.act_base = 0;
  p.off_big = 0;
  p.off_act = round_up(big, kRegionAlign);
  p.off_y = p.off_act + round_up(act, kRegionAlign);
  p.act_total = p.off_y + round_up(act, kRegionAlign);
  if (p.act_total < big) return VITBLK_ERR_UNSUPPORTED;
  p.total = p.packed.total + p.act_total;
  if (p.total < p.act_total) return VITBLK_ERR_UNSUPPORTED;
  *plan = p;
  return VITBLK_OK;
}

int plan_embed(int64_t B, int64_t C, int64_t H, int64_t W, int64_t P, int64_t D, int dtype,
               EmbedPlan* plan) {
  if (!dim_ok(B) || !dim_ok(C) || !dim_ok(H) || !dim_ok(W) || !dim_ok(P) || !dim_ok(D))
    return VITBLK_ERR_INVALID_ARG;
  if (H % P != 0 || W % P != 0) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (B > kMaxDim || C > kMaxDim || H > kMaxDim || W > kMaxDim || D > kMaxDim)
    return VITBLK_ERR_UNSUPPORTED;
  EmbedPlan p;
  p.N = (H / P) * (W / P);
  const int64_t K = P * P * C;  // P <= H, C, H < 2^31: may overflow only via P * P * C
  if (P > 65536 || K > kMaxDim / 2) return VITBLK_ERR_UNSUPPORTED;
  p.Kp = (K + 63) / 64 * 64;
  if (B * C > kMaxDim || B * (p.N + 1) > kMaxDim || (p.N + 1) > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t rows = static_cast<size_t>(B) * static_cast<size_t>(p.N);
  size_t wt, pa, em;
  if (!mul_ok(static_cast<size_t>(D), static_cast<size_t>(p.Kp) * es, &wt) ||
      !mul_ok(rows, static_cast<size_t>(p.Kp) * es, &pa) ||
      !mul_ok(rows, static_cast<size_t>(D) * es, &em))
    return VITBLK_ERR_UNSUPPORTED;
  if (rows * static_cast<size_t>(p.Kp) > static_cast<size_t>(kMaxDim) * 64)
    return VITBLK_ERR_UNSUPPORTED;
  p.off_wt = 0;
  p.off_patches = round_up(wt, kRegionAlign);
  p.off_embedded = p.off_patches + round_up(pa, kRegionAlign);
  p.total = p.off_embedded + round_up(em, kRegionAlign);
  *plan = p;
  return VITBLK_OK;
}

int validate_patch_embed(const void* images, const void* w_patch, const void* b_patch,
                         const void* cls_token, const void* pos_emb, const void* tokens,
                         int64_t B, int64_t C, int64_t H, int64_t W, int64_t P, int64_t D,
                         int dtype, const void* workspace, size_t workspace_bytes,
                         EmbedPlan* plan) {
  if (images == nullptr || w_patch == nullptr || tokens == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(images) || !aligned16(w_patch) || !aligned16(tokens) || !aligned16(b_patch) ||
      !aligned16(cls_token) || !aligned16(pos_emb))
    return VITBLK_ERR_INVALID_ARG;
  EmbedPlan p;
  int st = plan_embed(B, C, H, W, P, D, dtype, &p);
  if (st != VITBLK_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t d = static_cast<size_t>(D) * es;
  const size_t t = static_cast<size_t>(p.N + (cls_token != nullptr ? 1 : 0));
  const Span o = span(tokens, static_cast<size_t>(B) * t * d);
  const Span ws = span(workspace, p.total);
  if (overlap(o, ws)) return VITBLK_ERR_ALIAS;
  const void* ins[5] = {images, w_patch, b_patch, cls_token, pos_emb};
  const size_t bytes[5] = {static_cast<size_t>(B) * C * H * W * es,
                           static_cast<size_t>(P) * P * C * d, d, d, t * d};
  for (int i = 0; i < 5; ++i) {
    if (ins[i] == nullptr) continue;
    const Span s = span(ins[i], bytes[i]);
    if (overlap(s, o) || overlap(s, ws)) return VITBLK_ERR_ALIAS;
  }
  if (plan) *plan = p;
  return VITBLK_OK;
}

int plan_encoder(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                 EncoderPlan* plan) {
  EncoderPlan p;
  const int st = plan_workspace(N, T, D, F, H, dtype, &p.block);
  if (st != VITBLK_OK) return st;
  const size_t es = elem_size(dtype);
  size_t tok;
  if (!mul_ok(static_cast<size_t>(N) * static_cast<size_t>(T), static_cast<size_t>(D), &tok) ||
      !mul_ok(tok, es, &tok))
    return VITBLK_ERR_UNSUPPORTED;
  tok = round_up(tok, kRegionAlign);
  p.block.act_base = 0;
  p.off_tok0 = p.block.act_total;
  p.off_tok1 = p.off_tok0 + tok;
  p.total = p.off_tok1 + tok;
  if (p.total < p.off_tok1) return VITBLK_ERR_UNSUPPORTED;
  *plan = p;
  return VITBLK_OK;
}

int validate_forward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                     const void* w_o, const void* w_mlp1, const void* w_mlp2,
                     const void* out, int64_t N, int64_t T, int64_t D, int64_t F,
                     int64_t H, double eps, int dtype, const void* workspace,
                     size_t workspace_bytes, WorkspacePlan* plan) {
  const void* ins[7] = {x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2};
  for (const void* p : ins)
    if (p == nullptr || !aligned16(p)) return VITBLK_ERR_INVALID_ARG;
  if (out == nullptr || !aligned16(out)) return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  WorkspacePlan p;
  st = plan_workspace(N, T, D, F, H, dtype, &p);
  if (st != VITBLK_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t M = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t d = static_cast<size_t>(D), f = static_cast<size_t>(F);
  const size_t bytes[7] = {M * d * es, d * d * es, d * d * es, d * d * es,
                           d * d * es, d * f * es, f * d * es};
  st = check_aliases(ins, bytes, 7, span(out, M * d * es), span(workspace, p.total));
  if (st != VITBLK_OK) return st;
  p.act_base = p.packed.total;
  if (plan) *plan = p;
  return VITBLK_OK;
}

int validate_forward_packed(const void* x, const void* packed, const void* out, int64_t N,
                            int64_t T, int64_t D, int64_t F, int64_t H, double eps, int dtype,
                            const void* workspace, size_t workspace_bytes,
                            WorkspacePlan* plan) {
  if (x == nullptr || packed == nullptr || out == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(packed) || !aligned16(out)) return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  WorkspacePlan p;
  st = plan_workspace(N, T, D, F, H, dtype, &p);
  if (st != VITBLK_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < p.act_total) return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t M = static_cast<size_t>(N) * static_cast<size_t>(T);
  const void* ins[2] = {x, packed};
  const size_t bytes[2] = {M * static_cast<size_t>(D) * es, p.packed.total};
  st = check_aliases(ins, bytes, 2, span(out, M * static_cast<size_t>(D) * es),
                     span(workspace, p.act_total));
  if (st != VITBLK_OK) return st;
  p.act_base = 0;
  if (plan) *plan = p;
  return VITBLK_OK;
}

int validate_pack(const void* w_q, const void* w_k, const void* w_v, const void* w_o,
                  const void* w_mlp1, const void* w_mlp2, const void* packed, int64_t D,
                  int64_t F, int dtype, PackedPlan* plan) {
  const void* ins[6] = {w_q, w_k, w_v, w_o, w_mlp1, w_mlp2};
  for (const void* p : ins)
    if (p == nullptr || !aligned16(p)) return VITBLK_ERR_INVALID_ARG;
  if (packed == nullptr || !aligned16(packed)) return VITBLK_ERR_INVALID_ARG;
  PackedPlan p;
  int st = plan_packed(D, F, dtype, &p);
  if (st != VITBLK_OK) return st;
  const size_t es = elem_size(dtype);
  const size_t d = static_cast<size_t>(D), f = static_cast<size_t>(F);
  const size_t bytes[6] = {d * d * es, d * d * es, d * d * es, d * d * es, d * f * es,
                           f * d * es};
  const Span o = span(packed, p.total);
  for (int i = 0; i < 6; ++i)
    if (overlap(o, span(ins[i], bytes[i]))) return VITBLK_ERR_ALIAS;
  if (plan) *plan = p;
  return VITBLK_OK;
}

int validate_layernorm(const void* x, const void* gamma, const void* beta, const void* out,
                       int64_t rows, int64_t D, double eps, int dtype) {
  if (x == nullptr || out == nullptr || !aligned16(x) || !aligned16(out))
    return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(gamma) || !aligned16(beta)) return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(rows) || !dim_ok(D)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  if (rows > kMaxDim || D > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(D) * es;
  const Span o = span(out, n);
  if (overlap(span(x, n), o)) return VITBLK_ERR_ALIAS;
  const size_t v = static_cast<size_t>(D) * es;
  if ((gamma != nullptr && overlap(span(gamma, v), o)) ||
      (beta != nullptr && overlap(span(beta, v), o)))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_qkv(const void* xn, const void* w_qkv_t, const void* qkv, int64_t M, int64_t D,
                 int dtype) {
  if (xn == nullptr || w_qkv_t == nullptr || qkv == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(xn) || !aligned16(w_qkv_t) || !aligned16(qkv)) return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(M) || !dim_ok(D)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (M > kMaxDim || D > kMaxDim / 3) return VITBLK_ERR_UNSUPPORTED;
  const size_t m = static_cast<size_t>(M), d = static_cast<size_t>(D);
  const Span o = span(qkv, m * 3 * d * es);
  if (overlap(o, span(xn, m * d * es)) || overlap(o, span(w_qkv_t, 3 * d * d * es)))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_attention(const void* qkv, const void* att, int64_t N, int64_t T, int64_t D,
                       int64_t H, int dtype) {
  if (qkv == nullptr || att == nullptr || !aligned16(qkv) || !aligned16(att))
    return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(N) || !dim_ok(T) || !dim_ok(D) || !dim_ok(H) || D % H != 0)
    return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (N > kMaxDim || T > kMaxDim || D > kMaxDim / 3 || N * T > kMaxDim)
    return VITBLK_ERR_UNSUPPORTED;
  if (D / H > kMaxHeadDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t m = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t d = static_cast<size_t>(D);
  if (overlap(span(qkv, m * 3 * d * es), span(att, m * d * es))) return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_linear(const void* a, const void* w, const void* bias, const void* residual,
                    const void* out, int64_t M, int64_t K, int64_t Nout, int epilogue,
                    int dtype) {
  if (a == nullptr || w == nullptr || out == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w) || !aligned16(out) || !aligned16(bias))
    return VITBLK_ERR_INVALID_ARG;
  if (epilogue != VITBLK_EPI_NONE && epilogue != VITBLK_EPI_RESIDUAL &&
      epilogue != VITBLK_EPI_GELU && epilogue != VITBLK_EPI_GELU_GRAD)
    return VITBLK_ERR_INVALID_ARG;
  const bool reads_r = epilogue == VITBLK_EPI_RESIDUAL || epilogue == VITBLK_EPI_GELU_GRAD;
  if (reads_r && (residual == nullptr || !aligned16(residual))) return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(M) || !dim_ok(K) || !dim_ok(Nout)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (M > kMaxDim || K > kMaxDim || Nout > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K);
  const size_t n = static_cast<size_t>(Nout);
  const Span o = span(out, m * n * es);
  if (overlap(o, span(a, m * k * es)) || overlap(o, span(w, k * n * es)))
    return VITBLK_ERR_ALIAS;
  if (reads_r && overlap(o, span(residual, m * n * es))) return VITBLK_ERR_ALIAS;
  if (bias != nullptr && overlap(o, span(bias, n * es))) return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

size_t linear_stats_workspace_bytes(int64_t M, int64_t Nout) {
  if (!dim_ok(M) || !dim_ok(Nout) || M > kMaxDim || Nout > kMaxDim) return 0;
  const size_t strips = (static_cast<size_t>(Nout) + 63) / 64;
  return static_cast<size_t>(M) * strips * 2 * sizeof(float);
}

int validate_linear_residual_stats(const void* a, const void* w, const void* residual,
                                   const void* out, const float* stats, int64_t M, int64_t K,
                                   int64_t Nout, double eps, int dtype, const void* workspace,
                                   size_t workspace_bytes) {
  int st = validate_linear(a, w, nullptr, residual, out, M, K, Nout, VITBLK_EPI_RESIDUAL, dtype);
  if (st != VITBLK_OK) return st;
  if (stats == nullptr || (reinterpret_cast<uintptr_t>(stats) & 7u) != 0)
    return VITBLK_ERR_INVALID_ARG;
  st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  const size_t need = linear_stats_workspace_bytes(M, Nout);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need)
    return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K);
  const size_t n = static_cast<size_t>(Nout);
  const Span so = span(stats, m * 2 * sizeof(float)), ws = span(workspace, need);
  const Span o = span(out, m * n * es), sa = span(a, m * k * es), sw = span(w, k * n * es),
             sr = span(residual, m * n * es);
  if (overlap(so, o) || overlap(so, sa) || overlap(so, sw) || overlap(so, sr) ||
      overlap(so, ws) || overlap(ws, o) || overlap(ws, sa) || overlap(ws, sw) ||
      overlap(ws, sr))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_row_stats(const void* x, const float* stats, int64_t rows, int64_t D, double eps,
                       int dtype) {
  if (x == nullptr || stats == nullptr || !aligned16(x)) return VITBLK_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(stats) & 7u) != 0) return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(rows) || !dim_ok(D)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  const int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  if (rows > kMaxDim || D > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t r = static_cast<size_t>(rows);
  if (overlap(span(stats, r * 2 * sizeof(float)), span(x, r * static_cast<size_t>(D) * es)))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_linear_normed(const void* a, const void* w, const float* col_sums,
                           const float* row_stats, const void* bias, const void* out, int64_t M,
                           int64_t K, int64_t Nout, int epilogue, int dtype) {
  if (epilogue != VITBLK_EPI_NONE && epilogue != VITBLK_EPI_GELU) return VITBLK_ERR_INVALID_ARG;
  if (col_sums == nullptr || row_stats == nullptr || !aligned16(col_sums) ||
      (reinterpret_cast<uintptr_t>(row_stats) & 7u) != 0)
    return VITBLK_ERR_INVALID_ARG;
  const int st = validate_linear(a, w, bias, nullptr, out, M, K, Nout, epilogue, dtype);
  if (st != VITBLK_OK) return st;
  const size_t m = static_cast<size_t>(M), n = static_cast<size_t>(Nout);
  const Span o = span(out, m * n * elem_size(dtype));
  if (overlap(o, span(col_sums, n * sizeof(float))) ||
      overlap(o, span(row_stats, m * 2 * sizeof(float))))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_affine_fold(const void* w_t, const void* gamma, const void* beta, const void* bias,
                         const void* w_scaled, const float* col_sums, const void* bias_out,
                         int64_t Nout, int64_t K, int dtype) {
  if (w_t == nullptr || w_scaled == nullptr || col_sums == nullptr || bias_out == nullptr)
    return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(w_t) || !aligned16(w_scaled) || !aligned16(gamma) || !aligned16(beta) ||
      !aligned16(col_sums) || (reinterpret_cast<uintptr_t>(bias) & 1u) != 0 ||
      (reinterpret_cast<uintptr_t>(bias_out) & 1u) != 0)
    return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(Nout) || !dim_ok(K)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (dtype != VITBLK_BF16 || K % 8 != 0 || Nout > kMaxDim || K > kMaxDim)
    return VITBLK_ERR_UNSUPPORTED;
  const size_t n = static_cast<size_t>(Nout), k = static_cast<size_t>(K);
  const Span outs[3] = {span(w_scaled, n * k * es), span(col_sums, n * sizeof(float)),
                        span(bias_out, n * es)};
  const Span ins[4] = {span(w_t, n * k * es), span(gamma, gamma != nullptr ? k * es : 0),
                       span(beta, beta != nullptr ? k * es : 0),
                       span(bias, bias != nullptr ? n * es : 0)};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(outs[i], ins[j])) return VITBLK_ERR_ALIAS;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return VITBLK_ERR_ALIAS;
  }
  return VITBLK_OK;
}

int validate_encoder(const void* x, const void* const* packed, const vitblk_affine_params* params,
                     int64_t L, const void* final_gamma, const void* final_beta,
                     const void* out, const void* cls_out, int64_t N, int64_t T, int64_t D,
                     int64_t F, int64_t H, double eps, int dtype, const void* workspace,
                     size_t workspace_bytes, EncoderPlan* plan) {
  if (x == nullptr || packed == nullptr || L <= 0) return VITBLK_ERR_INVALID_ARG;
  if (out == nullptr && cls_out == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(out) || !aligned16(cls_out) || !aligned16(final_gamma) ||
      !aligned16(final_beta))
    return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  EncoderPlan p;
  st = plan_encoder(N, T, D, F, H, dtype, &p);
  if (st != VITBLK_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t m = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t d = static_cast<size_t>(D) * es;
  const Span ws = span(workspace, p.total);
  const Span o = span(out, out != nullptr ? m * d : 0);
  const Span c = span(cls_out, cls_out != nullptr ? static_cast<size_t>(N) * d : 0);
  if (overlap(o, c) || overlap(o, ws) || overlap(c, ws)) return VITBLK_ERR_ALIAS;
  // Read-only inputs against every output and the workspace.
  auto clear = [&](const void* ptr, size_t bytes) {
    const Span s = span(ptr, bytes);
    return !(overlap(s, o) || overlap(s, c) || overlap(s, ws));
  };
  if (!clear(x, m * d)) return VITBLK_ERR_ALIAS;
  if ((final_gamma != nullptr && !clear(final_gamma, d)) ||
      (final_beta != nullptr && !clear(final_beta, d)))
    return VITBLK_ERR_ALIAS;
  for (int64_t l = 0; l < L; ++l) {
    if (packed[l] == nullptr || !aligned16(packed[l])) return VITBLK_ERR_INVALID_ARG;
    if (!clear(packed[l], p.block.packed.total)) return VITBLK_ERR_ALIAS;
    if (params != nullptr) {
      // The block-level checks against out and the workspace, then cls_out.
      st = validate_affine_params(&params[l], out, N * T, D, F, dtype, workspace, p.total);
      if (st != VITBLK_OK) return st;
      st = validate_affine_params(&params[l], cls_out, N, D, F, dtype, workspace, p.total);
      if (st != VITBLK_OK) return st;
    }
  }
  if (plan) *plan = p;
  return VITBLK_OK;
}

int validate_affine_params(const vitblk_affine_params* params, const void* out, int64_t rows,
                           int64_t D, int64_t F, int dtype, const void* workspace,
                           size_t workspace_bytes) {
  if (params == nullptr) return VITBLK_OK;
  const size_t es = elem_size(dtype);
  if (es == 0 || !dim_ok(rows) || !dim_ok(D) || !dim_ok(F)) return VITBLK_ERR_INVALID_ARG;
  const size_t d = static_cast<size_t>(D) * es, f = static_cast<size_t>(F) * es;
  const void* ptrs[10] = {params->ln1_gamma, params->ln1_beta, params->b_q,
                          params->b_k,       params->b_v,      params->b_o,
                          params->ln2_gamma, params->ln2_beta, params->b_mlp1,
                          params->b_mlp2};
  const size_t bytes[10] = {d, d, d, d, d, d, d, d, f, d};
  const Span o = span(out, out != nullptr ? static_cast<size_t>(rows) * d : 0);
  const Span w = span(workspace, workspace_bytes);
  for (int i = 0; i < 10; ++i) {
    if (ptrs[i] == nullptr) continue;
    if (!aligned16(ptrs[i])) return VITBLK_ERR_INVALID_ARG;
    const Span s = span(ptrs[i], bytes[i]);
    if (overlap(s, o) || overlap(s, w)) return VITBLK_ERR_ALIAS;
  }
  return VITBLK_OK;
}

int wgrad_split(int64_t M, int64_t I, int64_t J) {
  if (!dim_ok(M) || !dim_ok(I) || !dim_ok(J)) return 1;
  const int64_t tiles = ((I + 255) / 256) * ((J + 255) / 256);
  int64_t split = tiles >= 256 ? 1 : 256 / tiles;
  const int64_t by_rows = M / 512 > 1 ? M / 512 : 1;
  if (split > by_rows) split = by_rows;
  return static_cast<int>(split);
}

size_t wgrad_partial_bytes(int64_t M, int64_t I, int64_t J) {
  if (!dim_ok(M) || !dim_ok(I) || !dim_ok(J) || I > kMaxDim || J > kMaxDim) return 0;
  size_t n;
  if (!mul_ok(static_cast<size_t>(I), static_cast<size_t>(J), &n) ||
      !mul_ok(n, static_cast<size_t>(wgrad_split(M, I, J)) * 4, &n))
    return 0;
  return round_up(n, kRegionAlign);
}

size_t attention_stats_bytes(int64_t N, int64_t T, int64_t H) {
  if (!dim_ok(N) || !dim_ok(T) || !dim_ok(H)) return 0;
  size_t n;
  if (!mul_ok(static_cast<size_t>(N) * static_cast<size_t>(T), static_cast<size_t>(H), &n) ||
      !mul_ok(n, 3 * sizeof(float), &n))
    return 0;
  return round_up(n, kRegionAlign);
}

int plan_backward(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                  BackwardPlan* plan) {
  int st = check_block_dims(N, T, D, F, H, dtype);
  if (st != VITBLK_OK) return st;
  BackwardPlan p;
  st = plan_packed(D, F, dtype, &p.packed);
  if (st != VITBLK_OK) return st;
  const size_t es = elem_size(dtype);
  const size_t M = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t d = static_cast<size_t>(D), f = static_cast<size_t>(F);
  const size_t wide = f > 3 * d ? f : 3 * d;
  size_t act, qkv, zb, hb, wcat;
  if (!mul_ok(M, d * es, &act) || !mul_ok(M, 3 * d * es, &qkv) || !mul_ok(M, wide * es, &zb) ||
      !mul_ok(M, f * es, &hb) || !mul_ok(d, 3 * d * es, &wcat))
    return VITBLK_ERR_UNSUPPORTED;
  act = round_up(act, kRegionAlign);
  // The largest of the four weight gradients' partials.
  size_t part = 0;
  const int64_t shapes[4][2] = {{F, D}, {D, F}, {D, D}, {D, 3 * D}};
  for (const auto& sh : shapes) {
    const size_t b = wgrad_partial_bytes(static_cast<int64_t>(M), sh[0], sh[1]);
    if (b == 0) return VITBLK_ERR_UNSUPPORTED;
    if (b > part) part = b;
  }
  const size_t stats = attention_stats_bytes(N, T, H);
  if (stats == 0) return VITBLK_ERR_UNSUPPORTED;
  size_t o = p.packed.total;
  p.off_wcat = o;
  o += round_up(wcat, kRegionAlign);
  p.off_xn = o;
  o += act;
  p.off_qkv = o;
  o += round_up(qkv, kRegionAlign);
  p.off_att = o;
  o += act;
  p.off_y = o;
  o += act;
  p.off_yn = o;
  o += act;
  p.off_z = o;
  o += round_up(zb, kRegionAlign);
  p.off_h = o;
  o += round_up(hb, kRegionAlign);
  p.off_dy = o;
  o += act;
  p.off_stats = o;
  o += stats;
  p.off_partial = o;
  p.partial_bytes = part;
  o += part;
  if (o < part) return VITBLK_ERR_UNSUPPORTED;
  p.total = o;
  *plan = p;
  return VITBLK_OK;
}

int validate_backward(const void* x, const void* const* w, const void* dout,
                      void* const* grads, int64_t N, int64_t T, int64_t D, int64_t F,
                      int64_t H, double eps, int dtype, const void* workspace,
                      size_t workspace_bytes, BackwardPlan* plan) {
  if (w == nullptr || grads == nullptr) return VITBLK_ERR_INVALID_ARG;
  const void* ins[8] = {x, w[0], w[1], w[2], w[3], w[4], w[5], dout};
  for (const void* q : ins)
    if (q == nullptr || !aligned16(q)) return VITBLK_ERR_INVALID_ARG;
  for (int i = 0; i < 7; ++i)
    if (grads[i] == nullptr || !aligned16(grads[i])) return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  BackwardPlan p;
  st = plan_backward(N, T, D, F, H, dtype, &p);
  if (st != VITBLK_OK) return st;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < p.total) return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t M = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t d = static_cast<size_t>(D), f = static_cast<size_t>(F);
  const size_t in_bytes[8] = {M * d * es, d * d * es, d * d * es, d * d * es,
                              d * d * es, d * f * es, f * d * es, M * d * es};
  const size_t out_bytes[7] = {M * d * es, d * d * es, d * d * es, d * d * es,
                               d * d * es, d * f * es, f * d * es};
  const Span ws = span(workspace, p.total);
  for (int i = 0; i < 7; ++i) {
    const Span o = span(grads[i], out_bytes[i]);
    if (overlap(o, ws)) return VITBLK_ERR_ALIAS;
    for (int j = 0; j < 8; ++j)
      if (overlap(o, span(ins[j], in_bytes[j]))) return VITBLK_ERR_ALIAS;
    for (int j = i + 1; j < 7; ++j)
      if (overlap(o, span(grads[j], out_bytes[j]))) return VITBLK_ERR_ALIAS;
  }
  for (int j = 0; j < 8; ++j)
    if (overlap(ws, span(ins[j], in_bytes[j]))) return VITBLK_ERR_ALIAS;
  if (plan) *plan = p;
  return VITBLK_OK;
}

int validate_weight_grad(const void* a, const void* b, const void* out, int64_t M, int64_t I,
                         int64_t J, int dtype, const void* workspace, size_t workspace_bytes) {
  if (a == nullptr || b == nullptr || out == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned16(out)) return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(M) || !dim_ok(I) || !dim_ok(J)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (M > kMaxDim || I > kMaxDim || J > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t need = wgrad_partial_bytes(M, I, J);
  if (need == 0) return VITBLK_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < need) return VITBLK_ERR_WORKSPACE;
  const size_t m = static_cast<size_t>(M), i = static_cast<size_t>(I), j = static_cast<size_t>(J);
  const Span o = span(out, i * j * es);
  const Span ws = span(workspace, need);
  const Span sa = span(a, m * i * es), sb = span(b, m * j * es);
  if (overlap(o, ws) || overlap(o, sa) || overlap(o, sb) || overlap(ws, sa) || overlap(ws, sb))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_layernorm_backward(const void* x, const void* g, const void* residual,
                                const void* dx, int64_t rows, int64_t D, double eps, int dtype) {
  if (x == nullptr || g == nullptr || dx == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(g) || !aligned16(dx) || !aligned16(residual))
    return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(rows) || !dim_ok(D)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  if (rows > kMaxDim || D > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(D) * es;
  const Span o = span(dx, n);
  if (overlap(o, span(x, n)) || overlap(o, span(g, n))) return VITBLK_ERR_ALIAS;
  if (residual != nullptr && overlap(o, span(residual, n))) return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_attention_backward(const void* qkv, const void* datt, const void* dqkv, int64_t N,
                                int64_t T, int64_t D, int64_t H, int dtype,
                                const void* workspace, size_t workspace_bytes) {
  if (datt == nullptr || dqkv == nullptr || !aligned16(datt) || !aligned16(dqkv))
    return VITBLK_ERR_INVALID_ARG;
  int st = validate_attention(qkv, datt, N, T, D, H, dtype);
  if (st != VITBLK_OK) return st;
  const size_t need = attention_stats_bytes(N, T, H);
  if (need == 0) return VITBLK_ERR_UNSUPPORTED;
  if (workspace == nullptr || !aligned16(workspace)) return VITBLK_ERR_WORKSPACE;
  if (workspace_bytes < need) return VITBLK_ERR_WORKSPACE;
  const size_t es = elem_size(dtype);
  const size_t m = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t d = static_cast<size_t>(D);
  const Span o = span(dqkv, m * 3 * d * es);
  const Span ws = span(workspace, need);
  const Span sq = span(qkv, m * 3 * d * es), sd = span(datt, m * d * es);
  if (overlap(o, sq) || overlap(o, sd) || overlap(o, ws) || overlap(ws, sq) || overlap(ws, sd))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

}  // namespace vitblk
