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

}  // namespace

size_t elem_size(int dtype) {
  switch (dtype) {
    case VITBLK_FP32: return 4;
    case VITBLK_BF16: return 2;
    default: return 0;
  }
}

int plan_workspace(int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, int dtype,
                   WorkspacePlan* plan) {
  if (!dim_ok(N) || !dim_ok(T) || !dim_ok(D) || !dim_ok(F) || !dim_ok(H))
    return VITBLK_ERR_INVALID_ARG;
  if (D % H != 0) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (N > kMaxDim || T > kMaxDim || D > kMaxDim / 3 || F > kMaxDim || N * T > kMaxDim)
    return VITBLK_ERR_UNSUPPORTED;
  if (D / H > kMaxHeadDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t M = static_cast<size_t>(N) * static_cast<size_t>(T);
  const size_t wide = static_cast<size_t>(F > 3 * D ? F : 3 * D);
  size_t big, act;
  if (!mul_ok(M, wide, &big) || !mul_ok(big, es, &big)) return VITBLK_ERR_UNSUPPORTED;
  if (!mul_ok(M, static_cast<size_t>(D), &act) || !mul_ok(act, es, &act))
    return VITBLK_ERR_UNSUPPORTED;
  WorkspacePlan p;
  p.off_big = 0;
  p.off_act = round_up(big, kRegionAlign);
  p.off_y = p.off_act + round_up(act, kRegionAlign);
  p.total = p.off_y + round_up(act, kRegionAlign);
  if (p.total < big) return VITBLK_ERR_UNSUPPORTED;
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
  const Span o = span(out, M * d * es);
  const Span ws = span(workspace, p.total);
  if (overlap(o, ws)) return VITBLK_ERR_ALIAS;
  for (int i = 0; i < 7; ++i) {
    const Span s = span(ins[i], bytes[i]);
    if (overlap(o, s) || overlap(ws, s)) return VITBLK_ERR_ALIAS;
  }
  if (plan) *plan = p;
  return VITBLK_OK;
}

int validate_layernorm(const void* x, const void* out, int64_t rows, int64_t D, double eps,
                       int dtype) {
  if (x == nullptr || out == nullptr || !aligned16(x) || !aligned16(out))
    return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(rows) || !dim_ok(D)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  int st = check_eps(eps);
  if (st != VITBLK_OK) return st;
  if (rows > kMaxDim || D > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t n = static_cast<size_t>(rows) * static_cast<size_t>(D) * es;
  if (overlap(span(x, n), span(out, n))) return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

int validate_qkv(const void* xn, const void* w_q, const void* w_k, const void* w_v,
                 const void* qkv, int64_t M, int64_t D, int dtype) {
  const void* ins[4] = {xn, w_q, w_k, w_v};
  for (const void* p : ins)
    if (p == nullptr || !aligned16(p)) return VITBLK_ERR_INVALID_ARG;
  if (qkv == nullptr || !aligned16(qkv)) return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(M) || !dim_ok(D)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (M > kMaxDim || D > kMaxDim / 3) return VITBLK_ERR_UNSUPPORTED;
  const size_t m = static_cast<size_t>(M), d = static_cast<size_t>(D);
  const Span o = span(qkv, m * 3 * d * es);
  const size_t bytes[4] = {m * d * es, d * d * es, d * d * es, d * d * es};
  for (int i = 0; i < 4; ++i)
    if (overlap(o, span(ins[i], bytes[i]))) return VITBLK_ERR_ALIAS;
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

int validate_linear(const void* a, const void* w, const void* residual, const void* out,
                    int64_t M, int64_t K, int64_t Nout, int epilogue, int dtype) {
  if (a == nullptr || w == nullptr || out == nullptr) return VITBLK_ERR_INVALID_ARG;
  if (!aligned16(a) || !aligned16(w) || !aligned16(out)) return VITBLK_ERR_INVALID_ARG;
  if (epilogue != VITBLK_EPI_NONE && epilogue != VITBLK_EPI_RESIDUAL &&
      epilogue != VITBLK_EPI_GELU)
    return VITBLK_ERR_INVALID_ARG;
  if (epilogue == VITBLK_EPI_RESIDUAL && (residual == nullptr || !aligned16(residual)))
    return VITBLK_ERR_INVALID_ARG;
  if (!dim_ok(M) || !dim_ok(K) || !dim_ok(Nout)) return VITBLK_ERR_INVALID_ARG;
  const size_t es = elem_size(dtype);
  if (es == 0) return VITBLK_ERR_INVALID_ARG;
  if (M > kMaxDim || K > kMaxDim || Nout > kMaxDim) return VITBLK_ERR_UNSUPPORTED;
  const size_t m = static_cast<size_t>(M), k = static_cast<size_t>(K);
  const size_t n = static_cast<size_t>(Nout);
  const Span o = span(out, m * n * es);
  if (overlap(o, span(a, m * k * es)) || overlap(o, span(w, k * n * es)))
    return VITBLK_ERR_ALIAS;
  if (epilogue == VITBLK_EPI_RESIDUAL && overlap(o, span(residual, m * n * es)))
    return VITBLK_ERR_ALIAS;
  return VITBLK_OK;
}

}  // namespace vitblk
