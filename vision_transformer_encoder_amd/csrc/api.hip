// C ABI of vitblk: argument checks (validate.cpp), workspace carving and the
// launch sequence of one pre-LN encoder block forward.
#include <hip/hip_runtime.h>

#include "kernels.h"
#include "plan.h"
#include "vitblk.h"

using namespace vitblk;

namespace {

// Launch-failure check after each kernel; the first failure ends the call.
#define VITBLK_LAUNCH(expr)                            \
  do {                                                 \
    if ((expr) != hipSuccess) return VITBLK_ERR_HIP;   \
  } while (0)

GemmProblem make_linear(const void* a, int64_t lda, const void* w, int64_t ldw, void* c,
                        int64_t ldc, const void* r, int64_t M, int64_t K, int64_t N, int epi,
                        int dtype) {
  GemmProblem p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.A = a;
  p.lda = lda;
  p.nprob = 1;
  p.B[0] = p.B[1] = p.B[2] = w;
  p.ldb = ldw;
  p.C = c;
  p.ldc = ldc;
  p.col_off[0] = p.col_off[1] = p.col_off[2] = 0;
  p.R = r;
  p.ldr = ldc;
  p.epi = epi;
  p.dtype = dtype;
  return p;
}

GemmProblem make_qkv(const void* xn, const void* wq, const void* wk, const void* wv, void* qkv,
                     int64_t M, int64_t D, int dtype) {
  GemmProblem p = make_linear(xn, D, wq, D, qkv, 3 * D, nullptr, M, D, D, VITBLK_EPI_NONE, dtype);
  p.nprob = 3;
  p.B[1] = wk;
  p.B[2] = wv;
  p.col_off[1] = D;
  p.col_off[2] = 2 * D;
  return p;
}

}  // namespace

extern "C" {

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

int vitblk_forward(const void* x, const void* w_q, const void* w_k, const void* w_v,
                   const void* w_o, const void* w_mlp1, const void* w_mlp2, void* out,
                   int64_t N, int64_t T, int64_t D, int64_t F, int64_t H, double eps,
                   int dtype, void* workspace, size_t workspace_bytes, vitblk_stream_t stream) {
  WorkspacePlan plan;
  const int st = validate_forward(x, w_q, w_k, w_v, w_o, w_mlp1, w_mlp2, out, N, T, D, F, H,
                                  eps, dtype, workspace, workspace_bytes, &plan);
  if (st != VITBLK_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t M = N * T;
  const size_t es = elem_size(dtype);
  char* ws = static_cast<char*>(workspace);
  void* big = ws + plan.off_big;  // qkv [M, 3D], later hidden [M, F]
  void* act = ws + plan.off_act;  // xn, then att, then yn: [M, D]
  void* y = ws + plan.off_y;      // [M, D]
  const float feps = static_cast<float>(eps);
  char* qkv = static_cast<char*>(big);

  // LN1: xn = LN(x)
  VITBLK_LAUNCH(launch_layernorm(x, act, M, D, feps, dtype, s));
  // Q | K | V = xn @ [w_q | w_k | w_v]
  VITBLK_LAUNCH(launch_gemm(make_qkv(act, w_q, w_k, w_v, big, M, D, dtype), s));
  // att = concat_h softmax(Q_h K_h^T / sqrt(dh)) V_h   (overwrites xn)
  VITBLK_LAUNCH(launch_attention(qkv, qkv + D * es, qkv + 2 * D * es, 3 * D, act, D, N, T, H,
                                 D / H, dtype, s));
  // y = x + att @ w_o
  VITBLK_LAUNCH(launch_gemm(
      make_linear(act, D, w_o, D, y, D, x, M, D, D, VITBLK_EPI_RESIDUAL, dtype), s));
  // LN2: yn = LN(y)   (overwrites att)
  VITBLK_LAUNCH(launch_layernorm(y, act, M, D, feps, dtype, s));
  // hidden = GELU(yn @ w_mlp1)   (overwrites qkv)
  VITBLK_LAUNCH(launch_gemm(
      make_linear(act, D, w_mlp1, F, big, F, nullptr, M, D, F, VITBLK_EPI_GELU, dtype), s));
  // out = y + hidden @ w_mlp2
  VITBLK_LAUNCH(launch_gemm(
      make_linear(big, F, w_mlp2, D, out, D, y, M, F, D, VITBLK_EPI_RESIDUAL, dtype), s));
  return VITBLK_OK;
}

int vitblk_layernorm(const void* x, void* out, int64_t rows, int64_t D, double eps, int dtype,
                     vitblk_stream_t stream) {
  const int st = validate_layernorm(x, out, rows, D, eps, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_layernorm(x, out, rows, D, static_cast<float>(eps), dtype,
                                 reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

int vitblk_qkv_projection(const void* xn, const void* w_q, const void* w_k, const void* w_v,
                          void* qkv, int64_t M, int64_t D, int dtype, vitblk_stream_t stream) {
  const int st = validate_qkv(xn, w_q, w_k, w_v, qkv, M, D, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_gemm(make_qkv(xn, w_q, w_k, w_v, qkv, M, D, dtype),
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

int vitblk_linear(const void* a, const void* w, const void* residual, void* out, int64_t M,
                  int64_t K, int64_t Nout, int epilogue, int dtype, vitblk_stream_t stream) {
  const int st = validate_linear(a, w, residual, out, M, K, Nout, epilogue, dtype);
  if (st != VITBLK_OK) return st;
  VITBLK_LAUNCH(launch_gemm(make_linear(a, K, w, Nout, out, Nout,
                                        epilogue == VITBLK_EPI_RESIDUAL ? residual : nullptr, M,
                                        K, Nout, epilogue, dtype),
                            reinterpret_cast<hipStream_t>(stream)));
  return VITBLK_OK;
}

}  // extern "C"
