// Backward-pass kernels of the block on the VALU (fp32 arithmetic): the
// any-shape LayerNorm backward, the any-shape weight gradient and the
// partial-sum reduction of every weight gradient, and the any-shape
// attention backward.  The matrix-core paths fall back to these for shapes
// they do not take and for fp32 tensors.
//
// The gradients are those of the block's forward definition
// (crackedaicode.com "ViT Encoder Block"), as training needs them
// (nipunbatra.github.io vision1 transcript, Pages 88 and 113).
#include <math.h>

#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kThreads = 256;

__device__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

// ---------------------------------------------------------- LayerNorm backward
//
// LN(x) = (x - mu) * r with r = 1 / sqrt(var + eps) (population variance).
// Its Jacobian-transpose product is r * (g - mean(g) - xhat * mean(g * xhat)):
// the mean term because every x_j moves mu, the xhat term because it moves
// var.  One row per workgroup; statistics in fp32.
template <typename T>
__global__ __launch_bounds__(kThreads) void ln_backward_kernel(const T* __restrict__ x,
                                                               const T* __restrict__ g,
                                                               const T* __restrict__ res,
                                                               T* __restrict__ dx, int64_t D,
                                                               float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * D;
  const T* gr = g + row * D;
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kThreads) s += load_f32(xr + i);
  const float inv_d = 1.0f / static_cast<float>(D);
  const float mean = block_sum(s, red) * inv_d;
  float q = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kThreads) {
    const float d = load_f32(xr + i) - mean;
    q += d * d;
  }
  const float rstd = 1.0f / sqrtf(block_sum(q, red) * inv_d + eps);
  float sg = 0.f, sgx = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kThreads) {
    const float gv = load_f32(gr + i);
    sg += gv;
    sgx += gv * (load_f32(xr + i) - mean) * rstd;
  }
  const float mg = block_sum(sg, red) * inv_d;
  const float mgx = block_sum(sgx, red) * inv_d;
  for (int64_t i = threadIdx.x; i < D; i += kThreads) {
    const float xhat = (load_f32(xr + i) - mean) * rstd;
    float o = rstd * (load_f32(gr + i) - mg - xhat * mgx);
    if (res != nullptr) o += load_f32(res + row * D + i);
    store_f32(dx + row * D + i, o);
  }
}

// -------------------------------------------------------- weight gradient
//
// 64x64 output tile per workgroup over one range of token rows: 16 rows of
// A and B staged in LDS per step (coalesced along the feature axis), 4x4
// outputs per thread, written to that range's fp32 partial.
template <typename T>
__global__ __launch_bounds__(kThreads) void wgrad_generic_kernel(WgradProblem p,
                                                                 float* __restrict__ partial,
                                                                 int64_t it, int64_t jt,
                                                                 int64_t row0,
                                                                 int64_t rows_per_split,
                                                                 bool accumulate) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int64_t b = blockIdx.x;
  const int64_t tile = b % (it * jt), sp = b / (it * jt);
  const int64_t i0 = (tile / jt) * 64, j0 = (tile % jt) * 64;
  const int64_t m_lo = row0 + sp * rows_per_split;
  const int64_t m_hi = m_lo + rows_per_split < p.M ? m_lo + rows_per_split : p.M;
  const T* A = static_cast<const T*>(p.A);
  const T* B = static_cast<const T*>(p.B);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int64_t m0 = m_lo; m0 < m_hi; m0 += 16) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int e = tid + u * kThreads;
      const int r = e >> 6, c = e & 63;
      const int64_t gm = m0 + r;
      const bool in = gm < m_hi;
      As[r][c] = (in && i0 + c < p.I) ? load_f32(A + gm * p.lda + i0 + c) : 0.f;
      Bs[r][c] = (in && j0 + c < p.J) ? load_f32(B + gm * p.ldb + j0 + c) : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bb[j] = Bs[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * bb[j];
    }
    __syncthreads();
  }
  float* out = partial + sp * p.I * p.J;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t gi = i0 + ty * 4 + i;
    if (gi >= p.I) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gj = j0 + tx * 4 + j;
      if (gj < p.J) {
        float* o = out + gi * p.J + gj;
        *o = accumulate ? *o + acc[i][j] : acc[i][j];
      }
    }
  }
}

// Sum of the split partials in split order (deterministic), rounded once,
// scattered to the output segments; 4 consecutive elements per thread (J and
// the segment width are multiples of 4).
template <typename T>
__global__ __launch_bounds__(kThreads) void wgrad_reduce4_kernel(WgradProblem p,
                                                                 const float* __restrict__ partial,
                                                                 int split) {
  const int64_t n = p.I * p.J, n4 = n / 4;
  for (int64_t e4 = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; e4 < n4;
       e4 += static_cast<int64_t>(gridDim.x) * kThreads) {
    float4 acc = reinterpret_cast<const float4*>(partial)[e4];
    for (int s = 1; s < split; ++s) {
      const float4 v = reinterpret_cast<const float4*>(partial + s * n)[e4];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const int64_t e = e4 * 4, i = e / p.J, j = e % p.J;
    const int64_t seg = j / p.seg;
    T* c = static_cast<T*>(p.C[seg]) + i * p.ldc + (j - seg * p.seg);
    store_f32(c + 0, acc.x);
    store_f32(c + 1, acc.y);
    store_f32(c + 2, acc.z);
    store_f32(c + 3, acc.w);
  }
}

template <typename T>
__global__ __launch_bounds__(kThreads) void wgrad_reduce_kernel(WgradProblem p,
                                                                const float* __restrict__ partial,
                                                                int split) {
  const int64_t n = p.I * p.J;
  for (int64_t e = blockIdx.x * static_cast<int64_t>(kThreads) + threadIdx.x; e < n;
       e += static_cast<int64_t>(gridDim.x) * kThreads) {
    float acc = 0.f;
    for (int s = 0; s < split; ++s) acc += partial[s * n + e];
    const int64_t i = e / p.J, j = e % p.J;
    const int64_t seg = j / p.seg;
    T* c = static_cast<T*>(p.C[seg]);
    store_f32(c + i * p.ldc + (j - seg * p.seg), acc);
  }
}

// ------------------------------------------------------- attention backward
//
// Per sequence and head, with S = Q K^T * scale, P = softmax(S) (rows),
// dP = dO V^T, Dsum_i = sum_j P_ij dP_ij and dS = P * (dP - Dsum):
//   dQ = dS K * scale, dK = dS^T Q * scale, dV = P^T dO.
// Two passes: one wave per query (its softmax statistics, Dsum and dQ row),
// then one wave per key (its dK and dV rows, from the stored statistics).
// Each lane handles one key (or query) at a time for the dot products and
// head features lane, lane + 64, ... for the accumulations.
constexpr int kMaxDhPerLane = 16;  // head width <= 1024

template <typename T>
__device__ float dot_row(const float* __restrict__ a, const T* __restrict__ row, int64_t dh) {
  float d = 0.f;
  for (int64_t c = 0; c < dh; ++c) d += a[c] * load_f32(row + c);
  return d;
}

// The scaled score, rounded on its own (contraction off: a multiply fused
// into the following subtraction would skip this rounding at some call sites
// and not at others), so every pass sees the same score and a query with one
// key gets P = 1 exactly.
template <typename T>
__device__ float score(const float* __restrict__ a, const T* __restrict__ row, int64_t dh,
                       float scale) {
#pragma clang fp contract(off)
  const float d = dot_row(a, row, dh);
  return d * scale;
}

template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_query_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ld,
    const T* __restrict__ d_o, int64_t ldo, T* __restrict__ dq, int64_t ldd, int64_t T_,
    int64_t H, int64_t dh, float scale, float* __restrict__ max_out, float* __restrict__ sum_out,
    float* __restrict__ dsum_out) {
  extern __shared__ float sm[];
  float* qs = sm;            // [dh]
  float* dos = sm + dh;      // [dh]
  float* ws = sm + 2 * dh;   // [64]
  int64_t b = blockIdx.x;
  const int64_t t = b % T_;
  b /= T_;
  const int64_t h = b % H;
  const int64_t n = b / H;
  const int lane = threadIdx.x;
  const int64_t base = n * T_, hoff = h * dh;
  for (int64_t c = lane; c < dh; c += 64) {
    qs[c] = load_f32(q + (base + t) * ld + hoff + c);
    dos[c] = load_f32(d_o + (base + t) * ldo + hoff + c);
  }
  __syncthreads();
  // Softmax statistics of the query's score row.
  float m = -INFINITY, l = 0.f;
  for (int64_t j0 = 0; j0 < T_; j0 += 64) {
    const int64_t j = j0 + lane;
    const float s = j < T_ ? score(qs, k + (base + j) * ld + hoff, dh, scale) : -INFINITY;
    const float mnew = fmaxf(m, wave_max(s));
    l = l * expf(m - mnew) + wave_sum(j < T_ ? expf(s - mnew) : 0.f);
    m = mnew;
  }
  // P_ij = exp(S_ij - m) / l (the maximum and the sum kept apart, not folded
  // into a log-sum-exp, so that a row with one key gets P = 1 exactly).
  const float inv_l = 1.0f / l;
  // Dsum = sum_j P_ij dP_ij.
  float ds = 0.f;
  for (int64_t j0 = 0; j0 < T_; j0 += 64) {
    const int64_t j = j0 + lane;
    if (j < T_) {
      const float p = expf(score(qs, k + (base + j) * ld + hoff, dh, scale) - m) * inv_l;
      ds += p * dot_row(dos, v + (base + j) * ld + hoff, dh);
    }
  }
  ds = wave_sum(ds);
  // dQ row = sum_j dS_ij K_j * scale.
  float acc[kMaxDhPerLane];
#pragma unroll
  for (int r = 0; r < kMaxDhPerLane; ++r) acc[r] = 0.f;
  for (int64_t j0 = 0; j0 < T_; j0 += 64) {
    const int64_t j = j0 + lane;
    float w = 0.f;
    if (j < T_) {
      const float p = expf(score(qs, k + (base + j) * ld + hoff, dh, scale) - m) * inv_l;
      w = p * (dot_row(dos, v + (base + j) * ld + hoff, dh) - ds);
    }
    ws[lane] = w;
    __syncthreads();
    const int64_t jn = T_ - j0 < 64 ? T_ - j0 : 64;
    for (int64_t jj = 0; jj < jn; ++jj) {
      const float wj = ws[jj];
      const T* krow = k + (base + j0 + jj) * ld + hoff;
#pragma unroll
      for (int r = 0; r < kMaxDhPerLane; ++r) {
        const int64_t c = lane + 64 * r;
        if (c < dh) acc[r] += wj * load_f32(krow + c);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kMaxDhPerLane; ++r) {
    const int64_t c = lane + 64 * r;
    if (c < dh) store_f32(dq + (base + t) * ldd + hoff + c, acc[r] * scale);
  }
  if (lane == 0) {
    const int64_t si = (n * H + h) * T_ + t;
    max_out[si] = m;
    sum_out[si] = l;
    dsum_out[si] = ds;
  }
}

template <typename T>
__global__ __launch_bounds__(64) void attn_bwd_key_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ld,
    const T* __restrict__ d_o, int64_t ldo, T* __restrict__ dk, T* __restrict__ dv, int64_t ldd,
    int64_t T_, int64_t H, int64_t dh, float scale, const float* __restrict__ max_in,
    const float* __restrict__ sum_in, const float* __restrict__ dsum_in) {
  extern __shared__ float sm[];
  float* ks = sm;             // [dh]
  float* vs = sm + dh;        // [dh]
  float* ps = sm + 2 * dh;    // [64]
  float* dss = ps + 64;       // [64]
  int64_t b = blockIdx.x;
  const int64_t j = b % T_;
  b /= T_;
  const int64_t h = b % H;
  const int64_t n = b / H;
  const int lane = threadIdx.x;
  const int64_t base = n * T_, hoff = h * dh;
  const int64_t sbase = (n * H + h) * T_;
  for (int64_t c = lane; c < dh; c += 64) {
    ks[c] = load_f32(k + (base + j) * ld + hoff + c);
    vs[c] = load_f32(v + (base + j) * ld + hoff + c);
  }
  __syncthreads();
  float ak[kMaxDhPerLane], av[kMaxDhPerLane];
#pragma unroll
  for (int r = 0; r < kMaxDhPerLane; ++r) ak[r] = av[r] = 0.f;
  for (int64_t i0 = 0; i0 < T_; i0 += 64) {
    const int64_t i = i0 + lane;
    float p = 0.f, dsv = 0.f;
    if (i < T_) {
      p = expf(score(ks, q + (base + i) * ld + hoff, dh, scale) - max_in[sbase + i]) /
          sum_in[sbase + i];
      dsv = p * (dot_row(vs, d_o + (base + i) * ldo + hoff, dh) - dsum_in[sbase + i]);
    }
    ps[lane] = p;
    dss[lane] = dsv;
    __syncthreads();
    const int64_t in = T_ - i0 < 64 ? T_ - i0 : 64;
    for (int64_t ii = 0; ii < in; ++ii) {
      const float pw = ps[ii], dw = dss[ii];
      const T* qrow = q + (base + i0 + ii) * ld + hoff;
      const T* orow = d_o + (base + i0 + ii) * ldo + hoff;
#pragma unroll
      for (int r = 0; r < kMaxDhPerLane; ++r) {
        const int64_t c = lane + 64 * r;
        if (c < dh) {
          av[r] += pw * load_f32(orow + c);
          ak[r] += dw * load_f32(qrow + c);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int r = 0; r < kMaxDhPerLane; ++r) {
    const int64_t c = lane + 64 * r;
    if (c < dh) {
      store_f32(dk + (base + j) * ldd + hoff + c, ak[r] * scale);
      store_f32(dv + (base + j) * ldd + hoff + c, av[r]);
    }
  }
}

template <typename T>
hipError_t attention_backward_typed(const void* q, const void* k, const void* v, int64_t ld,
                                    const void* d_o, int64_t ldo, void* dq, void* dk, void* dv,
                                    int64_t ldd, int64_t N, int64_t T_, int64_t H, int64_t dh,
                                    float* stats, hipStream_t s) {
  if (dh > 64 * kMaxDhPerLane) return hipErrorInvalidValue;
  const int64_t rows = N * H * T_;
  if (rows > 2147483647LL) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf(static_cast<float>(dh));
  float* rmax = stats;
  float* rsum = stats + rows;
  float* dsum = stats + 2 * rows;
  const dim3 grid(static_cast<unsigned>(rows));
  hipLaunchKernelGGL(attn_bwd_query_kernel<T>, grid, dim3(64),
                     static_cast<size_t>(2 * dh + 64) * sizeof(float), s,
                     static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), ld, static_cast<const T*>(d_o), ldo,
                     static_cast<T*>(dq), ldd, T_, H, dh, scale, rmax, rsum, dsum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_key_kernel<T>, grid, dim3(64),
                     static_cast<size_t>(2 * dh + 128) * sizeof(float), s,
                     static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), ld, static_cast<const T*>(d_o), ldo,
                     static_cast<T*>(dk), static_cast<T*>(dv), ldd, T_, H, dh, scale,
                     static_cast<const float*>(rmax), static_cast<const float*>(rsum),
                     static_cast<const float*>(dsum));
  return hipGetLastError();
}

// Token rows [row0, row0 + rows) in `split` ranges into partial[0 .. split)
// (accumulate: added to what the partials hold).
template <typename T>
hipError_t wgrad_generic_rows(const WgradProblem& p, float* partial, int64_t row0, int64_t rows,
                              int split, bool accumulate, hipStream_t s) {
  const int64_t it = (p.I + 63) / 64, jt = (p.J + 63) / 64;
  const int64_t rows_per_split = (rows + split - 1) / split;
  const int64_t blocks = it * jt * split;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(wgrad_generic_kernel<T>, dim3(static_cast<unsigned>(blocks)),
                     dim3(kThreads), 0, s, p, partial, it, jt, row0, rows_per_split, accumulate);
  return hipGetLastError();
}

template <typename T>
hipError_t wgrad_reduce(const WgradProblem& p, const float* partial, int split, hipStream_t s) {
  const int64_t n = p.I * p.J;
  const bool vec = p.J % 4 == 0 && p.seg % 4 == 0 && p.ldc % 4 == 0;
  const int64_t work = vec ? n / 4 : n;
  const int64_t rb = (work + kThreads - 1) / kThreads < 8192 ? (work + kThreads - 1) / kThreads
                                                              : 8192;
  if (vec)
    hipLaunchKernelGGL(wgrad_reduce4_kernel<T>, dim3(static_cast<unsigned>(rb)), dim3(kThreads),
                       0, s, p, partial, split);
  else
    hipLaunchKernelGGL(wgrad_reduce_kernel<T>, dim3(static_cast<unsigned>(rb)), dim3(kThreads),
                       0, s, p, partial, split);
  return hipGetLastError();
}

// Matrix-core path for the bf16 bulk (a multiple of 64 token rows); the
// generic kernel takes everything else and the leftover rows, which it adds
// into the last range's partial.
template <typename T>
hipError_t wgrad_typed(const WgradProblem& p, float* partial, int split, hipStream_t s) {
  int used = 0;
  int64_t done = 0;
  if (sizeof(T) == 2) {
    const hipError_t e = launch_wgrad_mfma(p, partial, split, &used, s);
    if (e == hipSuccess)
      done = wgrad_mfma_rows(p, split);
    else if (e != hipErrorNotSupported)
      return e;
  }
  hipError_t e = hipSuccess;
  if (done == 0) {
    used = split;
    e = wgrad_generic_rows<T>(p, partial, 0, p.M, split, false, s);
  } else if (done < p.M) {
    e = wgrad_generic_rows<T>(p, partial + static_cast<int64_t>(used - 1) * p.I * p.J, done,
                              p.M - done, 1, true, s);
  }
  if (e != hipSuccess) return e;
  return wgrad_reduce<T>(p, partial, used, s);
}

}  // namespace

hipError_t launch_layernorm_backward_generic(const void* x, const void* g, const void* res,
                                             void* dx, int64_t rows, int64_t D, float eps,
                                             int dtype, hipStream_t s) {
  if (rows > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(rows));
  if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL(ln_backward_kernel<bf16_t>, grid, dim3(kThreads), 0, s,
                       static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(g),
                       static_cast<const bf16_t*>(res), static_cast<bf16_t*>(dx), D, eps);
  else
    hipLaunchKernelGGL(ln_backward_kernel<float>, grid, dim3(kThreads), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(g),
                       static_cast<const float*>(res), static_cast<float*>(dx), D, eps);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradProblem& p, float* partial, int split, hipStream_t s) {
  if (split < 1) return hipErrorInvalidValue;
  return p.dtype == VITBLK_BF16 ? wgrad_typed<bf16_t>(p, partial, split, s)
                                : wgrad_typed<float>(p, partial, split, s);
}

hipError_t launch_attention_backward(const void* q, const void* k, const void* v, int64_t ld,
                                     const void* d_o, int64_t ldo, void* dq, void* dk, void* dv,
                                     int64_t ldd, int64_t N, int64_t T, int64_t H, int64_t dh,
                                     int dtype, float* stats, hipStream_t s) {
  if (dtype == VITBLK_BF16) {
    const hipError_t e = launch_attention_backward_mfma(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd,
                                                        N, T, H, dh, stats, s);
    if (e != hipErrorNotSupported) return e;
  }
  return dtype == VITBLK_BF16
             ? attention_backward_typed<bf16_t>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H,
                                                dh, stats, s)
             : attention_backward_typed<float>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H,
                                               dh, stats, s);
}

}  // namespace vitblk
