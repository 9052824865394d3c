// Row-wise LayerNorm (crackedaicode.com "ViT Encoder Block", "Normalize
// before each stage"): per token, the mean and the population variance over
// its D features, then (x - mean) / sqrt(var + eps); optionally times a
// per-feature gain and plus a per-feature shift (ai-engineer-exhaustive.pages.dev
// "ViT Encoder Block", "Key Equations" step 1).
//
// One wave per row, four rows per 256-thread workgroup.  Each lane loads its
// share of the row as 16-byte vectors and keeps it in registers, so the row
// is read from HBM once and written once: the kernel is bound by HBM
// bandwidth (2 * D * element size bytes per row).  Statistics are fp32 and
// two-pass over the registers (mean, then the squared deviations), reduced
// across the wave with DPP row operations and lane reads.
//
// The statistics-only kernel serves the products that fold a LayerNorm
// without gain or shift into their epilogue (LN(x) @ W = rstd (x @ W -
// mean colsum W)): it reads the row and writes its mean and rstd, half the
// LayerNorm's traffic (D * element size + 8 bytes per row).
#include <math.h>

#include "device.h"
#include "kernels.h"
#include "row_stats.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kRowsPerBlock = 4;

// 8 floats -> 8 consecutive elements.
__device__ __forceinline__ void store8(bf16_t* p, const float v[8]) {
  st_global16(p, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
}
__device__ __forceinline__ void store8(float* p, const float v[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <typename T, int NCH>
__global__ __launch_bounds__(64 * kRowsPerBlock) void ln_rows_kernel(
    const T* __restrict__ x, int64_t ld_in, const T* __restrict__ gamma,
    const T* __restrict__ beta, T* __restrict__ y, int64_t rows, int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave leaves; no workgroup barrier follows
  const int nchunks = D >> 3;
  T* yr = y + row * D;
  float v[NCH][8];
  float mean, rstd;
  row_stats<T, NCH>(x + row * ld_in, lane, D, eps, v, &mean, &rstd);
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunks) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = (v[c][e] - mean) * rstd;
      if (gamma != nullptr) {  // uniform: the same for every lane
        float g[8];
        load8(gamma + idx * 8, g);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] *= g[e];
      }
      if (beta != nullptr) {
        float b[8];
        load8(beta + idx * 8, b);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += b[e];
      }
      store8(yr + idx * 8, o);
    }
  }
}

// Statistics only (for products that fold the LayerNorm into their
// epilogue): reads the row once and writes 8 bytes.  (Four rows per wave,
// all requested before any is reduced, measured no faster.)
template <typename T, int NCH>
__global__ __launch_bounds__(64 * kRowsPerBlock) void ln_stats_kernel(
    const T* __restrict__ x, int64_t ld_in, float2* __restrict__ stats, int64_t rows, int D,
    float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;
  stats_of_row<T, NCH>(x, ld_in, stats, row, D, eps, lane);
}

template <typename T>
hipError_t stats_fast_typed(const T* x, int64_t ld, float2* st, int64_t rows, int D, float eps,
                            hipStream_t s) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kRowsPerBlock);
  const int cpl = (D / 8 + 63) / 64;
  if (cpl <= 1)
    hipLaunchKernelGGL((ln_stats_kernel<T, 1>), grid, block, 0, s, x, ld, st, rows, D, eps);
  else if (cpl <= 2)
    hipLaunchKernelGGL((ln_stats_kernel<T, 2>), grid, block, 0, s, x, ld, st, rows, D, eps);
  else if (cpl <= 4)
    hipLaunchKernelGGL((ln_stats_kernel<T, 4>), grid, block, 0, s, x, ld, st, rows, D, eps);
  else
    hipLaunchKernelGGL((ln_stats_kernel<T, 8>), grid, block, 0, s, x, ld, st, rows, D, eps);
  return hipGetLastError();
}

template <typename T>
hipError_t ln_fast_typed(const T* x, int64_t ld, const T* g, const T* b, T* y, int64_t rows,
                         int D, float eps, hipStream_t s) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kRowsPerBlock);
  const int cpl = (D / 8 + 63) / 64;  // chunks per lane
  if (cpl <= 1)
    hipLaunchKernelGGL((ln_rows_kernel<T, 1>), grid, block, 0, s, x, ld, g, b, y, rows, D, eps);
  else if (cpl <= 2)
    hipLaunchKernelGGL((ln_rows_kernel<T, 2>), grid, block, 0, s, x, ld, g, b, y, rows, D, eps);
  else if (cpl <= 3)
    hipLaunchKernelGGL((ln_rows_kernel<T, 3>), grid, block, 0, s, x, ld, g, b, y, rows, D, eps);
  else if (cpl <= 4)
    hipLaunchKernelGGL((ln_rows_kernel<T, 4>), grid, block, 0, s, x, ld, g, b, y, rows, D, eps);
  else
    hipLaunchKernelGGL((ln_rows_kernel<T, 8>), grid, block, 0, s, x, ld, g, b, y, rows, D, eps);
  return hipGetLastError();
}

// Backward of the plain LayerNorm plus a residual gradient, one wave per
// row with the row of x and of g held in registers:
// dx = res + rstd * (g - mean(g) - xhat * mean(g * xhat)).  Reads x, g and
// res once and writes dx once (4 * D * element size bytes per row).
template <typename T, int NCH>
__global__ __launch_bounds__(64 * kRowsPerBlock) void ln_bwd_rows_kernel(
    const T* __restrict__ x, const T* __restrict__ g, const T* __restrict__ res,
    T* __restrict__ dx, int64_t rows, int D, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave leaves; no workgroup barrier follows
  const int nchunks = D >> 3;
  const T* xr = x + row * D;
  const T* gr = g + row * D;
  float v[NCH][8], gv[NCH][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunks) {
      load8(xr + idx * 8, v[c]);
      load8(gr + idx * 8, gv[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    }
  }
  const float inv_d = 1.0f / static_cast<float>(D);
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f, sg = 0.f, sgd = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (lane + 64 * c < nchunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[c][e] - mean;
        q += d * d;
        sg += gv[c][e];
        sgd += gv[c][e] * d;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(q) * inv_d + eps);
  const float mg = wave_sum(sg) * inv_d;
  const float mgx = wave_sum(sgd) * rstd * inv_d;  // mean(g * xhat)
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunks) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = rstd * (gv[c][e] - mg - (v[c][e] - mean) * rstd * mgx);
      if (res != nullptr) {
        float r[8];
        load8(res + row * D + idx * 8, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += r[e];
      }
      store8(dx + row * D + idx * 8, o);
    }
  }
}

template <typename T>
hipError_t ln_bwd_fast_typed(const T* x, const T* g, const T* r, T* dx, int64_t rows, int D,
                             float eps, hipStream_t s) {
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid(static_cast<unsigned>(blocks)), block(64 * kRowsPerBlock);
  const int cpl = (D / 8 + 63) / 64;
  if (cpl <= 1)
    hipLaunchKernelGGL((ln_bwd_rows_kernel<T, 1>), grid, block, 0, s, x, g, r, dx, rows, D, eps);
  else if (cpl <= 2)
    hipLaunchKernelGGL((ln_bwd_rows_kernel<T, 2>), grid, block, 0, s, x, g, r, dx, rows, D, eps);
  else if (cpl <= 4)
    hipLaunchKernelGGL((ln_bwd_rows_kernel<T, 4>), grid, block, 0, s, x, g, r, dx, rows, D, eps);
  else
    hipLaunchKernelGGL((ln_bwd_rows_kernel<T, 8>), grid, block, 0, s, x, g, r, dx, rows, D, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layernorm_backward(const void* x, const void* g, const void* res, void* dx,
                                     int64_t rows, int64_t D, float eps, int dtype,
                                     hipStream_t s) {
  const bool fast = (D % 8 == 0) && (D <= 64 * 8 * 8) &&
                    (rows + kRowsPerBlock - 1) / kRowsPerBlock <= 2147483647LL;
  if (!fast) return launch_layernorm_backward_generic(x, g, res, dx, rows, D, eps, dtype, s);
  if (dtype == VITBLK_BF16)
    return ln_bwd_fast_typed(static_cast<const bf16_t*>(x), static_cast<const bf16_t*>(g),
                             static_cast<const bf16_t*>(res), static_cast<bf16_t*>(dx), rows,
                             static_cast<int>(D), eps, s);
  return ln_bwd_fast_typed(static_cast<const float*>(x), static_cast<const float*>(g),
                           static_cast<const float*>(res), static_cast<float*>(dx), rows,
                           static_cast<int>(D), eps, s);
}

hipError_t launch_row_stats(const void* x, int64_t ld_in, float* stats, int64_t rows, int64_t D,
                            float eps, int dtype, hipStream_t s) {
  const bool fast = (D % 8 == 0) && (ld_in % 8 == 0) && (D <= 64 * 8 * 8) &&
                    (reinterpret_cast<uintptr_t>(x) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(stats) & 7u) == 0 &&
                    (rows + kRowsPerBlock - 1) / kRowsPerBlock <= 2147483647LL;
  if (!fast) return launch_row_stats_generic(x, ld_in, stats, rows, D, eps, dtype, s);
  float2* st = reinterpret_cast<float2*>(stats);
  if (dtype == VITBLK_BF16)
    return stats_fast_typed(static_cast<const bf16_t*>(x), ld_in, st, rows, static_cast<int>(D),
                            eps, s);
  return stats_fast_typed(static_cast<const float*>(x), ld_in, st, rows, static_cast<int>(D), eps,
                          s);
}

// A row's statistics from its per-strip partials (count, mean, M2), every
// strip kStatsStrip values: folded left to right with Chan et al.'s update
// (n_ab = n_a + n_b, mean_ab = mean_a + d n_b / n_ab, M2_ab = M2_a + M2_b +
// d^2 n_a n_b / n_ab, d = mean_b - mean_a), then rstd = 1 / sqrt(M2 / D + eps)
// (population variance, eps inside the root).  One thread per row.
__global__ __launch_bounds__(256) void stats_from_partials_kernel(
    const float2* __restrict__ P, int nstrips, float2* __restrict__ stats, int64_t rows,
    float eps) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const float2* pr = P + r * nstrips;
  const float nb = static_cast<float>(kStatsStrip);
  float2 a = pr[0];
  float n = nb, mean = a.x, m2 = a.y;
  for (int k = 1; k < nstrips; ++k) {
    const float2 b = pr[k];
    const float nn = n + nb;
    const float d = b.x - mean;
    mean += d * (nb / nn);
    m2 += b.y + d * d * (n * nb / nn);
    n = nn;
  }
  stats[r] = make_float2(mean, 1.0f / sqrtf(m2 / n + eps));
}

hipError_t launch_row_stats_from_partials(const float2* partials, int64_t nstrips, float* stats,
                                          int64_t rows, int64_t D, float eps, hipStream_t s) {
  if (nstrips < 1 || nstrips * kStatsStrip != D || rows < 1) return hipErrorInvalidValue;
  const int64_t blocks = (rows + 255) / 256;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(stats_from_partials_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256),
                     0, s, partials, static_cast<int>(nstrips), reinterpret_cast<float2*>(stats),
                     rows, eps);
  return hipGetLastError();
}

hipError_t launch_layernorm(const void* x, int64_t ld_in, const void* gamma, const void* beta,
                            void* y, int64_t rows, int64_t D, float eps, int dtype,
                            hipStream_t s) {
  // Register-resident rows: D and the row stride multiples of 8 (16-byte
  // vectors), at most 8 chunks of 8 per lane.
  const bool fast = (D % 8 == 0) && (ld_in % 8 == 0) && (D <= 64 * 8 * 8);
  if (!fast) return launch_layernorm_generic(x, ld_in, gamma, beta, y, rows, D, eps, dtype, s);
  if (dtype == VITBLK_BF16)
    return ln_fast_typed(static_cast<const bf16_t*>(x), ld_in, static_cast<const bf16_t*>(gamma),
                         static_cast<const bf16_t*>(beta), static_cast<bf16_t*>(y), rows,
                         static_cast<int>(D), eps, s);
  return ln_fast_typed(static_cast<const float*>(x), ld_in, static_cast<const float*>(gamma),
                       static_cast<const float*>(beta), static_cast<float*>(y), rows,
                       static_cast<int>(D), eps, s);
}

}  // namespace vitblk
