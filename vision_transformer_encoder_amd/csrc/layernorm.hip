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
__device__ __forceinline__ void combine_partials(const float2* __restrict__ P, int nstrips,
                                                 float2* __restrict__ stats, int64_t r,
                                                 float eps) {
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

__global__ __launch_bounds__(256) void stats_from_partials_kernel(
    const float2* __restrict__ P, int nstrips, float2* __restrict__ stats, int64_t rows,
    float eps) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (r < rows) combine_partials(P, nstrips, stats, r, eps);
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


// ------------------------------------------------------------- affine fold

// The affine LayerNorm folded into the product after it (bf16).  With
// xn = gamma * LN(x) + beta (ai-engineer-exhaustive.pages.dev "ViT Encoder
// Block", "Key Equations", steps 1 and 4) and LN(x) = rstd (x - mean):
//   xn @ W + b = rstd (x @ W' - mean colsum(W')) + b',
//   W' = diag(gamma) W,  b' = b + beta @ W,
// so the product runs on x itself with the LayerNorm fold's row statistics.
// One wave per output column n (a row of the out-major W^T), four per
// workgroup: the lane's 8-element runs of the row scaled and rounded to bf16
// (W'), their fp32 sum (colsum(W') of the rounded values, as the product
// uses them) and the fp32 sum of beta_k W[k, n], then the wave sums and
// b'_n = bf16(b_n + sum).  Reads W^T once and writes W'^T once.  The launch
// is short and latency-bound, so the row statistics the product also needs
// (of x, or combined from row partials) ride in it as a second role.
namespace {

// One 8-element run of W^T row n at column k (wv, with the gains gv and
// shifts bv of those columns): W' stored, sums accumulated.
__device__ __forceinline__ void fold_run(const uint4& wv, const uint4& gv, const uint4& bv,
                                         int64_t k, bf16_t* ws, float& cs, float& bb) {
  const uint32_t wu[4] = {wv.x, wv.y, wv.z, wv.w};
  const uint32_t gu[4] = {gv.x, gv.y, gv.z, gv.w};
  const uint32_t bu[4] = {bv.x, bv.y, bv.z, bv.w};
  uint32_t out[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float w0 = __uint_as_float(wu[e] << 16), w1 = __uint_as_float(wu[e] & 0xffff0000u);
    const float g0 = __uint_as_float(gu[e] << 16), g1 = __uint_as_float(gu[e] & 0xffff0000u);
    const float b0 = __uint_as_float(bu[e] << 16), b1 = __uint_as_float(bu[e] & 0xffff0000u);
    out[e] = pack_bf16x2(g0 * w0, g1 * w1);
    cs += __uint_as_float(out[e] << 16);
    cs += __uint_as_float(out[e] & 0xffff0000u);
    bb = fmaf(b0, w0, bb);
    bb = fmaf(b1, w1, bb);
  }
  st_global16(ws + k, make_uint4(out[0], out[1], out[2], out[3]));
}

constexpr uint32_t kOnes = 0x3f803f80u;  // two bf16 1.0
__device__ __forceinline__ uint4 load_or(const bf16_t* p, int64_t k, uint32_t fill) {
  return p != nullptr ? ld_global16(p + k) : make_uint4(fill, fill, fill, fill);
}

// Rows up to 2048 wide: all of the lane's (at most four) runs, with their
// gains and shifts, are requested before any is used.
constexpr int kFoldRuns = 4;

__device__ __forceinline__ void fold_row(const AffineFoldJob& j, int64_t n, int lane) {
  const bf16_t* w = static_cast<const bf16_t*>(j.w_t) + n * j.K;
  bf16_t* ws = static_cast<bf16_t*>(j.w_scaled) + n * j.K;
  const bf16_t* g = static_cast<const bf16_t*>(j.gamma);
  const bf16_t* be = static_cast<const bf16_t*>(j.beta);
  // b_n, requested with the runs (used by lane 0 at the end).
  const int seg = static_cast<int>(n >= j.bias_seg) + static_cast<int>(n >= 2 * j.bias_seg);
  const bf16_t* bs = static_cast<const bf16_t*>(j.bias[seg]);
  const float b = bs != nullptr && lane == 0 ? bf16_to_f32(bs[n - seg * j.bias_seg]) : 0.f;
  float cs = 0.f, bb = 0.f;
  if (j.K <= kFoldRuns * 64 * 8) {
    uint4 wv[kFoldRuns], gv[kFoldRuns], bv[kFoldRuns];
#pragma unroll
    for (int r = 0; r < kFoldRuns; ++r) {
      const int64_t k = (r * 64 + lane) * 8;
      const bool in = k < j.K;
      wv[r] = in ? ld_global16(w + k) : make_uint4(0u, 0u, 0u, 0u);
      gv[r] = in ? load_or(g, k, kOnes) : make_uint4(0u, 0u, 0u, 0u);
      bv[r] = in ? load_or(be, k, 0u) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int r = 0; r < kFoldRuns; ++r) {
      const int64_t k = (r * 64 + lane) * 8;
      if (k < j.K) fold_run(wv[r], gv[r], bv[r], k, ws, cs, bb);
    }
  } else {
    for (int64_t k = lane * 8; k < j.K; k += 64 * 8)
      fold_run(ld_global16(w + k), load_or(g, k, kOnes), load_or(be, k, 0u), k, ws, cs, bb);
  }
  cs = wave_sum(cs);
  bb = wave_sum(bb);
  if (lane == 0) {
    j.col_sums[n] = cs;
    static_cast<bf16_t*>(j.bias_out)[n] = f32_to_bf16(b + bb);
  }
}

// The launch's second role: 0 none, 1 the row statistics of x (a wave per
// row, as ln_stats_kernel), 2 row statistics combined from row partials (a
// thread per row, as stats_from_partials_kernel).
struct FoldSideArgs {
  int kind;
  const bf16_t* x;
  int64_t ld;
  const float2* partials;
  int nstrips;
  float2* stats;
  int64_t rows;
  int D;
  float eps;
};

template <int NCH>
__global__ __launch_bounds__(256) void affine_fold_kernel(AffineFoldJob j, int64_t fold_blocks,
                                                          FoldSideArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t b = blockIdx.x;
  if (b < fold_blocks) {
    const int64_t n = b * 4 + wave;
    if (n < j.N) fold_row(j, n, lane);
    return;
  }
  const int64_t sb = b - fold_blocks;
  if (a.kind == 1) {
    const int64_t row = sb * 4 + wave;
    if (row < a.rows) stats_of_row<bf16_t, NCH>(a.x, a.ld, a.stats, row, a.D, a.eps, lane);
  } else if (a.kind == 2) {
    const int64_t r = sb * 256 + threadIdx.x;
    if (r < a.rows) combine_partials(a.partials, a.nstrips, a.stats, r, a.eps);
  }
}

}  // namespace

hipError_t launch_affine_fold(const AffineFoldJob& j, const FoldSide* side, hipStream_t s) {
  const auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  if (j.N <= 0 || j.K <= 0 || j.K % 8 != 0 || j.bias_seg <= 0 || j.N > 3 * j.bias_seg ||
      j.w_t == nullptr || j.w_scaled == nullptr || j.col_sums == nullptr ||
      j.bias_out == nullptr || !a16(j.w_t) || !a16(j.w_scaled) || !a16(j.gamma) ||
      !a16(j.beta))
    return hipErrorInvalidValue;
  const int64_t fold_blocks = (j.N + 3) / 4;
  FoldSideArgs a{};
  int64_t side_blocks = 0;
  int cpl = 1;
  if (side != nullptr && side->rows > 0) {
    if ((reinterpret_cast<uintptr_t>(side->stats) & 7u) != 0 || side->D < 1)
      return hipErrorNotSupported;
    a.stats = reinterpret_cast<float2*>(side->stats);
    a.rows = side->rows;
    a.D = static_cast<int>(side->D);
    a.eps = side->eps;
    if (side->partials != nullptr) {
      if (side->nstrips < 1 || side->nstrips * kStatsStrip != side->D) return hipErrorNotSupported;
      a.kind = 2;
      a.partials = side->partials;
      a.nstrips = static_cast<int>(side->nstrips);
      side_blocks = (side->rows + 255) / 256;
    } else {
      if (side->D % 8 != 0 || side->ld % 8 != 0 || side->D > 64 * 8 * 8 || !a16(side->x))
        return hipErrorNotSupported;
      a.kind = 1;
      a.x = static_cast<const bf16_t*>(side->x);
      a.ld = side->ld;
      side_blocks = (side->rows + 3) / 4;
      cpl = static_cast<int>((side->D / 8 + 63) / 64);
    }
  }
  const int64_t blocks = fold_blocks + side_blocks;
  if (blocks > 2147483647LL) return side != nullptr ? hipErrorNotSupported : hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  if (cpl <= 1)
    hipLaunchKernelGGL(affine_fold_kernel<1>, grid, block, 0, s, j, fold_blocks, a);
  else if (cpl <= 2)
    hipLaunchKernelGGL(affine_fold_kernel<2>, grid, block, 0, s, j, fold_blocks, a);
  else if (cpl <= 4)
    hipLaunchKernelGGL(affine_fold_kernel<4>, grid, block, 0, s, j, fold_blocks, a);
  else
    hipLaunchKernelGGL(affine_fold_kernel<8>, grid, block, 0, s, j, fold_blocks, a);
  return hipGetLastError();
}

}  // namespace vitblk
