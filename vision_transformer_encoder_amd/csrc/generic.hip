// Any-shape kernels for the block's steps, fp32 arithmetic on the VALU.
//
// They serve fp32 tensors (the fp32 tolerance rules out bf16 products) and
// bf16 shapes the MFMA kernels do not tile (D or F not a multiple of 64,
// odd head widths).  Simple, bounds-checked, not tuned.
#include <math.h>

#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kGenThreads = 256;

__device__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  const float t = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return t;
}

// LayerNorm of one row per workgroup: mean, then population variance of the
// deviations (two passes over the row), then (x - mean) / sqrt(var + eps).
template <typename T>
__global__ __launch_bounds__(kGenThreads) void ln_generic_kernel(
    const T* __restrict__ x, int64_t ld_in, const T* __restrict__ gamma,
    const T* __restrict__ beta, T* __restrict__ y, int64_t D, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ld_in;
  T* yr = y + row * D;
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kGenThreads) s += load_f32(xr + i);
  const float mean = block_sum_256(s, red) / static_cast<float>(D);
  float q = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kGenThreads) {
    const float d = load_f32(xr + i) - mean;
    q += d * d;
  }
  const float var = block_sum_256(q, red) / static_cast<float>(D);
  const float rstd = 1.0f / sqrtf(var + eps);
  for (int64_t i = threadIdx.x; i < D; i += kGenThreads) {
    float o = (load_f32(xr + i) - mean) * rstd;
    if (gamma != nullptr) o *= load_f32(gamma + i);
    if (beta != nullptr) o += load_f32(beta + i);
    store_f32(yr + i, o);
  }
}

// Statistics of one row per workgroup (as ln_generic_kernel): mean and
// 1 / sqrt(var + eps).
template <typename T>
__global__ __launch_bounds__(kGenThreads) void row_stats_generic_kernel(const T* __restrict__ x,
                                                                        int64_t ld_in,
                                                                        float* __restrict__ st,
                                                                        int64_t D, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const T* xr = x + row * ld_in;
  float s = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kGenThreads) s += load_f32(xr + i);
  const float mean = block_sum_256(s, red) / static_cast<float>(D);
  float q = 0.f;
  for (int64_t i = threadIdx.x; i < D; i += kGenThreads) {
    const float d = load_f32(xr + i) - mean;
    q += d * d;
  }
  const float var = block_sum_256(q, red) / static_cast<float>(D);
  if (threadIdx.x == 0) {
    st[2 * row] = mean;
    st[2 * row + 1] = 1.0f / sqrtf(var + eps);
  }
}

// 64x64 output tile per workgroup, 16-deep k slices staged in LDS, 4x4
// outputs per thread; tiles flattened into blockIdx.x.
template <typename T, int EPI>
__global__ __launch_bounds__(kGenThreads) void gemm_generic_kernel(GemmProblem p, int64_t nt) {
  __shared__ float As[16][64 + 4];
  __shared__ float Bs[16][64 + 4];
  const int64_t b = blockIdx.x;
  const int64_t m0 = (b / nt) * 64, n0 = (b % nt) * 64;
  const T* A = static_cast<const T*>(p.A);
  const T* B = static_cast<const T*>(p.B);
  T* C = static_cast<T*>(p.C);
  const T* R = static_cast<const T*>(p.R);
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int64_t k0 = 0; k0 < p.K; k0 += 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + i * kGenThreads;
      const int r = e >> 4, kk = e & 15;
      const int64_t gm = m0 + r, gk = k0 + kk;
      As[kk][r] = (gm < p.M && gk < p.K) ? load_f32(A + gm * p.lda + gk) : 0.f;
      const int64_t gn = n0 + r;
      Bs[kk][r] = (gn < p.N && gk < p.K) ? load_f32(B + gn * p.ldb + gk) : 0.f;
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
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= p.N) continue;
      float v = acc[i][j];
      if (p.row_stats != nullptr)  // LN(A) @ W = rstd (A @ W - mean colsum)
        v = p.row_stats[2 * m + 1] * (v - p.row_stats[2 * m] * p.col_sums[n]);
      if (has_bias(p)) {
        const int64_t seg = n / p.bias_seg;
        const void* bs = seg == 0 ? p.bias[0] : (seg == 1 ? p.bias[1] : p.bias[2]);
        if (bs != nullptr) v += load_f32(static_cast<const T*>(bs) + (n - seg * p.bias_seg));
      }
      if (EPI == VITBLK_EPI_RESIDUAL) v += load_f32(R + m * p.ldr + n);
      if (EPI == VITBLK_EPI_GELU_GRAD) v *= gelu_tanh_grad_precise(load_f32(R + m * p.ldr + n));
      if (EPI == kEpiMul) v *= load_f32(R + m * p.ldr + n);
      if (EPI == kEpiGeluDual) {
        store_f32(static_cast<T*>(p.C2) + m * p.ldc + n, gelu_tanh_grad_precise(v));
        v = gelu_tanh_precise(v);
      }
      if (EPI == VITBLK_EPI_GELU) v = gelu_tanh_precise(v);
      store_f32(C + m * p.ldc + n, v);
    }
  }
}

// One wave per (sequence, head, query): scores for 64 keys at a time (one
// key per lane), online softmax (running max and sum), and the weighted sum
// of value rows with each lane owning head features lane, lane+64, ...
constexpr int kMaxDhPerLane = 16;  // head width <= 1024

template <typename T>
__global__ __launch_bounds__(64) void attn_generic_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v, int64_t ld,
                                                          T* __restrict__ o, int64_t ldo,
                                                          int64_t T_, int64_t H, int64_t dh,
                                                          float scale) {
  extern __shared__ float sm[];
  float* qs = sm;       // [dh]
  float* ps = sm + dh;  // [64]
  int64_t b = blockIdx.x;
  const int64_t t = b % T_;
  b /= T_;
  const int64_t h = b % H;
  const int64_t n = b / H;
  const int lane = threadIdx.x;
  const int64_t base = n * T_;
  const T* qrow = q + (base + t) * ld + h * dh;
  for (int64_t c = lane; c < dh; c += 64) qs[c] = load_f32(qrow + c);
  __syncthreads();
  float m = -INFINITY, l = 0.f;
  float acc[kMaxDhPerLane];
#pragma unroll
  for (int r = 0; r < kMaxDhPerLane; ++r) acc[r] = 0.f;
  for (int64_t j0 = 0; j0 < T_; j0 += 64) {
    const int64_t j = j0 + lane;
    float s = -INFINITY;
    if (j < T_) {
      const T* krow = k + (base + j) * ld + h * dh;
      float d = 0.f;
      for (int64_t c = 0; c < dh; ++c) d += qs[c] * load_f32(krow + c);
      s = d * scale;
    }
    const float mnew = fmaxf(m, wave_max(s));
    const float alpha = expf(m - mnew);
    const float pj = (j < T_) ? expf(s - mnew) : 0.f;
    l = l * alpha + wave_sum(pj);
    m = mnew;
    ps[lane] = pj;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kMaxDhPerLane; ++r) acc[r] *= alpha;
    const int64_t jn = (T_ - j0 < 64) ? (T_ - j0) : 64;
    for (int64_t jj = 0; jj < jn; ++jj) {
      const float pw = ps[jj];
      const T* vrow = v + (base + j0 + jj) * ld + h * dh;
#pragma unroll
      for (int r = 0; r < kMaxDhPerLane; ++r) {
        const int64_t c = lane + 64 * r;
        if (c < dh) acc[r] += pw * load_f32(vrow + c);
      }
    }
    __syncthreads();
  }
  const float inv = 1.0f / l;
  T* orow = o + (base + t) * ldo + h * dh;
#pragma unroll
  for (int r = 0; r < kMaxDhPerLane; ++r) {
    const int64_t c = lane + 64 * r;
    if (c < dh) store_f32(orow + c, acc[r] * inv);
  }
}

template <typename T>
hipError_t gemm_generic_typed(const GemmProblem& p, hipStream_t s) {
  const int64_t mt = (p.M + 63) / 64, nt = (p.N + 63) / 64;
  const int64_t blocks = mt * nt;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks));
  switch (p.epi) {
    case VITBLK_EPI_RESIDUAL:
      hipLaunchKernelGGL((gemm_generic_kernel<T, VITBLK_EPI_RESIDUAL>), grid, dim3(kGenThreads),
                         0, s, p, nt);
      break;
    case VITBLK_EPI_GELU:
      hipLaunchKernelGGL((gemm_generic_kernel<T, VITBLK_EPI_GELU>), grid, dim3(kGenThreads), 0,
                         s, p, nt);
      break;
    case VITBLK_EPI_GELU_GRAD:
      hipLaunchKernelGGL((gemm_generic_kernel<T, VITBLK_EPI_GELU_GRAD>), grid, dim3(kGenThreads),
                         0, s, p, nt);
      break;
    case kEpiGeluDual:
      hipLaunchKernelGGL((gemm_generic_kernel<T, kEpiGeluDual>), grid, dim3(kGenThreads), 0, s,
                         p, nt);
      break;
    case kEpiMul:
      hipLaunchKernelGGL((gemm_generic_kernel<T, kEpiMul>), grid, dim3(kGenThreads), 0, s, p,
                         nt);
      break;
    default:
      hipLaunchKernelGGL((gemm_generic_kernel<T, VITBLK_EPI_NONE>), grid, dim3(kGenThreads), 0,
                         s, p, nt);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_layernorm_generic(const void* x, int64_t ld_in, const void* gamma,
                                    const void* beta, void* y, int64_t rows, int64_t D,
                                    float eps, int dtype, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(rows));
  if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL(ln_generic_kernel<bf16_t>, grid, dim3(kGenThreads), 0, s,
                       static_cast<const bf16_t*>(x), ld_in, static_cast<const bf16_t*>(gamma),
                       static_cast<const bf16_t*>(beta), static_cast<bf16_t*>(y), D, eps);
  else
    hipLaunchKernelGGL(ln_generic_kernel<float>, grid, dim3(kGenThreads), 0, s,
                       static_cast<const float*>(x), ld_in, static_cast<const float*>(gamma),
                       static_cast<const float*>(beta), static_cast<float*>(y), D, eps);
  return hipGetLastError();
}

hipError_t launch_row_stats_generic(const void* x, int64_t ld_in, float* stats, int64_t rows,
                                    int64_t D, float eps, int dtype, hipStream_t s) {
  if (rows > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(rows));
  if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL(row_stats_generic_kernel<bf16_t>, grid, dim3(kGenThreads), 0, s,
                       static_cast<const bf16_t*>(x), ld_in, stats, D, eps);
  else
    hipLaunchKernelGGL(row_stats_generic_kernel<float>, grid, dim3(kGenThreads), 0, s,
                       static_cast<const float*>(x), ld_in, stats, D, eps);
  return hipGetLastError();
}

hipError_t launch_gemm_generic(const GemmProblem& p, hipStream_t s) {
  if (reads_r(p) && p.R == nullptr) return hipErrorInvalidValue;
  if (p.epi == kEpiGeluDual && p.C2 == nullptr) return hipErrorInvalidValue;
  return p.dtype == VITBLK_BF16 ? gemm_generic_typed<bf16_t>(p, s)
                                : gemm_generic_typed<float>(p, s);
}

hipError_t launch_attention_generic(const void* q, const void* k, const void* v, int64_t ld,
                                    void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                    int64_t dh, int dtype, hipStream_t s) {
  if (dh > 64 * kMaxDhPerLane) return hipErrorInvalidValue;
  const int64_t blocks = N * H * T;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const float scale = 1.0f / sqrtf(static_cast<float>(dh));
  const size_t shmem = static_cast<size_t>(dh + 64) * sizeof(float);
  const dim3 grid(static_cast<unsigned>(blocks));
  if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL(attn_generic_kernel<bf16_t>, grid, dim3(64), shmem, s,
                       static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), ld, static_cast<bf16_t*>(o), ldo, T, H,
                       dh, scale);
  else
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(64), shmem, s,
                       static_cast<const float*>(q), static_cast<const float*>(k),
                       static_cast<const float*>(v), ld, static_cast<float*>(o), ldo, T, H, dh,
                       scale);
  return hipGetLastError();
}

}  // namespace vitblk
