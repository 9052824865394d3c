// Any-shape kernels for the block's steps, fp32 arithmetic on the VALU.
//
// They serve fp32 tensors (the fp32 tolerance rules out bf16 products) and
// bf16 shapes the MFMA kernels do not tile (D or F not a multiple of 64,
// odd head widths).  Bounds-checked; only attention is tiled for speed.
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

// Tiled attention on the VALU, fp32 arithmetic (fp32 tensors; bf16 head widths
// the matrix-core kernels do not take).  One workgroup of 256 threads per
// (sequence, head, block of 256 / G queries); G threads per query, each
// holding DH / G features of the query (pre-scaled by log2(e) / sqrt(dh)) and
// of its output row.  Keys pass in chunks of kVKeys through two LDS stages
// (fp32), read as broadcasts (every thread of a pair group reads the same
// key row); each thread's share of the next chunk is requested before the
// work on the current one and written to the other stage after, one barrier
// per chunk.  Online softmax per query, key by key: a running maximum and
// sum, the sum and the accumulators rescaled when a key's score exceeds the
// maximum (exp2 of the pre-scaled scores); keys past T are not visited.
constexpr int kVKeys = 32;
constexpr int kVThreads = 256;

template <typename T, int DH, int G>
__global__ __launch_bounds__(kVThreads) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v, int64_t ld,
    T* __restrict__ o, int64_t ldo, int T_, int H, int qblocks, float scale_log2) {
  constexpr int DL = DH / G;                  // features per thread
  constexpr int QPB = kVThreads / G;          // queries per workgroup
  constexpr int PER = kVKeys * DH / kVThreads;  // chunk elements per thread and operand
  static_assert(DH % G == 0 && DL % 4 == 0 && (kVKeys * DH) % kVThreads == 0, "layout");
  static_assert(G == 1 || G == 2, "one or two threads per query");
  extern __shared__ __attribute__((aligned(16))) float kvs[];  // [2 stages][K | V][kVKeys][DH]
  constexpr int STAGE = 2 * kVKeys * DH;

  const int tid = threadIdx.x;
  int64_t b = blockIdx.x;
  const int qb = static_cast<int>(b % qblocks);
  b /= qblocks;
  const int h = static_cast<int>(b % H);
  const int64_t base = (b / H) * static_cast<int64_t>(T_);
  const int tq = qb * QPB + tid / G;  // this thread's query
  const int foff = (tid % G) * DL;    // its features
  const int tqc = tq < T_ ? tq : T_ - 1;

  float qr[DL], acc[DL];
  const T* qrow = q + (base + tqc) * ld + static_cast<int64_t>(h) * DH + foff;
#pragma unroll
  for (int c = 0; c < DL; ++c) {
    qr[c] = load_f32(qrow + c) * scale_log2;
    acc[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;

  float rk[PER], rv[PER];
  auto fetch = [&](int c0) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kVThreads;
      int key = c0 + e / DH;
      key = key < T_ ? key : T_ - 1;
      const int64_t g = (base + key) * ld + static_cast<int64_t>(h) * DH + e % DH;
      rk[i] = load_f32(k + g);
      rv[i] = load_f32(v + g);
    }
  };
  auto stash = [&](int st) {
    float* ks = kvs + st * STAGE;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kVThreads;
      ks[e] = rk[i];
      ks[kVKeys * DH + e] = rv[i];
    }
  };

  const int nchunks = (T_ + kVKeys - 1) / kVKeys;
  fetch(0);
  stash(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    if (c + 1 < nchunks) fetch((c + 1) * kVKeys);
    const float* ks = kvs + (c & 1) * STAGE;
    const float* vs = ks + kVKeys * DH;
    int nvalid = T_ - c * kVKeys;  // keys of this chunk below T (>= 1)
    nvalid = nvalid < kVKeys ? nvalid : kVKeys;
#pragma unroll 2
    for (int j = 0; j < nvalid; ++j) {
      const float4* kr = reinterpret_cast<const float4*>(ks + j * DH + foff);
      float d = 0.f;
#pragma unroll
      for (int c4 = 0; c4 < DL / 4; ++c4) {
        const float4 kk = kr[c4];
        d = fmaf(qr[4 * c4 + 0], kk.x, d);
        d = fmaf(qr[4 * c4 + 1], kk.y, d);
        d = fmaf(qr[4 * c4 + 2], kk.z, d);
        d = fmaf(qr[4 * c4 + 3], kk.w, d);
      }
      if (G == 2) d += __shfl_xor(d, 1);
      // A new maximum rescales the running sum and the accumulators (the
      // first key always does: m starts at -inf).
      if (d > m) {
        const float alpha = exp2f(m - d);
        l *= alpha;
#pragma unroll
        for (int c2 = 0; c2 < DL; ++c2) acc[c2] *= alpha;
        m = d;
      }
      const float p = exp2f(d - m);
      l += p;
      const float4* vr = reinterpret_cast<const float4*>(vs + j * DH + foff);
#pragma unroll
      for (int c4 = 0; c4 < DL / 4; ++c4) {
        const float4 vv = vr[c4];
        acc[4 * c4 + 0] = fmaf(p, vv.x, acc[4 * c4 + 0]);
        acc[4 * c4 + 1] = fmaf(p, vv.y, acc[4 * c4 + 1]);
        acc[4 * c4 + 2] = fmaf(p, vv.z, acc[4 * c4 + 2]);
        acc[4 * c4 + 3] = fmaf(p, vv.w, acc[4 * c4 + 3]);
      }
    }
    if (c + 1 < nchunks) stash((c + 1) & 1);
    __syncthreads();
  }
  if (tq < T_) {
    const float inv = 1.0f / l;
    T* orow = o + (base + tq) * ldo + static_cast<int64_t>(h) * DH + foff;
#pragma unroll
    for (int c = 0; c < DL; ++c) store_f32(orow + c, acc[c] * inv);
  }
}

template <typename E, int DH, int G>
hipError_t launch_attn_valu(const void* q, const void* k, const void* v, int64_t ld, void* o,
                            int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s) {
  constexpr int QPB = kVThreads / G;
  constexpr size_t bytes = 2 * 2 * kVKeys * DH * sizeof(float);
  const int64_t qblocks = (T + QPB - 1) / QPB;
  const int64_t blocks = N * H * qblocks;
  if (blocks > 2147483647LL || T > 2147483647LL || H > 2147483647LL) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL((attn_valu_kernel<E, DH, G>), dim3(static_cast<unsigned>(blocks)),
                     dim3(kVThreads), bytes, s, static_cast<const E*>(q),
                     static_cast<const E*>(k), static_cast<const E*>(v), ld, static_cast<E*>(o),
                     ldo, static_cast<int>(T), static_cast<int>(H), static_cast<int>(qblocks),
                     scale_log2);
  return hipGetLastError();
}

// The tiled VALU kernel for the head widths it is instantiated for (multiples
// of 8 up to 64 with one thread per query, 80, 96 and 128 with two);
// hipErrorNotSupported otherwise.
template <typename E>
hipError_t attn_valu_dh(const void* q, const void* k, const void* v, int64_t ld, void* o,
                        int64_t ldo, int64_t N, int64_t T, int64_t H, int64_t dh, hipStream_t s) {
  switch (dh) {
    case 8: return launch_attn_valu<E, 8, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 16: return launch_attn_valu<E, 16, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 24: return launch_attn_valu<E, 24, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 32: return launch_attn_valu<E, 32, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 40: return launch_attn_valu<E, 40, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 48: return launch_attn_valu<E, 48, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 56: return launch_attn_valu<E, 56, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 64: return launch_attn_valu<E, 64, 1>(q, k, v, ld, o, ldo, N, T, H, s);
    case 80: return launch_attn_valu<E, 80, 2>(q, k, v, ld, o, ldo, N, T, H, s);
    case 96: return launch_attn_valu<E, 96, 2>(q, k, v, ld, o, ldo, N, T, H, s);
    case 128: return launch_attn_valu<E, 128, 2>(q, k, v, ld, o, ldo, N, T, H, s);
    default: return hipErrorNotSupported;
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
  if (p.dtype == VITBLK_BF16) return gemm_generic_typed<bf16_t>(p, s);
  const hipError_t r = launch_gemm_f32_mfma(p, s);  // aligned fp32: the matrix cores
  return r != hipErrorNotSupported ? r : gemm_generic_typed<float>(p, s);
}

hipError_t launch_attention_generic(const void* q, const void* k, const void* v, int64_t ld,
                                    void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                    int64_t dh, int dtype, hipStream_t s) {
  // Tiled kernel where the head width has an instantiation; the one-query-per-
  // wave kernel below for every other width.
  const hipError_t r = dtype == VITBLK_BF16
                           ? attn_valu_dh<bf16_t>(q, k, v, ld, o, ldo, N, T, H, dh, s)
                           : attn_valu_dh<float>(q, k, v, ld, o, ldo, N, T, H, dh, s);
  if (r != hipErrorNotSupported) return r;
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
