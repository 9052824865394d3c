// A token row's LayerNorm statistics on one wave, for the LayerNorm kernels
// (crackedaicode.com "ViT Encoder Block", "Normalize before each stage": the
// token mean and the population variance over its D features, eps inside the
// square root).
#pragma once

#include <math.h>

#include "device.h"

namespace vitblk {

// 8 consecutive elements -> 8 floats (16-byte aligned).
__device__ __forceinline__ void load8(const bf16_t* p, float v[8]) {
  const uint4 u = ld_global16(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float v[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// The row held in registers: lane l loads chunks l, l + 64, ... of 8
// elements into v (NCH = upper bound on chunks per lane, D <= 512 * NCH, D a
// multiple of 8); mean and rstd = 1 / sqrt(var + eps) in fp32, two-pass
// (mean, then the squared deviations), reduced across the wave.
template <typename T, int NCH>
__device__ __forceinline__ void row_stats(const T* xr, int lane, int D, float eps,
                                          float (&v)[NCH][8], float* mean_out,
                                          float* rstd_out) {
  const int nchunks = D >> 3;
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int idx = lane + 64 * c;
    if (idx < nchunks) {
      load8(xr + idx * 8, v[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += v[c][e];
    }
  }
  const float inv_d = 1.0f / static_cast<float>(D);
  const float mean = wave_sum(s) * inv_d;
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    if (lane + 64 * c < nchunks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = v[c][e] - mean;
        q += d * d;
      }
    }
  }
  const float var = wave_sum(q) * inv_d;
  *mean_out = mean;
  *rstd_out = 1.0f / sqrtf(var + eps);
}

// stats[row] = (mean, rstd) of row `row` of x (row stride ld elements).
template <typename T, int NCH>
__device__ __forceinline__ void stats_of_row(const T* x, int64_t ld, float2* stats, int64_t row,
                                             int D, float eps, int lane) {
  float v[NCH][8];
  float mean, rstd;
  row_stats<T, NCH>(x + row * ld, lane, D, eps, v, &mean, &rstd);
  if (lane == 0) stats[row] = make_float2(mean, rstd);
}

}  // namespace vitblk
