// Device-side helpers shared by the vitblk kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vitblk {

typedef uint16_t bf16_t;  // bfloat16 bit pattern as stored in memory

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------- conversions

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bfloat16.  gfx950 converts in hardware
// (v_cvt_pk_bf16_f32, IEEE round-to-nearest-even; NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats -> two packed bf16 in one dword (low half = a).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}

// Element load/store of the storage type T (float or bf16_t) as float.
template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(*p);
}
template <typename T> __device__ __forceinline__ void store_f32(T* p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, float v) {
  *p = f32_to_bf16(v);
}

// ------------------------------------------------------------- math

// GELU, tanh form: 0.5 z (1 + tanh(u)) with u = sqrt(2/pi) (z + 0.044715 z^3).
// Uses 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u)), evaluated with the hardware
// base-2 exponential; exact limits z -> +inf (z) and z -> -inf (-0).  The
// exponent -2 log2(e) u = z (c0 + c1 z^2) with the constants folded in double
// precision: five VALU operations and two transcendentals per element.
__device__ __forceinline__ float gelu_tanh_fast(float z) {
  constexpr double kU0 = 0.7978845608028654;         // sqrt(2/pi)
  constexpr double kM2Log2e = -2.8853900817779268;   // -2 * log2(e)
  constexpr float c0 = static_cast<float>(kM2Log2e * kU0);
  constexpr float c1 = static_cast<float>(kM2Log2e * kU0 * 0.044715);
  const float t = __builtin_fmaf(z * z, c1, c0);
  const float e = __builtin_amdgcn_exp2f(z * t);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Same function through the library tanh, for the fp32 path.
__device__ __forceinline__ float gelu_tanh_precise(float z) {
  const float k0 = 0.7978845608028654f;
  return 0.5f * z * (1.0f + tanhf(k0 * (z + 0.044715f * z * z * z)));
}

// Derivative of the tanh-form GELU: with s = 0.5 (1 + tanh(u)) = 1 / (1 + exp(-2u))
// and 1 - tanh(u)^2 = 4 s (1 - s),  d/dz GELU = s + 2 z s (1 - s) u'(z),
// u'(z) = sqrt(2/pi) (1 + 3 * 0.044715 z^2).  z is clamped inside u'(z) only,
// where s (1 - s) is already exactly 0 (|z| > 100), so that z^2 cannot overflow.
__device__ __forceinline__ float gelu_tanh_grad_fast(float z) {
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  const float m2log2e = -2.8853900817779268f;
  const float zc = fminf(fmaxf(z, -100.0f), 100.0f);
  const float u = k0 * (zc + k1 * zc * zc * zc);
  const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(m2log2e * u));
  const float du = k0 * (1.0f + 3.0f * k1 * zc * zc);
  return s + 2.0f * zc * s * (1.0f - s) * du;
}

// Same derivative through the library tanh, for the fp32 path:
// 0.5 (1 + t) + 0.5 z (1 - t^2) u'(z), t = tanh(u).
__device__ __forceinline__ float gelu_tanh_grad_precise(float z) {
  const float k0 = 0.7978845608028654f;
  const float k1 = 0.044715f;
  const float zc = fminf(fmaxf(z, -100.0f), 100.0f);
  const float t = tanhf(k0 * (zc + k1 * zc * zc * zc));
  const float du = k0 * (1.0f + 3.0f * k1 * zc * zc);
  return 0.5f * (1.0f + t) + 0.5f * zc * (1.0f - t * t) * du;
}

// ------------------------------------------------------------- wave reductions

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over all 64 lanes of the wave; every lane receives the total.
// Inside each 16-lane row: two quad permutes and two row rotations (DPP);
// across the four rows: read one lane of each row.
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x124>(v);  // row_ror:4
  v += dpp_mov<0x128>(v);  // row_ror:8
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x124>(v));
  v = fmaxf(v, dpp_mov<0x128>(v));
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// ------------------------------------------------------------- 16-byte memory ops

__device__ __forceinline__ uint4 ld_global16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st_global16(void* p, uint4 v) {
  *reinterpret_cast<uint4*>(p) = v;
}

// 8x8 transpose of 16-bit elements held as 8 rows of 8 (one uint4 per row):
// out[j] holds element j of every input row, row 0 in the lowest half-word.
__device__ __forceinline__ void transpose8x8_b16(const uint4 in[8], uint4 out[8]) {
  const uint32_t* w[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) w[r] = reinterpret_cast<const uint32_t*>(&in[r]);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // element c of row r lives in dword c/2 of row r, half (c & 1)
    uint32_t o[4];
#pragma unroll
    for (int rp = 0; rp < 4; ++rp) {
      const uint32_t a = w[2 * rp][c >> 1];
      const uint32_t b = w[2 * rp + 1][c >> 1];
      o[rp] = (c & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
    out[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ------------------------------------------------------------- row blocks <-> whole lines
//
// A 32-row x 64-column bf16 block held as v[2j + q], lane l: row l & 31,
// columns j*32 + q*16 + (l >> 5)*8 .. +7 (16 bytes) -- the layout of a
// 32x32x16 MFMA accumulator pair after one v_permlane32_swap, and of eight
// consecutive 16-wide k-steps of an MFMA operand.  A memory instruction in that
// layout touches 32 rows x 32 bytes, a quarter of each row's 128-byte line.
// rows_to_lines turns it into v[t]: rows 8t .. 8t+7, lane L row 8t + (L >> 3),
// columns (L & 7)*8 .. +7, so each group of 8 lanes covers one row's 64
// columns, one full line; lines_to_rows is the inverse.
// The register index bits (j, q) trade places with the lane bits 4 and 3
// (v_permlane16_swap swaps 16-lane rows; a row_ror:8 DPP read plus a select
// swaps lanes l and l ^ 8), then one ds_bpermute per dword moves lane
// (h, j, q, r2 r1 r0) to lane (r2 r1 r0, j, q, h).
__device__ __forceinline__ void rows_to_lines(uint4 v[4], int lane) {
  uint32_t w[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    w[s][0] = v[s].x;
    w[s][1] = v[s].y;
    w[s][2] = v[s].z;
    w[s][3] = v[s].w;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto r = __builtin_amdgcn_permlane16_swap(w[q][d], w[2 + q][d], false, false);
      w[q][d] = r[0];
      w[2 + q][d] = r[1];
    }
  const bool hi8 = (lane >> 3) & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = w[2 * a][d], y = w[2 * a + 1][d];
      const uint32_t xr = __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xf, 0xf, false);
      const uint32_t yr = __builtin_amdgcn_update_dpp(0u, y, 0x128, 0xf, 0xf, false);
      w[2 * a][d] = hi8 ? yr : x;
      w[2 * a + 1][d] = hi8 ? y : xr;
    }
  const int src = ((((lane & 1) << 5) | (((lane >> 2) & 1) << 4) | (((lane >> 1) & 1) << 3) |
                    (lane >> 3)) << 2);
#pragma unroll
  for (int t = 0; t < 4; ++t)
    v[t] = make_uint4(__builtin_amdgcn_ds_bpermute(src, w[t][0]),
                      __builtin_amdgcn_ds_bpermute(src, w[t][1]),
                      __builtin_amdgcn_ds_bpermute(src, w[t][2]),
                      __builtin_amdgcn_ds_bpermute(src, w[t][3]));
}

// Inverse of rows_to_lines (the two exchange steps are involutions; the lane
// permutation is undone by the inverse ds_bpermute).
__device__ __forceinline__ void lines_to_rows(uint4 v[4], int lane) {
  uint32_t w[4][4];
  const int src = ((((lane & 7) << 3) | (((lane >> 4) & 1) << 2) | (((lane >> 3) & 1) << 1) |
                    (lane >> 5)) << 2);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    w[s][0] = __builtin_amdgcn_ds_bpermute(src, v[s].x);
    w[s][1] = __builtin_amdgcn_ds_bpermute(src, v[s].y);
    w[s][2] = __builtin_amdgcn_ds_bpermute(src, v[s].z);
    w[s][3] = __builtin_amdgcn_ds_bpermute(src, v[s].w);
  }
  const bool hi8 = (lane >> 3) & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t x = w[2 * a][d], y = w[2 * a + 1][d];
      const uint32_t xr = __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xf, 0xf, false);
      const uint32_t yr = __builtin_amdgcn_update_dpp(0u, y, 0x128, 0xf, 0xf, false);
      w[2 * a][d] = hi8 ? yr : x;
      w[2 * a + 1][d] = hi8 ? y : xr;
    }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const auto r = __builtin_amdgcn_permlane16_swap(w[q][d], w[2 + q][d], false, false);
      w[q][d] = r[0];
      w[2 + q][d] = r[1];
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) v[s] = make_uint4(w[s][0], w[s][1], w[s][2], w[s][3]);
}

}  // namespace vitblk
