// Attention backward on the gfx950 matrix cores, one (sequence, head) per
// workgroup with that head's operands resident in LDS (sequences up to a few
// hundred tokens: ViT's 197 and 257).
//
// Per sequence and head (the derivative of softmax(Q K^T / sqrt(dh)) V,
// crackedaicode.com "ViT Encoder Block", "Multi-head attention"; gradients
// as training needs them, nipunbatra.github.io vision1 transcript, Pages 88
// and 113), with c = log2(e) / sqrt(dh), t = S * c, P = 2^(t - m) / l:
//   dP = dO V^T,  Dsum_i = sum_j P_ij dP_ij,  dS = P * (dP - Dsum)
//   dQ = dS K / sqrt(dh),  dK = dS^T Q / sqrt(dh),  dV = P^T dO.
//
// Two kernels:
// * query-major (dq): each wave takes 32-query tiles with K and V in LDS.
//   Pass 1 walks the keys once with S^T = K Q^T and dP^T = V dO^T, keeping
//   the running maximum m, the sum l = sum 2^(t - m) and sum 2^(t - m) dP
//   (both rescaled when m moves), which gives Dsum = (that sum) / l with no
//   second look at the keys.  Pass 2 recomputes S^T and dP^T, forms dS^T
//   and accumulates dQ^T += K^T dS^T.  m, 1/l and Dsum go to a small buffer.
// * key-major (dkv): each wave takes 32-key tiles with Q, dO and the
//   statistics in LDS; per 32-query block S = Q K^T, dP = dO V^T, then
//   dV^T += dO^T P and dK^T += Q^T dS.
// Both use v_mfma_f32_32x32x16_bf16.  In an accumulator block, lane l holds
// column l % 32 and rows 8a + 4(l/32) + i (a, i = 0..3): the probabilities
// and dS of one key (dkv) or query (dq) over 16 rows, which are exactly the
// second MFMA operand of the dV/dK (or dQ) products, 8 rows per k-step.  The
// first operand of those products is a transposed read (ds_read_b64_tr_b16)
// of the same rows of Q / dO (or K).
//
// Row order inside a 32-row block: the A-operand of S (resp. S^T) takes row
// perm32(x) for lane row x, so accumulator row x is block row perm32(x).
// perm32 puts the 4 rows of each transposed read 4 apart and keeps the 16
// rows of each 16-byte read distinct modulo 16; with an LDS row stride of
// dh*2 + 16 bytes (an odd multiple of 16) both kinds of read are then free
// of bank conflicts on gfx950's 64 banks.
//
// Scaled scores t = S * c are rounded on their own (never fused into the
// following subtraction), so every pass and both kernels see the same t and
// a one-key row gets P = 1 exactly.
#include <math.h>

#include <atomic>

#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kLds = 160 * 1024;

typedef short v4i16 __attribute__((ext_vector_type(4)));

template <int DH>
struct BwdCfg {
  static_assert(DH % 16 == 0, "head width must be a multiple of 16");
  static constexpr int DHP = (DH + 31) / 32 * 32;  // rows of the transposed accumulators
  static constexpr int SR = DH * 2 + 16;           // LDS row stride in bytes (odd multiple of 16)
  static_assert((SR / 16) % 2 == 1, "row stride must be an odd multiple of 16 bytes");
};

// Block row of accumulator row x = 8a + 4g + i.
__device__ __forceinline__ int perm32(int x) {
  const int a = x >> 3, g = (x >> 2) & 1, i = x & 3;
  return i * 4 + (a & 1) * 2 + g + (a >> 1) * 16;
}

__device__ __forceinline__ uint2 with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return make_uint2(r[0], r[1]);
}
__device__ __forceinline__ float max_halves(float x) {
  const uint2 r = with_other_half(x);
  return fmaxf(__uint_as_float(r.x), __uint_as_float(r.y));
}
__device__ __forceinline__ float sum_halves(float x) {
  const uint2 r = with_other_half(x);
  return __uint_as_float(r.x) + __uint_as_float(r.y);
}

__device__ __forceinline__ v4i16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<char*>(p)));
}

// t = s * c as its own rounded product.
__device__ __forceinline__ float scaled(float s, float c) {
#pragma clang fp contract(off)
  return s * c;
}

// Copy rows [0, T_pad) of a head's [T, DH] slice (row stride ld elements)
// into LDS with row stride SR; rows past T repeat row T - 1 (finite values).
template <int DH>
__device__ __forceinline__ void stage_rows(const bf16_t* __restrict__ src, int64_t ld, int T,
                                           int T_pad, char* dst) {
  using C = BwdCfg<DH>;
  constexpr int CPR = DH / 8;
  const int chunks = T_pad * CPR;
  for (int c0 = threadIdx.x; c0 < chunks; c0 += 4 * blockDim.x) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * blockDim.x;
      if (c < chunks) {
        const int r = c / CPR, t = r < T ? r : T - 1;
        v[u] = ld_global16(src + static_cast<int64_t>(t) * ld + (c % CPR) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * blockDim.x;
      if (c < chunks) *reinterpret_cast<uint4*>(dst + (c / CPR) * C::SR + (c % CPR) * 16) = v[u];
    }
  }
}

// Fragments of one row of a [T, DH] slice for the MFMA's second operand:
// lane (lrow, g) gets features 16s + 8g .. +7 of `row`, s = 0 .. DH/16 - 1.
template <int DH>
__device__ __forceinline__ void row_frags(const bf16_t* __restrict__ row, int g, bf16x8* f) {
#pragma unroll
  for (int s = 0; s < DH / 16; ++s)
    f[s] = __builtin_bit_cast(bf16x8, ld_global16(row + g * 8 + s * 16));
}

// 32x32 block of X Y^T over DH: first operand rows of X from LDS (block row
// perm32(lrow) of the 32 rows at x0), second operand the register fragments yf.
template <int DH>
__device__ __forceinline__ f32x16 block_xyT(const char* xs, int x0, int lrow, int g,
                                            const bf16x8* yf) {
  using C = BwdCfg<DH>;
  const char* xr = xs + (x0 + perm32(lrow)) * C::SR + g * 16;
  f32x16 acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(xr),
                                                       yf[0], f32x16{}, 0, 0, 0);
#pragma unroll
  for (int s = 1; s < DH / 16; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(xr + s * 32),
                                                  yf[s], acc, 0, 0, 0);
  return acc;
}

// acc[d] += X^T W over the 32 rows at x0, W given as the packed accumulator
// rows of a block (pk[e] holds rows 2e, 2e+1 of the lane's column): for each
// 16-row step s2, the first operand is the transposed read of block rows
// perm32(8*(2 s2 + h) + 4g + i), i = 0..3 (h = 0: lo, 1: hi), which are
// s2*16 + g + 2h + 4i.
template <int DH>
__device__ __forceinline__ void acc_xT(const char* xs, int x0, int lane, const uint32_t* pk,
                                       f32x16* acc) {
  using C = BwdCfg<DH>;
  const int g = lane >> 5, q16 = (lane >> 4) & 1, i16 = lane & 15;
  const int lane_off = (4 * (i16 >> 2)) * C::SR + (q16 * 16 + 4 * (i16 & 3)) * 2;
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2) {
    const bf16x8 wf = __builtin_bit_cast(
        bf16x8, make_uint4(pk[s2 * 4 + 0], pk[s2 * 4 + 1], pk[s2 * 4 + 2], pk[s2 * 4 + 3]));
    const char* xb = xs + (x0 + s2 * 16 + g) * C::SR + lane_off;
#pragma unroll
    for (int d = 0; d < C::DHP / 32; ++d) {
      const v4i16 lo = ds_read_tr16(xb + d * 64);
      const v4i16 hi = ds_read_tr16(xb + 2 * C::SR + d * 64);
      const bf16x8 xf = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xf, wf, acc[d], 0, 0, 0);
    }
  }
}

// Store the transposed accumulators (rows: features, column: the lane's
// token) scaled by `mul`: lane (lrow, g) writes features d*32 + 8a + 4g + 0..3.
template <int DH>
__device__ __forceinline__ void store_rowT(bf16_t* __restrict__ row, int g, const f32x16* acc,
                                           float mul) {
  using C = BwdCfg<DH>;
#pragma unroll
  for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int f = d * 32 + a * 8 + g * 4;
      if (f < DH)
        *reinterpret_cast<uint2*>(row + f) =
            make_uint2(pack_bf16x2(acc[d][a * 4 + 0] * mul, acc[d][a * 4 + 1] * mul),
                       pack_bf16x2(acc[d][a * 4 + 2] * mul, acc[d][a * 4 + 3] * mul));
    }
}

// ------------------------------------------------------------- query-major
template <int DH>
__global__ __launch_bounds__(64 * kMaxWaves, 2) void attn_bwd_dq_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int64_t ld, const bf16_t* __restrict__ dO, int64_t ldo, bf16_t* __restrict__ dQ,
    int64_t ldd, float* __restrict__ stats, int64_t R, int T, int H, int T_pad, float c,
    float scale) {
  using C = BwdCfg<DH>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const ks = smem;
  char* const vs = smem + T_pad * C::SR;

  const int h = static_cast<int>(blockIdx.x % H);
  const int64_t n = blockIdx.x / H;
  const int64_t seq0 = n * T, hoff = static_cast<int64_t>(h) * DH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int lrow = lane & 31, g = lane >> 5;
  const int nqt = T_pad / 32;

  stage_rows<DH>(K + seq0 * ld + hoff, ld, T, T_pad, ks);
  stage_rows<DH>(V + seq0 * ld + hoff, ld, T, T_pad, vs);
  __syncthreads();

  for (int qt = wave; qt < nqt; qt += nw) {
    const int q = qt * 32 + lrow, qc = q < T ? q : T - 1;
    bf16x8 qf[DH / 16], of[DH / 16];
    row_frags<DH>(Q + (seq0 + qc) * ld + hoff, g, qf);
    row_frags<DH>(dO + (seq0 + qc) * ldo + hoff, g, of);

    // Accumulator row x of a 32-key block is key k0 + kb*32 + perm32(x);
    // lane (lrow, g), element r: x = 8 (r/4) + 4g + r%4.
    auto key_of = [&](int r) { return perm32(8 * (r >> 2) + 4 * g + (r & 3)); };

    // Pass 1: running max m (of t), l = sum 2^(t - m), u = sum 2^(t - m) dP.
    float m = -INFINITY, l = 0.f, u = 0.f;
    for (int k0 = 0; k0 < T; k0 += 32) {
      const f32x16 st = block_xyT<DH>(ks, k0, lrow, g, qf);
      const f32x16 dp = block_xyT<DH>(vs, k0, lrow, g, of);
      const bool tail = T - k0 < 32;
      float t[16];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        t[r] = (tail && key_of(r) >= T - k0) ? -INFINITY : scaled(st[r], c);
        mx = fmaxf(mx, t[r]);
      }
      mx = max_halves(mx);
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // m = -inf: 0
      l *= alpha;
      u *= alpha;
      m = m_new;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float e = __builtin_amdgcn_exp2f(t[r] - m);
        l += e;
        u = fmaf(e, dp[r], u);
      }
    }
    const float inv_l = 1.0f / sum_halves(l);
    const float dsum = sum_halves(u) * inv_l;
    if (g == 0 && q < T) {
      const int64_t si = (n * H + h) * T + q;
      stats[si] = m;
      stats[R + si] = inv_l;
      stats[2 * R + si] = dsum;
    }

    // Pass 2: dQ^T += K^T dS^T.
    f32x16 acc[C::DHP / 32];
#pragma unroll
    for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] = 0.f;
    for (int k0 = 0; k0 < T; k0 += 32) {
      const f32x16 st = block_xyT<DH>(ks, k0, lrow, g, qf);
      const f32x16 dp = block_xyT<DH>(vs, k0, lrow, g, of);
      const bool tail = T - k0 < 32;
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float ds2[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int r = 2 * e + w;
          const float p = __builtin_amdgcn_exp2f(scaled(st[r], c) - m) * inv_l;
          ds2[w] = (tail && key_of(r) >= T - k0) ? 0.f : p * (dp[r] - dsum);
        }
        pk[e] = pack_bf16x2(ds2[0], ds2[1]);
      }
      acc_xT<DH>(ks, k0, lane, pk, acc);
    }
    if (q < T) store_rowT<DH>(dQ + (seq0 + q) * ldd + hoff, g, acc, scale);
  }
}

// --------------------------------------------------------------- key-major
template <int DH>
__global__ __launch_bounds__(64 * kMaxWaves, 2) void attn_bwd_dkv_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int64_t ld, const bf16_t* __restrict__ dO, int64_t ldo, bf16_t* __restrict__ dK,
    bf16_t* __restrict__ dV, int64_t ldd, const float* __restrict__ stats, int64_t R, int T,
    int H, int T_pad, float c, float scale) {
  using C = BwdCfg<DH>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const qs = smem;
  char* const os = smem + T_pad * C::SR;
  // Per query: (m, 1/l, Dsum, 0), one 16-byte read per use.
  float4* const st = reinterpret_cast<float4*>(smem + 2 * T_pad * C::SR);

  const int h = static_cast<int>(blockIdx.x % H);
  const int64_t n = blockIdx.x / H;
  const int64_t seq0 = n * T, hoff = static_cast<int64_t>(h) * DH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const int lrow = lane & 31, g = lane >> 5;
  const int nkt = T_pad / 32;

  stage_rows<DH>(Q + seq0 * ld + hoff, ld, T, T_pad, qs);
  stage_rows<DH>(dO + seq0 * ldo + hoff, ldo, T, T_pad, os);
  const int64_t sb = (n * H + h) * T;
  for (int i = threadIdx.x; i < T_pad; i += blockDim.x) {
    // Queries past T get P = 0: m = +inf, 1/l = 0, Dsum = 0.
    st[i] = i < T ? make_float4(stats[sb + i], stats[R + sb + i], stats[2 * R + sb + i], 0.f)
                  : make_float4(INFINITY, 0.f, 0.f, 0.f);
  }
  __syncthreads();

  for (int kt = wave; kt < nkt; kt += nw) {
    const int key = kt * 32 + lrow, kc = key < T ? key : T - 1;
    bf16x8 kf[DH / 16], vf[DH / 16];
    row_frags<DH>(K + (seq0 + kc) * ld + hoff, g, kf);
    row_frags<DH>(V + (seq0 + kc) * ld + hoff, g, vf);
    f32x16 dk[C::DHP / 32], dv[C::DHP / 32];
#pragma unroll
    for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) dk[d][r] = dv[d][r] = 0.f;

    for (int q0 = 0; q0 < T; q0 += 32) {
      // Accumulator row x is query q0 + perm32(x); the lane's column is its key.
      const f32x16 s = block_xyT<DH>(qs, q0, lrow, g, kf);
      const f32x16 dp = block_xyT<DH>(os, q0, lrow, g, vf);
      uint32_t pp[8], pd[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float pv[2], dv2[2];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const int r = 2 * e + w;
          const int qi = q0 + perm32(8 * (r >> 2) + 4 * g + (r & 3));
          const float4 sq = st[qi];
          const float p = __builtin_amdgcn_exp2f(scaled(s[r], c) - sq.x) * sq.y;
          pv[w] = p;
          dv2[w] = p * (dp[r] - sq.z);
        }
        pp[e] = pack_bf16x2(pv[0], pv[1]);
        pd[e] = pack_bf16x2(dv2[0], dv2[1]);
      }
      acc_xT<DH>(os, q0, lane, pp, dv);  // dV^T += dO^T P
      acc_xT<DH>(qs, q0, lane, pd, dk);  // dK^T += Q^T dS
    }
    if (key < T) {
      store_rowT<DH>(dK + (seq0 + key) * ldd + hoff, g, dk, scale);
      store_rowT<DH>(dV + (seq0 + key) * ldd + hoff, g, dv, 1.0f);
    }
  }
}

template <int DH>
hipError_t launch_bwd(const void* q, const void* k, const void* v, int64_t ld, const void* d_o,
                      int64_t ldo, void* dq, void* dk, void* dv, int64_t ldd, int64_t N,
                      int64_t T, int64_t H, float* stats, hipStream_t s) {
  using C = BwdCfg<DH>;
  const int64_t T_pad = (T + 31) / 32 * 32;
  // Transposed reads of DHP > DH features run up to DHP*2 - DH*2 bytes past
  // a row; the last row's overrun lands in this slack.
  const int64_t slack = (C::DHP - DH) * 2 + 64;
  const int64_t bytes_dq = 2 * T_pad * C::SR + slack;
  const int64_t bytes_dkv = 2 * T_pad * C::SR + T_pad * 16 + slack;
  if (bytes_dq > kLds || bytes_dkv > kLds) return hipErrorNotSupported;
  static std::atomic<bool> attr_set{false};  // set once, idempotent
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<DH>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_dkv_kernel<DH>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLds) != hipSuccess) {
      (void)hipGetLastError();
      return hipErrorNotSupported;
    }
    attr_set.store(true, std::memory_order_relaxed);
  }
  const int64_t tiles = T_pad / 32;
  const int per_wave = static_cast<int>((tiles + kMaxWaves - 1) / kMaxWaves);
  const int nw = static_cast<int>((tiles + per_wave - 1) / per_wave);
  const int64_t blocks = N * H;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const int64_t R = N * H * T;
  const float c = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  const float scale = 1.0f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL(attn_bwd_dq_kernel<DH>, dim3(static_cast<unsigned>(blocks)), dim3(64 * nw),
                     static_cast<size_t>(bytes_dq), s, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), ld,
                     static_cast<const bf16_t*>(d_o), ldo, static_cast<bf16_t*>(dq), ldd, stats,
                     R, static_cast<int>(T), static_cast<int>(H), static_cast<int>(T_pad), c,
                     scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dkv_kernel<DH>, dim3(static_cast<unsigned>(blocks)), dim3(64 * nw),
                     static_cast<size_t>(bytes_dkv), s, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), ld,
                     static_cast<const bf16_t*>(d_o), ldo, static_cast<bf16_t*>(dk),
                     static_cast<bf16_t*>(dv), ldd, static_cast<const float*>(stats), R,
                     static_cast<int>(T), static_cast<int>(H), static_cast<int>(T_pad), c, scale);
  return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// hipErrorNotSupported (nothing launched) when the shape does not qualify:
// bf16 only, a head width with an instantiation, 16-byte aligned rows, and
// the head's two operands resident in LDS.
hipError_t launch_attention_backward_mfma(const void* q, const void* k, const void* v,
                                          int64_t ld, const void* d_o, int64_t ldo, void* dq,
                                          void* dk, void* dv, int64_t ldd, int64_t N, int64_t T,
                                          int64_t H, int64_t dh, float* stats, hipStream_t s) {
  if (ld % 8 != 0 || ldo % 8 != 0 || ldd % 8 != 0 || !aligned16(q) || !aligned16(k) ||
      !aligned16(v) || !aligned16(d_o) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return hipErrorNotSupported;
  switch (dh) {
    case 32: return launch_bwd<32>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H, stats, s);
    case 64: return launch_bwd<64>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H, stats, s);
    case 80: return launch_bwd<80>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H, stats, s);
    case 96: return launch_bwd<96>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H, stats, s);
    case 128: return launch_bwd<128>(q, k, v, ld, d_o, ldo, dq, dk, dv, ldd, N, T, H, stats, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace vitblk
