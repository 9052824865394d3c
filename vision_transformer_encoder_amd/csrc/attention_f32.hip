// fp32 bidirectional multi-head attention on the gfx950 matrix cores.
//
// For every sequence n and head h: O_h = softmax(Q_h K_h^T / sqrt(dh)) V_h
// with no mask (crackedaicode.com "ViT Encoder Block", "Multi-head
// attention"), every product, sum and probability in fp32:
// v_mfma_f32_32x32x2_f32 multiplies and accumulates in full fp32, the
// probabilities stay fp32 (no rounding before the PV product) and their row
// sums are fp32 additions of those same values.
//
// Structure as the bf16 streaming kernel (attention.hip): one workgroup of W
// waves per (sequence, head, up to W query tiles of 32), K and V in 64-key
// chunks through two LDS stages (each thread's share of the next chunk
// requested into registers before the current chunk's tile work, written to
// the other stage after it, one barrier per chunk), online softmax with a
// reference maximum that moves only when a query's maximum exceeds it by
// more than 8 in log2 units.
//
// Matrix-core mapping.  Scores transposed, S^T = K Q^T: MFMA step s of a
// 16-byte read pairs feature 8q + s (lanes 0-31) with 8q + 4 + s (lanes
// 32-63) for both operands; K rows come from LDS (16 consecutive keys per
// read phase, row stride dh + 4 floats: conflict-free), Q from registers.
// Each accumulator lane then holds 16 keys of one query (keys 8b + 4g + r
// of its 32-key block, g = lane / 32), which are exactly the second operand
// of O^T = V^T P^T when step (b, r) pairs key 8b + r (lanes 0-31) with
// 8b + 4 + r (lanes 32-63); V^T's operand is then one float per lane read
// from V's natural [key][feature] layout (row stride a multiple of 16 plus
// 8 floats, so the two lane halves' rows, 4 keys apart, fall in opposite
// bank halves).  Head features past dh up to the next multiple of 32 read
// zeros from LDS padding and feed output rows that are never stored.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kNumXcd = 8;
constexpr float kSlackF32 = 8.0f;  // probabilities < 2^8 between moves of the maximum

template <int DH>
struct F32Cfg {
  static_assert(DH % 16 == 0 && DH <= 128, "head width: a multiple of 16, at most 128");
  static constexpr int DHP = (DH + 31) / 32 * 32;  // V^T rows per MFMA block
  static constexpr int SK = DH + 4;                // K row stride, floats
  static constexpr int SV = DHP + 8;               // V row stride, floats
  static constexpr int STAGE = 64 * (SK + SV);     // floats per LDS stage
};

// x of lanes l and l ^ 32 combined (the same value, in the same order, in
// both): v_permlane32_swap hands every lane both halves' values.
__device__ __forceinline__ float max_of_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_of_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DH, int W>
__global__ __launch_bounds__(64 * W, 2) void attn_f32_mfma_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    int64_t ld, float* __restrict__ O, int64_t ldo, int T, int H, int nqb, int tpb,
    float scale_log2) {
  using C = F32Cfg<DH>;
  extern __shared__ __attribute__((aligned(16))) float smem[];  // [2][64 K rows | 64 V rows]

  // Workgroup -> (n, h, query block); each XCD gets a contiguous run so the
  // query blocks of one head share its K/V in that XCD's L2.
  const int64_t total = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t qx = total / kNumXcd, rx = total % kNumXcd;
  const int64_t x = bid % kNumXcd;
  const int64_t b2 = x * qx + (x < rx ? x : rx) + bid / kNumXcd;
  const int qb = static_cast<int>(b2 % nqb);
  const int64_t nh = b2 / nqb;
  const int64_t seq0 = (nh / H) * static_cast<int64_t>(T);
  const int64_t hoff = static_cast<int64_t>(nh % H) * DH;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, g = lane >> 5;
  const int nqt = (T + 31) / 32;
  const int qt = qb * tpb + wave;
  const bool active = wave < tpb && qt < nqt;  // wave-uniform

  // Staging of one chunk: 64 keys x DH/4 chunks of 16 bytes per operand.
  constexpr int CPR = DH / 4;
  constexpr int PER = 64 * CPR;
  constexpr int NL = (PER + 64 * W - 1) / (64 * W);
  f32x4 rk[NL], rv[NL];
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * 64 * W;
      if (e < PER) {
        int t = c * 64 + e / CPR;
        t = t < T ? t : T - 1;
        const int64_t gofs = (seq0 + t) * ld + hoff + (e % CPR) * 4;
        rk[i] = *reinterpret_cast<const f32x4*>(K + gofs);
        rv[i] = *reinterpret_cast<const f32x4*>(V + gofs);
      }
    }
  };
  auto stash = [&](int st) {
    float* const ks = smem + st * C::STAGE;
    float* const vs = ks + 64 * C::SK;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * 64 * W;
      if (e < PER) {
        *reinterpret_cast<f32x4*>(ks + (e / CPR) * C::SK + (e % CPR) * 4) = rk[i];
        *reinterpret_cast<f32x4*>(vs + (e / CPR) * C::SV + (e % CPR) * 4) = rv[i];
      }
    }
  };

  // This lane's query (clamped to T - 1: its output row is never stored):
  // features 8s + 4g .. +3.
  f32x4 qv[DH / 8];
  if (active) {
    const int q = qt * 32 + l32;
    const float* qrow = Q + (seq0 + (q < T ? q : T - 1)) * ld + hoff + 4 * g;
#pragma unroll
    for (int s = 0; s < DH / 8; ++s) qv[s] = *reinterpret_cast<const f32x4*>(qrow + 8 * s);
  }
  fetch(0);
  if (C::DHP > DH) {  // V features DH..DHP-1 of both stages: zeros
    constexpr int PC = (C::DHP - DH) / 4;
    for (int e = tid; e < 2 * 64 * PC; e += 64 * W) {
      const int st = e / (64 * PC), r = (e / PC) % 64;
      *reinterpret_cast<f32x4*>(smem + st * C::STAGE + 64 * C::SK + r * C::SV + DH +
                                (e % PC) * 4) = f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  stash(0);
  __syncthreads();

  f32x16 o[C::DHP / 32];
#pragma unroll
  for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  // One chunk of 64 keys at (ks, vs); nvalid (>= 1) of them are real.  TAIL:
  // nvalid < 64 (keys past it get score -inf, and a second 32-key block with
  // no real key is skipped).
  auto chunk = [&](auto tail, const float* ks, const float* vs, int nvalid) {
    constexpr bool TAIL = decltype(tail)::value;
    const int nkb = (!TAIL || nvalid > 32) ? 2 : 1;  // 32-key blocks holding a valid key
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
      if (kb < nkb) {
        const float* krow = ks + (kb * 32 + l32) * C::SK + 4 * g;
#pragma unroll
        for (int s = 0; s < DH / 8; ++s) {
          const f32x4 kf = *reinterpret_cast<const f32x4*>(krow + 8 * s);
#pragma unroll
          for (int u = 0; u < 4; ++u)
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[u], qv[s][u], sc[kb], 0, 0, 0);
        }
      }
    }
    // Key kb*32 + 8b + 4g + r of the chunk is element 4b + r of block kb.
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (TAIL && (kb >= nkb || kb * 32 + (r >> 2) * 8 + 4 * g + (r & 3) >= nvalid))
          sc[kb][r] = -INFINITY;
        mx = fmaxf(mx, sc[kb][r]);
      }
    mx = max_of_halves(mx) * scale_log2;
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kSlackF32) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = m_new == m_run ? 1.0f : exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sc[kb][r] = exp2f(fmaf(sc[kb][r], scale_log2, -m_run));
        l_run += sc[kb][r];
      }
    // O^T += V^T P^T.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb >= nkb) continue;
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float* vrow = vs + (kb * 32 + 8 * b + 4 * g + r) * C::SV + l32;
#pragma unroll
          for (int d = 0; d < C::DHP / 32; ++d)
            o[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vrow[d * 32], sc[kb][4 * b + r], o[d],
                                                        0, 0, 0);
        }
    }
  };

  const int KF = T / 64;  // whole 64-key chunks
  const int KC = KF + (T % 64 != 0 ? 1 : 0);
  for (int c = 0; c < KF; ++c) {
    const int st = c & 1;
    if (c + 1 < KC) fetch(c + 1);
    if (active) {
      const float* ks = smem + st * C::STAGE;
      chunk(std::false_type{}, ks, ks + 64 * C::SK, 64);
    }
    if (c + 1 < KC) stash(st ^ 1);
    __syncthreads();
  }
  if (KC > KF && active) {  // the last, partial chunk (already in its stage)
    const float* ks = smem + (KF & 1) * C::STAGE;
    chunk(std::true_type{}, ks, ks + 64 * C::SK, T - KF * 64);
  }
  if (!active) return;
  // O row q, features d*32 + 8b + 4g .. +3 (those < DH), divided by the sum.
  const float inv = 1.0f / sum_of_halves(l_run);
  const int q = qt * 32 + l32;
  if (q >= T) return;
  float* orow = O + (seq0 + q) * ldo + hoff;
#pragma unroll
  for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int f = d * 32 + 8 * b + 4 * g;
      if (f < DH)
        *reinterpret_cast<f32x4*>(orow + f) =
            f32x4{o[d][4 * b] * inv, o[d][4 * b + 1] * inv, o[d][4 * b + 2] * inv,
                  o[d][4 * b + 3] * inv};
    }
}

template <int DH, int W>
hipError_t launch_f32(const void* q, const void* k, const void* v, int64_t ld, void* o,
                      int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s) {
  using C = F32Cfg<DH>;
  constexpr size_t bytes = 2 * static_cast<size_t>(C::STAGE) * sizeof(float);
  static std::atomic<bool> attr_set{false};  // set once, idempotent
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_f32_mfma_kernel<DH, W>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes)) != hipSuccess) {
      (void)hipGetLastError();
      return hipErrorNotSupported;
    }
    attr_set.store(true, std::memory_order_relaxed);
  }
  const int64_t nqt = (T + 31) / 32;
  const int64_t nqb = (nqt + W - 1) / W;
  const int64_t tpb = (nqt + nqb - 1) / nqb;  // query tiles per workgroup, balanced
  const int64_t blocks = N * H * nqb;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL((attn_f32_mfma_kernel<DH, W>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * W), bytes, s, static_cast<const float*>(q),
                     static_cast<const float*>(k), static_cast<const float*>(v), ld,
                     static_cast<float*>(o), ldo, static_cast<int>(T), static_cast<int>(H),
                     static_cast<int>(nqb), static_cast<int>(tpb), scale_log2);
  return hipGetLastError();
}

bool al16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

// fp32 attention on the matrix cores for head widths 32, 64, 80, 96 and 128
// with 16-byte-aligned rows; hipErrorNotSupported (nothing launched)
// otherwise.
hipError_t launch_attention_f32_mfma(const void* q, const void* k, const void* v, int64_t ld,
                                     void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                     int64_t dh, hipStream_t s) {
  if (T <= 0 || ld % 4 != 0 || ldo % 4 != 0 || !al16(q) || !al16(k) || !al16(v) || !al16(o))
    return hipErrorNotSupported;
  switch (dh) {
    case 32: return launch_f32<32, 8>(q, k, v, ld, o, ldo, N, T, H, s);
    case 64: return launch_f32<64, 8>(q, k, v, ld, o, ldo, N, T, H, s);
    case 80: return launch_f32<80, 8>(q, k, v, ld, o, ldo, N, T, H, s);
    case 96: return launch_f32<96, 8>(q, k, v, ld, o, ldo, N, T, H, s);
    case 128: return launch_f32<128, 8>(q, k, v, ld, o, ldo, N, T, H, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace vitblk
