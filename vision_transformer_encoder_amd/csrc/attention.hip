// Bidirectional multi-head attention, flash style, on the gfx950 matrix cores.
//
// For every sequence n and head h: O_h = softmax(Q_h K_h^T / sqrt(dh)) V_h
// with no mask, head h owning the features [h*dh, (h+1)*dh) of Q, K, V and of
// the output (crackedaicode.com "ViT Encoder Block", "Multi-head attention";
// nipunbatra.github.io vision1 transcript, Page 70).  The T x T score matrix
// is never stored: keys are visited in tiles of 64 with a running maximum
// and running sum per query (online softmax), so any T works, including the
// non-power-of-two lengths 197, 257 and 1025.
//
// Layout choices (wave64, v_mfma_f32_32x32x16_bf16):
// * A workgroup is 4 waves; each wave owns 32 queries of one (n, h).
// * Scores are computed transposed, S^T = K Q^T: K rows are the MFMA's first
//   operand (from LDS), Q the second (registers, loaded once).  Each
//   accumulator lane then holds 16 keys of ONE query, so the softmax
//   rescaling is per lane and the probabilities are already laid out as the
//   second operand of O^T = V^T P^T -- no shuffle of P through LDS.  The MFMA
//   k-slot j of lane half g maps to key (j/4)*8 + g*4 + j%4 of a 16-key step,
//   the same mapping for both operands.
// * V is needed key-contiguous (V^T) for that product: each staging thread
//   loads an 8 (key) x 8 (feature) block and transposes it in registers.
// * K/V tiles are double-buffered in LDS; rows are padded by 16 bytes so the
//   32 rows a wave reads per MFMA operand fall in distinct banks.
// * Keys past T are clamped to row T-1 when loaded (finite values) and their
//   scores set to -inf; 32-key blocks entirely past T are skipped.
#include <math.h>

#include "attention_tile.h"
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kWaves = 4;
constexpr int kBQ = 32 * kWaves;  // queries per workgroup
constexpr int kBKV = 64;          // keys per tile
constexpr int kNumXcd = 8;

template <int DH>
struct AttnCfg {
  static_assert(DH % 16 == 0, "head width must be a multiple of 16");
  static constexpr int DHP = (DH + 31) / 32 * 32;  // V^T rows padded to whole 32-row blocks
  static constexpr int KS = DH + 8;                // K tile row stride (elements)
  static constexpr int VS = kBKV + 8;              // V^T tile row stride (elements)
  static constexpr int K_ELEMS = kBKV * KS;
  static constexpr int V_ELEMS = DHP * VS;
  static constexpr int K_CHUNKS = kBKV * DH / 8;         // 16-B chunks per K tile
  static constexpr int K_PER_THREAD = (K_CHUNKS + 255) / 256;
  static constexpr int V_BLOCKS = (kBKV / 8) * (DH / 8);  // 8x8 blocks per V tile
  static constexpr int V_PER_THREAD = (V_BLOCKS + 255) / 256;
};

template <int DH>
__global__ __launch_bounds__(64 * kWaves) void attn_fwd_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int64_t ld, bf16_t* __restrict__ O, int64_t ldo, int T, int H, int nqb, float scale_log2) {
  using C = AttnCfg<DH>;
  __shared__ __attribute__((aligned(16))) bf16_t ks_buf[2][C::K_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16_t vt_buf[2][C::V_ELEMS];

  // Workgroup -> (n, h, query block); each XCD gets a contiguous run so the
  // query blocks of one head share its K/V in that XCD's L2.
  const int64_t total = gridDim.x;
  const int64_t bid = blockIdx.x;
  const int64_t qx = total / kNumXcd, rx = total % kNumXcd;
  const int64_t x = bid % kNumXcd;
  const int64_t b2 = x * qx + (x < rx ? x : rx) + bid / kNumXcd;
  const int qb = static_cast<int>(b2 % nqb);
  const int64_t nh = b2 / nqb;
  const int h = static_cast<int>(nh % H);
  const int64_t n = nh / H;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, g = lane >> 5;
  const int64_t seq0 = n * static_cast<int64_t>(T);
  const int64_t hoff = static_cast<int64_t>(h) * DH;

  // This lane's query (column of S^T) and its Q fragments for every 16-wide k-step.
  const int q = qb * kBQ + wave * 32 + lrow;
  const int qc = q < T ? q : T - 1;
  bf16x8 qf[DH / 16];
  {
    const bf16_t* qrow = Q + (seq0 + qc) * ld + hoff + g * 8;
#pragma unroll
    for (int s = 0; s < DH / 16; ++s) qf[s] = __builtin_bit_cast(bf16x8, ld_global16(qrow + s * 16));
  }

  // Padding rows of V^T (features DH..DHP-1) only feed discarded output rows;
  // zero them once so they hold finite values.
  if (C::DHP > DH) {
    for (int e = tid; e < (C::DHP - DH) * C::VS; e += 64 * kWaves) {
      vt_buf[0][DH * C::VS + e] = 0;
      vt_buf[1][DH * C::VS + e] = 0;
    }
  }

  uint4 rk[C::K_PER_THREAD];
  uint4 rv[C::V_PER_THREAD][8];
  auto fetch = [&](int kt) {
    const int key0 = kt * kBKV;
#pragma unroll
    for (int i = 0; i < C::K_PER_THREAD; ++i) {
      const int c = tid + i * 256;
      if (c < C::K_CHUNKS) {
        const int key = c / (DH / 8), dc = c % (DH / 8);
        int t = key0 + key;
        t = t < T ? t : T - 1;
        rk[i] = ld_global16(K + (seq0 + t) * ld + hoff + dc * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_THREAD; ++i) {
      const int blk = tid + i * 256;
      if (blk < C::V_BLOCKS) {
        const int kb8 = blk / (DH / 8), dc = blk % (DH / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          int t = key0 + kb8 * 8 + r;
          t = t < T ? t : T - 1;
          rv[i][r] = ld_global16(V + (seq0 + t) * ld + hoff + dc * 8);
        }
      }
    }
  };
  auto stash = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::K_PER_THREAD; ++i) {
      const int c = tid + i * 256;
      if (c < C::K_CHUNKS) {
        const int key = c / (DH / 8), dc = c % (DH / 8);
        *reinterpret_cast<uint4*>(&ks_buf[st][key * C::KS + dc * 8]) = rk[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::V_PER_THREAD; ++i) {
      const int blk = tid + i * 256;
      if (blk < C::V_BLOCKS) {
        const int kb8 = blk / (DH / 8), dc = blk % (DH / 8);
        uint4 tr[8];
        transpose8x8_b16(rv[i], tr);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          *reinterpret_cast<uint4*>(&vt_buf[st][(dc * 8 + j) * C::VS + kb8 * 8]) = tr[j];
      }
    }
  };

  f32x16 o[C::DHP / 32];
#pragma unroll
  for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int KT = (T + kBKV - 1) / kBKV;
  fetch(0);
  stash(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) fetch(kt + 1);
    const bf16_t* ks = ks_buf[st];
    const bf16_t* vt = vt_buf[st];
    const int key0 = kt * kBKV;
    const int nkb = (T - key0) > 32 ? 2 : 1;  // 32-key blocks holding a valid key

    // S^T for up to two 32-key blocks: rows = keys, columns = this wave's queries.
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      if (kb < nkb) {
#pragma unroll
        for (int ks_ = 0; ks_ < DH / 16; ++ks_) {
          const bf16x8 kf = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const uint4*>(&ks[(kb * 32 + lrow) * C::KS + ks_ * 16 + g * 8]));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks_], s[kb], 0, 0, 0);
        }
      }
    }

    // Running maximum of the raw scores (keys past T masked to -inf: key
    // kb*32 + (r/4)*8 + g*4 + r%4 of the tile is valid iff it is < lim), then
    // p = 2^(s * scale * log2(e) - m) with one FMA per score.
    const int lim = T - key0 - g * 4;
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kb * 32 + (r >> 2) * 8 + (r & 3) >= lim) s[kb][r] = -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][r], scale_log2, -m_new));
        s[kb][r] = pv;
        psum += pv;
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] *= alpha;

    // O^T += V^T P^T, 16 keys per MFMA step.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb >= nkb) continue;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t pw[4] = {pack_bf16x2(s[kb][s2 * 8 + 0], s[kb][s2 * 8 + 1]),
                                pack_bf16x2(s[kb][s2 * 8 + 2], s[kb][s2 * 8 + 3]),
                                pack_bf16x2(s[kb][s2 * 8 + 4], s[kb][s2 * 8 + 5]),
                                pack_bf16x2(s[kb][s2 * 8 + 6], s[kb][s2 * 8 + 7])};
        const bf16x8 pf = __builtin_bit_cast(bf16x8, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        const int kofs = kb * 32 + s2 * 16 + g * 4;
#pragma unroll
        for (int d = 0; d < C::DHP / 32; ++d) {
          const bf16_t* vrow = vt + (d * 32 + lrow) * C::VS + kofs;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          const bf16x8 vf = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[d], 0, 0, 0);
        }
      }
    }

    if (kt + 1 < KT) stash(st ^ 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.0f / l_tot;
  if (q < T) {
    bf16_t* orow = O + (seq0 + q) * ldo + hoff;
#pragma unroll
    for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int f = d * 32 + rr * 8 + g * 4;
        if (f < DH)
          *reinterpret_cast<uint2*>(orow + f) =
              make_uint2(pack_bf16x2(o[d][rr * 4 + 0] * inv, o[d][rr * 4 + 1] * inv),
                         pack_bf16x2(o[d][rr * 4 + 2] * inv, o[d][rr * 4 + 3] * inv));
      }
  }
}

// ---------------------------------------------------------------- streaming kernel
//
// Sequences too long for the resident kernel (ViT at 512 px: T = 1025): keys
// stream through LDS in 64-key chunks, two stages deep.  A workgroup is 8
// waves over one (sequence, head) and up to 8 query tiles of 32, so each
// K/V chunk copied into LDS serves up to 256 queries; per chunk every thread
// requests its share of the next chunk before the tile work on the current
// one and writes it to the other stage after, and one barrier ends the chunk.
// The per-tile work is attention_tile.h's (the resident kernel's).
constexpr int kStreamWaves = 8;

template <int DH>
__global__ __launch_bounds__(64 * kStreamWaves, (DH <= 64 ? 4 : 2)) void attn_stream_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int64_t ld, bf16_t* __restrict__ O, int64_t ldo, int T, int H, int nqb, int tpb,
    float scale_log2) {
  using C = attn::Cfg<DH>;
  extern __shared__ __attribute__((aligned(16))) char smem[];  // [2][64 K rows | 64 V rows]
  constexpr int STAGE = 64 * C::ROW;

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
  const int nqt = (T + 31) / 32;
  const int qt = qb * tpb + wave;
  const bool active = wave < tpb && qt < nqt;  // wave-uniform

  // Staging of one chunk: 64 keys x DH/8 chunks of 16 bytes per operand.
  constexpr int CPR = DH / 8;
  constexpr int PER = 64 * CPR;
  constexpr int NL = (PER + 64 * kStreamWaves - 1) / (64 * kStreamWaves);
  uint4 rk[NL], rv[NL];
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * 64 * kStreamWaves;
      if (e < PER) {
        int t = c * 64 + e / CPR;
        t = t < T ? t : T - 1;
        const int64_t gofs = (seq0 + t) * ld + hoff + (e % CPR) * 8;
        rk[i] = ld_global16(K + gofs);
        rv[i] = ld_global16(V + gofs);
      }
    }
  };
  auto stash = [&](int st) {
    char* const ks = smem + st * STAGE;
    char* const vs = ks + 64 * C::SK;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * 64 * kStreamWaves;
      if (e < PER) {
        *reinterpret_cast<uint4*>(ks + (e / CPR) * C::SK + (e % CPR) * 16) = rk[i];
        *reinterpret_cast<uint4*>(vs + (e / CPR) * C::SV + (e % CPR) * 16) = rv[i];
      }
    }
  };

  attn::QLoad<DH> ql;
  if (active) ql.issue(Q, ld, seq0, hoff, T, qt * 32, lane);
  fetch(0);
  if (C::DHP > DH) {  // features DH..DHP-1 of V feed only discarded output rows; keep them 0
    constexpr int PC = (C::DHP - DH) / 8;
    for (int e = tid; e < 2 * 64 * PC; e += 64 * kStreamWaves) {
      const int st = e / (64 * PC), r = (e / PC) % 64;
      *reinterpret_cast<uint4*>(smem + st * STAGE + 64 * C::SK + r * C::SV +
                                (DH + (e % PC) * 8) * 2) = make_uint4(0, 0, 0, 0);
    }
  }
  stash(0);
  if (active) ql.finish(lane);
  __syncthreads();

  attn::Tile<DH> tile;
  tile.init();
  const int v_lane = attn::v_lane_offset<DH>(lane);
  const int KF = T / 64;                 // whole 64-key chunks
  const int KC = KF + (T % 64 != 0 ? 1 : 0);
  for (int c = 0; c < KF; ++c) {
    const int st = c & 1;
    if (c + 1 < KC) fetch(c + 1);
    if (active) {
      const char* ks = smem + st * STAGE;
      tile.template chunk<false>(ql.qf, ks, ks + 64 * C::SK, 64, scale_log2, lane, v_lane);
    }
    if (c + 1 < KC) stash(st ^ 1);
    __syncthreads();
  }
  if (KC > KF && active) {  // the last, partial chunk (already in its stage)
    const char* ks = smem + (KF & 1) * STAGE;
    tile.template chunk<true>(ql.qf, ks, ks + 64 * C::SK, T - KF * 64, scale_log2, lane, v_lane);
  }
  if (active) tile.store(O, ldo, seq0, hoff, T, qt * 32, lane);
}

template <int DH>
hipError_t launch_stream(const void* q, const void* k, const void* v, int64_t ld, void* o,
                         int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s) {
  using C = attn::Cfg<DH>;
  constexpr size_t bytes = 2 * 64 * C::ROW;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_stream_kernel<DH>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes)) != hipSuccess) {
      (void)hipGetLastError();
      return hipErrorNotSupported;
    }
    attr_set = true;
  }
  const int64_t nqt = (T + 31) / 32;
  const int64_t nqb = (nqt + kStreamWaves - 1) / kStreamWaves;
  const int64_t tpb = (nqt + nqb - 1) / nqb;  // query tiles per workgroup, balanced
  const int64_t blocks = N * H * nqb;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL(attn_stream_kernel<DH>, dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * kStreamWaves), bytes, s, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), ld,
                     static_cast<bf16_t*>(o), ldo, static_cast<int>(T), static_cast<int>(H),
                     static_cast<int>(nqb), static_cast<int>(tpb), scale_log2);
  return hipGetLastError();
}

template <int DH>
hipError_t launch_dh(const void* q, const void* k, const void* v, int64_t ld, void* o,
                     int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s) {
  const int64_t nqb = (T + kBQ - 1) / kBQ;
  const int64_t blocks = N * H * nqb;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL(attn_fwd_kernel<DH>, dim3(static_cast<unsigned>(blocks)), dim3(64 * kWaves),
                     0, s, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), ld, static_cast<bf16_t*>(o), ldo,
                     static_cast<int>(T), static_cast<int>(H), static_cast<int>(nqb), scale_log2);
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

hipError_t launch_attention(const void* q, const void* k, const void* v, int64_t ld, void* o,
                            int64_t ldo, int64_t N, int64_t T, int64_t H, int64_t dh, int dtype,
                            hipStream_t s) {
  const bool fast = dtype == VITBLK_BF16 && ld % 8 == 0 && ldo % 8 == 0 && aligned16(q) &&
                    aligned16(k) && aligned16(v) && aligned16(o);
  if (fast) {
    hipError_t r = launch_attention_resident(q, k, v, ld, o, ldo, N, T, H, dh, s);
    if (r != hipErrorNotSupported) return r;
    switch (dh) {
      case 32: r = launch_stream<32>(q, k, v, ld, o, ldo, N, T, H, s); break;
      case 64: r = launch_stream<64>(q, k, v, ld, o, ldo, N, T, H, s); break;
      case 80: r = launch_stream<80>(q, k, v, ld, o, ldo, N, T, H, s); break;
      case 96: r = launch_stream<96>(q, k, v, ld, o, ldo, N, T, H, s); break;
      case 128: r = launch_stream<128>(q, k, v, ld, o, ldo, N, T, H, s); break;
      default: break;
    }
    if (r != hipErrorNotSupported) return r;
    switch (dh) {
      case 32: return launch_dh<32>(q, k, v, ld, o, ldo, N, T, H, s);
      case 64: return launch_dh<64>(q, k, v, ld, o, ldo, N, T, H, s);
      case 80: return launch_dh<80>(q, k, v, ld, o, ldo, N, T, H, s);
      case 96: return launch_dh<96>(q, k, v, ld, o, ldo, N, T, H, s);
      case 128: return launch_dh<128>(q, k, v, ld, o, ldo, N, T, H, s);
      default: break;
    }
  }
  return launch_attention_generic(q, k, v, ld, o, ldo, N, T, H, dh, dtype, s);
}

}  // namespace vitblk
