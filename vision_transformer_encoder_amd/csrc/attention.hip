// Bidirectional multi-head attention, flash style, on the gfx950 matrix cores:
// the streaming kernel and the choice between it, the resident kernel
// (attention_resident.hip) and the generic one.
//
// For every sequence n and head h: O_h = softmax(Q_h K_h^T / sqrt(dh)) V_h
// with no mask, head h owning the features [h*dh, (h+1)*dh) of Q, K, V and of
// the output (crackedaicode.com "ViT Encoder Block", "Multi-head attention";
// nipunbatra.github.io vision1 transcript, Page 70).  The T x T score matrix
// is never stored: keys are visited in chunks of 64 with a running maximum
// and running sum per query (online softmax), so any T works, including the
// non-power-of-two lengths 197, 257 and 1025.  Keys past T are clamped to row
// T-1 when loaded (finite values) and their scores set to -inf.
#include <math.h>

#include <atomic>

#include "attention_tile.h"
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kNumXcd = 8;

// ---------------------------------------------------------------- streaming kernel
//
// W waves per workgroup (kStreamWaves unless a head width says otherwise).
constexpr int kStreamWaves = 8;
//
// Keys stream through LDS in 64-key chunks, two stages deep.  A workgroup is 8
// waves over one (sequence, head) and up to 8 query tiles of 32, so each
// K/V chunk copied into LDS serves up to 256 queries; per chunk every thread
// requests its share of the next chunk before the tile work on the current
// one and writes it to the other stage after, and one barrier ends the chunk.
// The per-tile work is attention_tile.h's (the resident kernel's).
template <int DH, int W>
__global__ __launch_bounds__(64 * W, (DH <= 64 ? 4 : 2)) void attn_stream_kernel(
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
  constexpr int NL = (PER + 64 * W - 1) / (64 * W);
  uint4 rk[NL], rv[NL];
  auto fetch = [&](int c) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + i * 64 * W;
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
      const int e = tid + i * 64 * W;
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
    for (int e = tid; e < 2 * 64 * PC; e += 64 * W) {
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

// max_qt > 0: only the first max_qt query tiles of each sequence (all keys).
template <int DH, int W = kStreamWaves>
hipError_t launch_stream(const void* q, const void* k, const void* v, int64_t ld, void* o,
                         int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s,
                         int64_t max_qt = 0) {
  using C = attn::Cfg<DH>;
  constexpr size_t bytes = 2 * 64 * C::ROW;
  static std::atomic<bool> attr_set{false};  // set once, idempotent
  if (!attr_set.load(std::memory_order_relaxed)) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_stream_kernel<DH, W>),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(bytes)) != hipSuccess) {
      (void)hipGetLastError();
      return hipErrorNotSupported;
    }
    attr_set.store(true, std::memory_order_relaxed);
  }
  int64_t nqt = (T + 31) / 32;
  if (max_qt > 0 && nqt > max_qt) nqt = max_qt;  // the kernel then skips waves past tpb
  const int64_t nqb = (nqt + W - 1) / W;
  const int64_t tpb = (nqt + nqb - 1) / nqb;  // query tiles per workgroup, balanced
  const int64_t blocks = N * H * nqb;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL((attn_stream_kernel<DH, W>), dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * W), bytes, s, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v), ld,
                     static_cast<bf16_t*>(o), ldo, static_cast<int>(T), static_cast<int>(H),
                     static_cast<int>(nqb), static_cast<int>(tpb), scale_log2);
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

hipError_t launch_stream_dh(const void* q, const void* k, const void* v, int64_t ld, void* o,
                            int64_t ldo, int64_t N, int64_t T, int64_t H, int64_t dh,
                            hipStream_t s, int64_t max_qt = 0) {
  switch (dh) {
    case 32: return launch_stream<32>(q, k, v, ld, o, ldo, N, T, H, s, max_qt);
    case 64: return launch_stream<64>(q, k, v, ld, o, ldo, N, T, H, s, max_qt);
    case 80: return launch_stream<80, 4>(q, k, v, ld, o, ldo, N, T, H, s, max_qt);
    case 96: return launch_stream<96>(q, k, v, ld, o, ldo, N, T, H, s, max_qt);
    case 128: return launch_stream<128>(q, k, v, ld, o, ldo, N, T, H, s, max_qt);
    default: return hipErrorNotSupported;
  }
}

}  // namespace

// Kernel choice (bf16): head widths up to 80 take the streaming kernel at every
// T (measured at ViT-B/16 and ViT-L/16: its chunk-by-chunk copies overlap the
// tile work, 8-9% faster than holding the whole sequence).  Width 80 needs
// about 150 registers per wave, so it streams with 4-wave workgroups, three
// per CU (ViT-H/14: 123 us, against 159 on the resident kernel and 181 with
// 8-wave workgroups, one per CU).  Wider heads take the resident kernel while
// the sequence fits in LDS and stream beyond.  fp32 with the same head widths:
// the fp32 matrix-core kernel (attention_f32.hip).  Other shapes: the generic
// kernel.
hipError_t launch_attention(const void* q, const void* k, const void* v, int64_t ld, void* o,
                            int64_t ldo, int64_t N, int64_t T, int64_t H, int64_t dh, int dtype,
                            hipStream_t s) {
  const bool fast = dtype == VITBLK_BF16 && ld % 8 == 0 && ldo % 8 == 0 && aligned16(q) &&
                    aligned16(k) && aligned16(v) && aligned16(o);
  if (fast) {
    hipError_t r = hipErrorNotSupported;
    if (dh <= 80) r = launch_stream_dh(q, k, v, ld, o, ldo, N, T, H, dh, s);
    if (r == hipErrorNotSupported) r = launch_attention_resident(q, k, v, ld, o, ldo, N, T, H, dh, s);
    if (r == hipErrorNotSupported) r = launch_stream_dh(q, k, v, ld, o, ldo, N, T, H, dh, s);
    if (r != hipErrorNotSupported) return r;
  }
  if (dtype == VITBLK_FP32) {
    const hipError_t r = launch_attention_f32_mfma(q, k, v, ld, o, ldo, N, T, H, dh, s);
    if (r != hipErrorNotSupported) return r;
  }
  return launch_attention_generic(q, k, v, ld, o, ldo, N, T, H, dh, dtype, s);
}

hipError_t launch_attention_first_queries(const void* q, const void* k, const void* v,
                                          int64_t ld, void* o, int64_t ldo, int64_t N, int64_t T,
                                          int64_t H, int64_t dh, int dtype, hipStream_t s) {
  const bool fast = dtype == VITBLK_BF16 && ld % 8 == 0 && ldo % 8 == 0 && aligned16(q) &&
                    aligned16(k) && aligned16(v) && aligned16(o);
  if (fast && dh <= 64) {
    const hipError_t r = launch_stream_dh(q, k, v, ld, o, ldo, N, T, H, dh, s, 1);
    if (r != hipErrorNotSupported) return r;
  }
  return launch_attention(q, k, v, ld, o, ldo, N, T, H, dh, dtype, s);
}

}  // namespace vitblk
