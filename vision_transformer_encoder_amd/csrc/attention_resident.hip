// Bidirectional multi-head attention with the whole sequence's K and V
// resident in LDS (sequences up to a few hundred tokens: ViT's 197 and 257).
//
// Computes, for every sequence n and head h, O_h = softmax(Q_h K_h^T /
// sqrt(dh)) V_h with no mask, head h owning features [h*dh, (h+1)*dh)
// (crackedaicode.com "ViT Encoder Block", "Multi-head attention";
// nipunbatra.github.io vision1 transcript, Page 70).
//
// One workgroup per (sequence, head).  All its threads first copy K and V of
// that head into LDS (one round of global loads, so memory latency is paid
// once per workgroup), then each wave takes 32-query tiles and walks the keys
// in chunks of 64 with a running maximum and sum per query (online softmax),
// with no further barriers.  The per-tile work (matrix-core mapping, LDS
// layouts, softmax) is in attention_tile.h.  Keys past T are loaded from row
// T-1 (finite values) and their scores are set to -inf.
#include <math.h>

#include <atomic>

#include "attention_tile.h"
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup

template <int DH>
__global__ __launch_bounds__(64 * kMaxWaves, (DH <= 64 ? 4 : 2)) void attn_resident_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int64_t ld, bf16_t* __restrict__ O, int64_t ldo, int T, int H, int T_pad,
    float scale_log2) {
  using C = attn::Cfg<DH>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const ks = smem;                 // [T_pad][SK]
  char* const vs = smem + T_pad * C::SK;  // [T_pad][SV]

  const int h = static_cast<int>(blockIdx.x % H);
  const int64_t n = blockIdx.x / H;
  const int64_t seq0 = n * T;
  const int64_t hoff = static_cast<int64_t>(h) * DH;
  const int tid = threadIdx.x, nthreads = blockDim.x;

  const int lane = tid & 63, wave = tid >> 6, nw = nthreads >> 6;
  const int nqt = T_pad / 32;

  // The wave's first Q tile is requested together with K and V, so the
  // workgroup waits for one round of memory latency, not two.
  attn::QLoad<DH> ql;
  if (wave < nqt) ql.issue(Q, ld, seq0, hoff, T, wave * 32, lane);

  // ---- K and V of this head into LDS (4 chunks of 16 B per operand in flight per thread).
  constexpr int CPR = DH / 8;  // 16-byte chunks per row
  const int chunks = T_pad * CPR;
  for (int c0 = tid; c0 < chunks; c0 += 4 * nthreads) {
    uint4 kv[4], vv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * nthreads;
      if (c < chunks) {
        const int key = c / CPR, dc = c % CPR;
        const int t = key < T ? key : T - 1;
        const int64_t g = (seq0 + t) * ld + hoff + dc * 8;
        kv[u] = ld_global16(K + g);
        vv[u] = ld_global16(V + g);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int c = c0 + u * nthreads;
      if (c < chunks) {
        const int key = c / CPR, dc = c % CPR;
        *reinterpret_cast<uint4*>(ks + key * C::SK + dc * 16) = kv[u];
        *reinterpret_cast<uint4*>(vs + key * C::SV + dc * 16) = vv[u];
      }
    }
  }
  if (C::DHP > DH) {  // features DH..DHP-1 of V feed only discarded output rows; keep them 0
    constexpr int PC = (C::DHP - DH) / 8;
    for (int c = tid; c < T_pad * PC; c += nthreads)
      *reinterpret_cast<uint4*>(vs + (c / PC) * C::SV + (DH + (c % PC) * 8) * 2) =
          make_uint4(0, 0, 0, 0);
  }
  if (wave < nqt) ql.finish(lane);
  __syncthreads();

  const int v_lane = attn::v_lane_offset<DH>(lane);
  for (int qt = wave; qt < nqt; qt += nw) {
    if (qt != wave) {
      ql.issue(Q, ld, seq0, hoff, T, qt * 32, lane);
      ql.finish(lane);
    }
    attn::Tile<DH> tile;
    tile.init();
    int k0 = 0;
    for (; k0 + 64 <= T; k0 += 64)
      tile.template chunk<false>(ql.qf, ks + k0 * C::SK, vs + k0 * C::SV, 64, scale_log2, lane,
                                 v_lane);
    if (k0 < T)
      tile.template chunk<true>(ql.qf, ks + k0 * C::SK, vs + k0 * C::SV, T - k0, scale_log2,
                                lane, v_lane);
    tile.store(O, ldo, seq0, hoff, T, qt * 32, lane);
  }
}

template <int DH>
hipError_t launch_res(const void* q, const void* k, const void* v, int64_t ld, void* o,
                      int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s) {
  using C = attn::Cfg<DH>;
  const int64_t T_pad = (T + 31) / 32 * 32;
  const int64_t bytes = T_pad * C::ROW;
  if (bytes > kLdsBytes) return hipErrorNotSupported;
  static std::atomic<bool> attr_set{false};  // set once, idempotent
  if (!attr_set.load(std::memory_order_relaxed)) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_resident_kernel<DH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // clear it: the caller falls back to the streaming kernel
      return hipErrorNotSupported;
    }
    attr_set.store(true, std::memory_order_relaxed);
  }
  const int64_t nqt = T_pad / 32;
  const int per_wave = static_cast<int>((nqt + kMaxWaves - 1) / kMaxWaves);
  const int nw = static_cast<int>((nqt + per_wave - 1) / per_wave);
  const int64_t blocks = N * H;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(DH));
  hipLaunchKernelGGL(attn_resident_kernel<DH>, dim3(static_cast<unsigned>(blocks)),
                     dim3(64 * nw), static_cast<size_t>(bytes), s,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), ld, static_cast<bf16_t*>(o), ldo,
                     static_cast<int>(T), static_cast<int>(H), static_cast<int>(T_pad),
                     scale_log2);
  return hipGetLastError();
}

}  // namespace

// Returns hipErrorNotSupported (launching nothing) when the sequence does not
// fit in LDS or the head width has no instantiation; the caller then uses the
// streaming kernel.
hipError_t launch_attention_resident(const void* q, const void* k, const void* v, int64_t ld,
                                     void* o, int64_t ldo, int64_t N, int64_t T, int64_t H,
                                     int64_t dh, hipStream_t s) {
  switch (dh) {
    case 32: return launch_res<32>(q, k, v, ld, o, ldo, N, T, H, s);
    case 64: return launch_res<64>(q, k, v, ld, o, ldo, N, T, H, s);
    case 80: return launch_res<80>(q, k, v, ld, o, ldo, N, T, H, s);
    case 96: return launch_res<96>(q, k, v, ld, o, ldo, N, T, H, s);
    case 128: return launch_res<128>(q, k, v, ld, o, ldo, N, T, H, s);
    default: return hipErrorNotSupported;
  }
}

}  // namespace vitblk
