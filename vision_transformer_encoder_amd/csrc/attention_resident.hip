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
// with no further barriers.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16), as in the streaming kernel:
// scores are formed transposed, S^T = K Q^T, so each accumulator lane holds
// 16 keys of one query and the probabilities are already the second operand
// of O^T = V^T P^T.  V stays in its natural [key][feature] layout in LDS; its
// transpose is read with ds_read_b64_tr_b16, which hands lane i of a 16-lane
// group column i of the 4 x 16 block that the group's lanes point at (lane
// m points at row m/4, columns 4*(m%4)..+3).
//
// LDS rows are padded so that reads are conflict-free on gfx950 (64 banks):
// K rows (read 16 consecutive keys x 16 B) use a stride of dh*2 + 16 bytes;
// V rows (read 4 consecutive keys x 64 B) use a stride that is 64 or 192
// modulo 256.  Keys past T are loaded from row T-1 (finite values) and their
// scores are set to -inf.
#include <math.h>

#include <type_traits>

#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kMaxWaves = 8;
constexpr int kLdsBytes = 160 * 1024;  // gfx950 LDS per workgroup

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Slack of the reference maximum, in log2 units (probabilities < 2^8).
constexpr float kSlack = 8.0f;
// bf16 pair (1, 1): a dot product with it sums a packed pair.
constexpr bf16x2_t kOnes = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

template <int DH>
struct ResCfg {
  static_assert(DH % 16 == 0, "head width must be a multiple of 16");
  static constexpr int DHP = (DH + 31) / 32 * 32;                     // V^T rows per MFMA block
  static constexpr int SK = DH * 2 + 16;                              // K row stride, bytes
  static constexpr int SV = (DHP * 2) % 128 == 0 ? DHP * 2 + 64 : DHP * 2;  // V row stride
  static constexpr int ROW = SK + SV;
};

// (x of lane l, x of lane l ^ 32) for every lane, by one v_permlane32_swap:
// its first result holds lanes 0-31 of x in both halves, its second lanes
// 32-63 in both halves.
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

template <int DH>
__global__ __launch_bounds__(64 * kMaxWaves, (DH <= 64 ? 4 : 2)) void attn_resident_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ K, const bf16_t* __restrict__ V,
    int64_t ld, bf16_t* __restrict__ O, int64_t ldo, int T, int H, int T_pad,
    float scale_log2) {
  using C = ResCfg<DH>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const ks = smem;                 // [T_pad][SK]
  char* const vs = smem + T_pad * C::SK;  // [T_pad][SV]

  const int h = static_cast<int>(blockIdx.x % H);
  const int64_t n = blockIdx.x / H;
  const int64_t seq0 = n * T;
  const int64_t hoff = static_cast<int64_t>(h) * DH;
  const int tid = threadIdx.x, nthreads = blockDim.x;

  const int lane = tid & 63, wave = tid >> 6, nw = nthreads >> 6;
  const int lrow = lane & 31, g = lane >> 5;
  const int nqt = T_pad / 32;

  // Q fragments of a 32-query tile: lane (lrow, g) holds features
  // 16s + 8g .. +7 of query qt*32 + lrow (clamped to T-1), s = 0 .. DH/16-1.
  // Each whole 64-feature group is read as full 128-byte row lines (8 lanes
  // per query row) and regrouped into that layout (lines_to_rows); the rest
  // (DH % 64) is read in the fragment layout directly.
  constexpr int G64 = DH / 64;
  bf16x8 qf[DH / 16];
  uint4 qv[G64 > 0 ? G64 : 1][4];
  auto issue_q = [&](int qt) {
#pragma unroll
    for (int gi = 0; gi < G64; ++gi)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int qq = qt * 32 + t * 8 + (lane >> 3);
        qv[gi][t] = ld_global16(Q + (seq0 + (qq < T ? qq : T - 1)) * ld + hoff + gi * 64 +
                                (lane & 7) * 8);
      }
    const int q = qt * 32 + lrow;
    const bf16_t* qrow = Q + (seq0 + (q < T ? q : T - 1)) * ld + hoff + g * 8;
#pragma unroll
    for (int s = G64 * 4; s < DH / 16; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, ld_global16(qrow + s * 16));
  };
  auto finish_q = [&]() {
#pragma unroll
    for (int gi = 0; gi < G64; ++gi) {
      lines_to_rows(qv[gi], lane);
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[gi * 4 + s] = __builtin_bit_cast(bf16x8, qv[gi][s]);
    }
  };
  // The wave's first Q tile is requested together with K and V, so the
  // workgroup waits for one round of memory latency, not two.
  if (wave < nqt) issue_q(wave);

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
  if (wave < nqt) finish_q();
  __syncthreads();

  const int i16 = lane & 15, q16 = (lane >> 4) & 1;
  // Lane's V^T read address relative to (key0, feature block): row key0 + i16/4,
  // columns q16*16 + 4*(i16 % 4) of the 32-feature block.
  const int v_lane = (i16 >> 2) * C::SV + (q16 * 16 + 4 * (i16 & 3)) * 2;

  for (int qt = wave; qt < nqt; qt += nw) {
    const int q = qt * 32 + lrow;
    if (qt != wave) {
      issue_q(qt);
      finish_q();
    }
    f32x16 o[C::DHP / 32];
#pragma unroll
    for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    // m_run: the reference maximum (log2 units) the probabilities are taken
    // against; l_run: this lane's share of their sum (the other lane half
    // holds the rest of the query's keys).
    float m_run = -INFINITY, l_run = 0.f;

    // One chunk of 64 keys starting at k0.  TAIL: the chunk runs past T
    // (its keys >= T get score -inf, and a second 32-key block with no
    // valid key is skipped).
    auto chunk = [&](const int k0, auto tail) {
      constexpr bool TAIL = decltype(tail)::value;
      const int nkb = (!TAIL || T - k0 > 32) ? 2 : 1;  // 32-key blocks holding a valid key
      f32x16 sc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb < nkb) {
          const char* krow = ks + (k0 + kb * 32 + lrow) * C::SK + g * 16;
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(krow), qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
          for (int ks_ = 1; ks_ < DH / 16; ++ks_) {
            const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks_ * 32);
            sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks_], sc[kb], 0, 0, 0);
          }
        }
      }
      // Maximum of the raw scores.  Key kb*32 + (r/4)*8 + g*4 + r%4 of the
      // chunk is valid iff it is < T - k0.
      float mx = -INFINITY;
      if (TAIL) {
        const int lim = T - k0 - g * 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (kb >= nkb || kb * 32 + (r >> 2) * 8 + (r & 3) >= lim) sc[kb][r] = -INFINITY;
            mx = fmaxf(mx, sc[kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      }
      mx = max_halves(mx) * scale_log2;
      // The reference maximum moves only when some query's maximum exceeds
      // it by more than kSlack (so probabilities stay below 2^kSlack); the
      // accumulators are rescaled only then, for the whole wave at once.
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(mx > m_run + kSlack) != 0, 0)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int d = 0; d < C::DHP / 32; ++d)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[d][r] *= alpha;
      }
      // p = 2^(s * scale * log2(e) - m), rounded once to bf16: that is the
      // MFMA operand, and its row sum is taken from the same rounded values.
      uint32_t pk[2][8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb >= nkb) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pk[kb][e] = pack_bf16x2(
              __builtin_amdgcn_exp2f(fmaf(sc[kb][2 * e], scale_log2, -m_run)),
              __builtin_amdgcn_exp2f(fmaf(sc[kb][2 * e + 1], scale_log2, -m_run)));
          l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[kb][e]),
                                                  kOnes, l_run, false);
        }
      }
      // O^T += V^T P^T, 16 keys per MFMA: MFMA k-slot j of lane half g is key
      // (j/4)*8 + g*4 + j%4 of the 16-key step, for both operands.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb >= nkb) continue;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const bf16x8 pf = __builtin_bit_cast(
              bf16x8, make_uint4(pk[kb][s2 * 4 + 0], pk[kb][s2 * 4 + 1], pk[kb][s2 * 4 + 2],
                                 pk[kb][s2 * 4 + 3]));
          const char* vb = vs + (k0 + kb * 32 + s2 * 16 + g * 4) * C::SV + v_lane;
#pragma unroll
          for (int d = 0; d < C::DHP / 32; ++d) {
            const v4i16 lo = ds_read_tr16(vb + d * 64);
            const v4i16 hi = ds_read_tr16(vb + 8 * C::SV + d * 64);
            const bf16x8 vf = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[d], 0, 0, 0);
          }
        }
      }
    };
    int k0 = 0;
    for (; k0 + 64 <= T; k0 += 64) chunk(k0, std::false_type{});
    if (k0 < T) chunk(k0, std::true_type{});

    const float inv = 1.0f / sum_halves(l_run);
    // Each whole 64-feature group leaves as full row lines: the pair of
    // 32-feature accumulator blocks is normalised, rounded, half-exchanged
    // (v_permlane32_swap) and regrouped (rows_to_lines), 8 lanes per row.
#pragma unroll
    for (int gi = 0; gi < G64; ++gi) {
      uint4 v[4];
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          uint32_t w[2][2];
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const f32x16& od = o[gi * 2 + jj];
            const int r0 = (2 * qh + h2) * 4;
            w[h2][0] = pack_bf16x2(od[r0 + 0] * inv, od[r0 + 1] * inv);
            w[h2][1] = pack_bf16x2(od[r0 + 2] * inv, od[r0 + 3] * inv);
          }
          const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
          const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
          v[2 * jj + qh] = make_uint4(s0[0], s1[0], s0[1], s1[1]);
        }
      rows_to_lines(v, lane);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int qq = qt * 32 + t * 8 + (lane >> 3);
        if (qq < T)
          st_global16(O + (seq0 + qq) * ldo + hoff + gi * 64 + (lane & 7) * 8, v[t]);
      }
    }
    // Blocks past the whole 64-feature groups: direct 8-byte stores.
    if (q < T) {
      bf16_t* orow = O + (seq0 + q) * ldo + hoff;
#pragma unroll
      for (int d = 2 * G64; d < C::DHP / 32; ++d)
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
}

template <int DH>
hipError_t launch_res(const void* q, const void* k, const void* v, int64_t ld, void* o,
                      int64_t ldo, int64_t N, int64_t T, int64_t H, hipStream_t s) {
  using C = ResCfg<DH>;
  const int64_t T_pad = (T + 31) / 32 * 32;
  const int64_t bytes = T_pad * C::ROW;
  if (bytes > kLdsBytes) return hipErrorNotSupported;
  static bool attr_set = false;
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&attn_resident_kernel<DH>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // clear it: the caller falls back to the streaming kernel
      return hipErrorNotSupported;
    }
    attr_set = true;
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
