// One 32-query tile of bidirectional attention on the gfx950 matrix cores:
// the pieces shared by the resident kernel (whole sequence's K/V in LDS) and
// the streaming kernel (64-key chunks through an LDS ring).
//
// O_h = softmax(Q_h K_h^T / sqrt(dh)) V_h for one head, no mask
// (crackedaicode.com "ViT Encoder Block", "Multi-head attention").
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16): scores are formed
// transposed, S^T = K Q^T, so each accumulator lane holds 16 keys of one
// query and the probabilities are already the second operand of
// O^T = V^T P^T.  V stays in its natural [key][feature] layout in LDS; its
// transpose is read with ds_read_b64_tr_b16, which hands lane i of a 16-lane
// group column i of the 4 x 16 block that the group's lanes point at (lane m
// points at row m/4, columns 4*(m%4)..+3).  LDS rows are padded so that both
// read patterns are conflict-free on gfx950 (64 banks): K rows (16
// consecutive keys x 16 B per read) use a stride of dh*2 + 16 bytes; V rows
// (4 consecutive keys x 64 B) a stride that is 64 or 192 modulo 256.
//
// Online softmax, per 64-key chunk: the reference maximum moves (and the
// accumulators are rescaled, for the whole wave at once) only when some
// query's maximum exceeds it by more than kSlack in log2 units; the
// probabilities are rounded once to bf16 (the PV operand) and their row sum
// is taken from those same rounded values with v_dot2c_f32_bf16.
#pragma once

#include <math.h>

#include "device.h"

namespace vitblk {
namespace attn {

typedef short v4i16 __attribute__((ext_vector_type(4)));

// Slack of the reference maximum, in log2 units (probabilities < 2^8).
constexpr float kSlack = 8.0f;
// bf16 pair (1, 1): a dot product with it sums a packed pair.
constexpr bf16x2_t kOnes = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

template <int DH>
struct Cfg {
  static_assert(DH % 16 == 0, "head width must be a multiple of 16");
  static constexpr int DHP = (DH + 31) / 32 * 32;                     // V^T rows per MFMA block
  static constexpr int SK = DH * 2 + 16;                              // K row stride, bytes
  static constexpr int SV = (DHP * 2) % 128 == 0 ? DHP * 2 + 64 : DHP * 2;  // V row stride
  static constexpr int ROW = SK + SV;
  static constexpr int G64 = DH / 64;  // whole 64-feature groups of a head
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

// Q fragments of a 32-query tile: lane (l & 31, g = l >> 5) holds features
// 16s + 8g .. +7 of query q0 + (l & 31) (clamped to T - 1), s = 0 .. DH/16-1.
// Each whole 64-feature group is read as full 128-byte row lines (8 lanes per
// query row) into qv and later regrouped into that layout (finish); the rest
// (DH % 64) is read in the fragment layout directly.
template <int DH>
struct QLoad {
  bf16x8 qf[DH / 16];
  uint4 qv[Cfg<DH>::G64 > 0 ? Cfg<DH>::G64 : 1][4];

  __device__ __forceinline__ void issue(const bf16_t* Q, int64_t ld, int64_t seq0, int64_t hoff,
                                        int T, int q0, int lane) {
#pragma unroll
    for (int gi = 0; gi < Cfg<DH>::G64; ++gi)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int qq = q0 + t * 8 + (lane >> 3);
        qv[gi][t] = ld_global16(Q + (seq0 + (qq < T ? qq : T - 1)) * ld + hoff + gi * 64 +
                                (lane & 7) * 8);
      }
    const int q = q0 + (lane & 31);
    const bf16_t* qrow = Q + (seq0 + (q < T ? q : T - 1)) * ld + hoff + (lane >> 5) * 8;
#pragma unroll
    for (int s = Cfg<DH>::G64 * 4; s < DH / 16; ++s)
      qf[s] = __builtin_bit_cast(bf16x8, ld_global16(qrow + s * 16));
  }
  __device__ __forceinline__ void finish(int lane) {
#pragma unroll
    for (int gi = 0; gi < Cfg<DH>::G64; ++gi) {
      lines_to_rows(qv[gi], lane);
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[gi * 4 + s] = __builtin_bit_cast(bf16x8, qv[gi][s]);
    }
  }
};

// Running state of one query tile.  m_run: the reference maximum (log2
// units) the probabilities are taken against; l_run: this lane's share of
// their sum (the other lane half holds the rest of the query's keys).
template <int DH>
struct Tile {
  f32x16 o[Cfg<DH>::DHP / 32];
  float m_run, l_run;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int d = 0; d < Cfg<DH>::DHP / 32; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[d][r] = 0.f;
    m_run = -INFINITY;
    l_run = 0.f;
  }

  // One chunk of 64 keys whose K rows start at kc and V rows at vc in LDS;
  // nvalid (>= 1) of them are real keys.  TAIL: nvalid < 64 (keys past it
  // get score -inf, and a second 32-key block with no real key is skipped).
  // v_lane: this lane's V^T read offset within a 4-key x 32-feature block.
  template <bool TAIL>
  __device__ __forceinline__ void chunk(const bf16x8* qf, const char* kc, const char* vc,
                                        int nvalid, float scale_log2, int lane, int v_lane) {
    using C = Cfg<DH>;
    const int lrow = lane & 31, g = lane >> 5;
    const int nkb = (!TAIL || nvalid > 32) ? 2 : 1;  // 32-key blocks holding a valid key
    f32x16 sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb < nkb) {
        const char* krow = kc + (kb * 32 + lrow) * C::SK + g * 16;
        sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(krow),
                                                         qf[0], f32x16{}, 0, 0, 0);
#pragma unroll
        for (int ks_ = 1; ks_ < DH / 16; ++ks_) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + ks_ * 32);
          sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks_], sc[kb], 0, 0, 0);
        }
      }
    }
    // Maximum of the raw scores.  Key kb*32 + (r/4)*8 + g*4 + r%4 of the
    // chunk is valid iff it is < nvalid.
    float mx = -INFINITY;
    if (TAIL) {
      const int lim = nvalid - g * 4;
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
    // p = 2^(s * scale * log2(e) - m), rounded once to bf16.
    uint32_t pk[2][8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (kb >= nkb) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pk[kb][e] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sc[kb][2 * e], scale_log2, -m_run)),
                                __builtin_amdgcn_exp2f(fmaf(sc[kb][2 * e + 1], scale_log2, -m_run)));
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[kb][e]), kOnes,
                                                l_run, false);
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
        const char* vb = vc + (kb * 32 + s2 * 16 + g * 4) * C::SV + v_lane;
#pragma unroll
        for (int d = 0; d < C::DHP / 32; ++d) {
          const v4i16 lo = ds_read_tr16(vb + d * 64);
          const v4i16 hi = ds_read_tr16(vb + 8 * C::SV + d * 64);
          const bf16x8 vf =
              __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          o[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[d], 0, 0, 0);
        }
      }
    }
  }

  // O rows q0 .. q0+31 (those < T): each whole 64-feature group leaves as
  // full row lines (the pair of 32-feature accumulator blocks is normalised,
  // rounded, half-exchanged with v_permlane32_swap and regrouped with
  // rows_to_lines, 8 lanes per row); blocks past them as 8-byte stores.
  __device__ __forceinline__ void store(bf16_t* O, int64_t ldo, int64_t seq0, int64_t hoff, int T,
                                        int q0, int lane) {
    using C = Cfg<DH>;
    const int g = lane >> 5;
    const float inv = 1.0f / sum_halves(l_run);
#pragma unroll
    for (int gi = 0; gi < C::G64; ++gi) {
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
        const int qq = q0 + t * 8 + (lane >> 3);
        if (qq < T) st_global16(O + (seq0 + qq) * ldo + hoff + gi * 64 + (lane & 7) * 8, v[t]);
      }
    }
    const int q = q0 + (lane & 31);
    if (q < T) {
      bf16_t* orow = O + (seq0 + q) * ldo + hoff;
#pragma unroll
      for (int d = 2 * C::G64; d < C::DHP / 32; ++d)
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
};

// This lane's V^T read offset (bytes) relative to (first key, feature block):
// row (i16 / 4), columns q16*16 + 4*(i16 % 4) of the 32-feature block, for
// i16 = lane % 16 and q16 = (lane / 16) % 2.
template <int DH>
__device__ __forceinline__ int v_lane_offset(int lane) {
  const int i16 = lane & 15, q16 = (lane >> 4) & 1;
  return (i16 >> 2) * Cfg<DH>::SV + (q16 * 16 + 4 * (i16 & 3)) * 2;
}

}  // namespace attn
}  // namespace vitblk
