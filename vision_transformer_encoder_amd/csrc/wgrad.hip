// Weight gradients on the gfx950 matrix cores: C[i, j] = sum_m A[m, i] B[m, j]
// over the token rows m, for every projection of the block's backward
// (dW = input^T * output-gradient; the exact derivative of the forward
// definition on crackedaicode.com "ViT Encoder Block", the parameter
// gradients of nipunbatra.github.io vision1 transcript, Pages 88 and 113).
//
// Both operands are token-major ([M, I] and [M, J], feature axis
// contiguous), so the reduction runs down the rows.  Design (wave64):
// * Tiles of BK token rows go straight from global memory into LDS with
//   buffer_load_dwordx4 ... lds, keeping their [token][feature] layout: a
//   load instruction moves 2 rows of 512 B, so global reads are contiguous.
// * v_mfma_f32_32x32x16_bf16 wants, in each lane, 8 consecutive k (= token)
//   values of one feature.  ds_read_b64_tr_b16 returns exactly that from
//   the [token][feature] layout: lane i of a 16-lane group receives feature
//   i of the 4 x 16 block the group points at (lane m points at row m / 4,
//   features 4 (m % 4) .. + 3); two such reads give a lane its 8 tokens.
// * Bank conflicts: a half-wave's tr read touches 4 rows x 64 B.  Rows are
//   512 B (a multiple of the 256-B bank period), so the 16-byte chunk index
//   is XOR-ed with 4 * (row % 4): the 4 rows then cover all 64 banks once.
//   Each lane realises the swizzle by choosing which global chunk it fetches.
// * Each wave owns a 64 (j) x 128 (i) block of C^T: the B tile is the MFMA's
//   first operand, so an accumulator lane holds 4 consecutive j of one i and
//   writes them as one 16-byte fp32 store.
// * Work split: the output is cut into 256 x 256 tiles and the token rows
//   into `split` ranges (a multiple of BK rows each); one workgroup per
//   (range, tile) writes that range's fp32 partial.  Workgroups are mapped
//   so that the tiles of one range sit on one XCD (the hardware deals
//   workgroups round-robin over the 8 XCDs) and share its L2.  A separate
//   kernel sums the partials in order.
// * k pipeline as in the forward GEMM: 3 A stages and 2 B stages (160 KB),
//   the A slice issued two slices ahead, B one, one wait + barrier per slice.
//   The LDS DMA is issued from inline assembly: the compiler does not see it
//   as a write to LDS, so it does not wait for it before every transposing
//   read; the explicit vmcnt waits and barriers order them instead.
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kXcd = 8;
constexpr int kBufferFlags = 0x00020000;  // raw buffer access, word 3

constexpr int BI = 256, BJ = 256, BK = 64;
constexpr int WI = 2, WJ = 4;              // waves along i and j
constexpr int NT = WI * WJ * 64;           // 512 threads
constexpr int WTI = BI / WI, WTJ = BJ / WJ;  // 128 x 64 per wave
constexpr int TI = WTI / 32, TJ = WTJ / 32;  // 4 x 2 MFMA blocks
constexpr int ROW_BYTES = BI * 2;          // 512 B per LDS row (both operands)
constexpr int CPR = ROW_BYTES / 16;        // 32 chunks per row
constexpr int STAGE = BK * ROW_BYTES;      // 32 KB
constexpr int NSA = 3, NSB = 2;
constexpr int LDS_BYTES = (NSA + NSB) * STAGE;  // 160 KB
constexpr int LOADS = BK * CPR / NT;       // 4 chunks per thread per operand and slice
static_assert(BJ * 2 == ROW_BYTES, "A and B rows have the same width");
static_assert(LDS_BYTES <= 160 * 1024, "LDS");

typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int swz(int row) { return (row & 3) << 2; }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff,
                                           kBufferFlags);
}

// 16 bytes per lane into LDS at dst + 16 * lane (dst wave-uniform), through M0.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, const char* dst, uint32_t voff,
                                      int soff) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(dst)));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(m0)), "v"(voff), "s"(rs), "s"(soff)
      : "memory", "m0");
}

__device__ __forceinline__ v4i16 ds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<char*>(p)));
}

struct WgradArgs {
  const bf16_t* A;
  const bf16_t* B;
  int64_t lda, ldb;
  int64_t I, J;
  int64_t rows_per_split;  // multiple of BK
  int64_t rows;            // token rows handled here (a multiple of BK)
  int ti, tj, splits;      // tile grid and ranges
  float* partial;          // [splits][I][J]
};

__global__ __launch_bounds__(NT, 1) void wgrad_mfma_kernel(WgradArgs p) {
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  char* const a_lds = lds;
  char* const b_lds = lds + NSA * STAGE;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wi = wave / WJ, wj = wave % WJ;

  // Work item: the tiles of one token range are consecutive and land on one XCD.
  const int G = gridDim.x, b = blockIdx.x;
  const int logical = (G % kXcd == 0) ? (b % kXcd) * (G / kXcd) + b / kXcd : b;
  const int tiles = p.ti * p.tj;
  const int range = logical / tiles, tile = logical % tiles;
  const int64_t i0 = static_cast<int64_t>(tile / p.tj) * BI;
  const int64_t j0 = static_cast<int64_t>(tile % p.tj) * BJ;
  const int64_t m_lo = range * p.rows_per_split;
  const int64_t m_hi = m_lo + p.rows_per_split < p.rows ? m_lo + p.rows_per_split : p.rows;
  const int KT = static_cast<int>((m_hi - m_lo) / BK);

  const __amdgpu_buffer_rsrc_t a_rs = make_rsrc(p.A + m_lo * p.lda + i0);
  const __amdgpu_buffer_rsrc_t b_rs = make_rsrc(p.B + m_lo * p.ldb + j0);
  // Per-lane byte offsets of its chunks within a slice (chunks past the
  // feature range are clamped to the last valid chunk: their products reach
  // only outputs that are never stored).
  // Waves 0..3 (one per SIMD) issue every global->LDS load, their own chunks
  // and those of wave + 4; waves 4..7 issue none, so each SIMD always has a
  // wave that is not stalled on LDS-DMA issue and keeps the matrix core busy.
  constexpr int HW = NT / 128;
  const bool loader = wave < HW;
  uint32_t a_off[2 * LOADS], b_off[2 * LOADS];
  const int a_last = static_cast<int>((p.I - i0 < BI ? p.I - i0 : BI) / 8) - 1;
  const int b_last = static_cast<int>((p.J - j0 < BJ ? p.J - j0 : BJ) / 8) - 1;
#pragma unroll
  for (int u = 0; u < 2 * LOADS; ++u) {
    const int e = (u % LOADS) * NT + tid + (u / LOADS) * HW * 64, row = e / CPR;
    const int c = (e % CPR) ^ swz(row);
    a_off[u] = static_cast<uint32_t>(row * p.lda * 2 + (c < a_last ? c : a_last) * 16);
    b_off[u] = static_cast<uint32_t>(row * p.ldb * 2 + (c < b_last ? c : b_last) * 16);
  }
  const int a_step = static_cast<int>(BK * p.lda * 2);  // bytes per slice
  const int b_step = static_cast<int>(BK * p.ldb * 2);
  auto issue_a = [&](int kt, int st) {
    if (!loader) return;
#pragma unroll
    for (int u = 0; u < 2 * LOADS; ++u)
      dma16(a_rs, a_lds + st * STAGE + ((u % LOADS) * NT + (wave + (u / LOADS) * HW) * 64) * 16,
            a_off[u], kt * a_step);
  };
  auto issue_b = [&](int kt, int st) {
    if (!loader) return;
#pragma unroll
    for (int u = 0; u < 2 * LOADS; ++u)
      dma16(b_rs, b_lds + st * STAGE + ((u % LOADS) * NT + (wave + (u / LOADS) * HW) * 64) * 16,
            b_off[u], kt * b_step);
  };

  // Fragment read offsets.  For MFMA block `blk` of a wave tile starting at
  // feature cb, k-step s and half h (tokens s*16 + g*8 + 4h + 0..3), lane
  // (g, q16, i16) reads row s*16 + g*8 + 4h + i16/4, features
  // cb + blk*32 + q16*16 + 4*(i16 % 4) .. + 3.
  const int g = lane >> 5, q16 = (lane >> 4) & 1, i16 = lane & 15;
  auto frag_off = [&](int cb, int blk) {
    const int L = (cb + blk * 32 + q16 * 16 + 4 * (i16 & 3)) >> 3;
    const int row = g * 8 + (i16 >> 2);
    return row * ROW_BYTES + (L ^ swz(row)) * 16 + (i16 & 1) * 8;
  };
  int a_rd[TI], b_rd[TJ];
#pragma unroll
  for (int t = 0; t < TI; ++t) a_rd[t] = frag_off(wi * WTI, t);
#pragma unroll
  for (int t = 0; t < TJ; ++t) b_rd[t] = frag_off(wj * WTJ, t);

  f32x16 acc[TJ][TI];
#pragma unroll
  for (int j = 0; j < TJ; ++j)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  auto frag = [&](const char* base, int off, int s) {
    const v4i16 lo = ds_read_tr16(base + off + s * 16 * ROW_BYTES);
    const v4i16 hi = ds_read_tr16(base + off + s * 16 * ROW_BYTES + 4 * ROW_BYTES);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  if (KT > 0) {
    issue_a(0, 0);
    issue_b(0, 0);
    if (1 < KT) issue_a(1, 1);
  }
  for (int kt = 0; kt < KT; ++kt) {
    // Issue order: W(kt+1) then A(kt+2) per iteration, so at the top of
    // iteration kt only A(kt+1) (2 * LOADS per loading wave) is newer than
    // slice kt's loads.
    if (kt > 0 && kt + 1 < KT)
      wait_vmcnt<2 * LOADS>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    const char* as = a_lds + (kt % NSA) * STAGE;
    const char* bs = b_lds + (kt % NSB) * STAGE;
    bf16x8 af[2][TI], bf[2][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i) af[0][i] = frag(as, a_rd[i], 0);
#pragma unroll
    for (int j = 0; j < TJ; ++j) bf[0][j] = frag(bs, b_rd[j], 0);
    if (kt + 1 < KT) issue_b(kt + 1, (kt + 1) % NSB);
    if (kt + 2 < KT) issue_a(kt + 2, (kt + 2) % NSA);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      if (s + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TI; ++i) af[(s + 1) & 1][i] = frag(as, a_rd[i], s + 1);
#pragma unroll
        for (int j = 0; j < TJ; ++j) bf[(s + 1) & 1][j] = frag(bs, b_rd[j], s + 1);
      }
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int i = 0; i < TI; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s & 1][j], af[s & 1][i],
                                                              acc[j][i], 0, 0, 0);
    }
  }

  // acc[j][i][r] = C[i0 + wi*WTI + i*32 + (lane & 31)]
  //                 [j0 + wj*WTJ + j*32 + (r/4)*8 + (lane/32)*4 + r%4]
  float* out = p.partial + static_cast<int64_t>(range) * p.I * p.J;
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int64_t gi = i0 + wi * WTI + i * 32 + (lane & 31);
    if (gi >= p.I) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t gj = j0 + wj * WTJ + j * 32 + q * 8 + g * 4;
        if (gj < p.J)
          *reinterpret_cast<float4*>(out + gi * p.J + gj) =
              make_float4(acc[j][i][q * 4 + 0], acc[j][i][q * 4 + 1], acc[j][i][q * 4 + 2],
                          acc[j][i][q * 4 + 3]);
      }
  }
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

// The matrix-core path: bf16, feature counts and row strides multiples of 8,
// 16-byte aligned operands, at least one BK-row slice, and every range's
// byte offsets within the 32-bit buffer offsets.  Returns the number of
// token rows it covers (a multiple of BK; the caller reduces the rest), or
// 0 when the problem does not qualify (nothing launched).
int64_t wgrad_mfma_rows(const WgradProblem& p, int split) {
  if (p.dtype != VITBLK_BF16 || p.I % 8 != 0 || p.J % 8 != 0 || p.lda % 8 != 0 ||
      p.ldb % 8 != 0 || !aligned16(p.A) || !aligned16(p.B) || p.M < BK || split < 1)
    return 0;
  const int64_t rows = p.M / BK * BK;
  const int64_t per = ((rows + split - 1) / split + BK - 1) / BK * BK;
  const int64_t span_a = (per + BK) * p.lda * 2, span_b = (per + BK) * p.ldb * 2;
  if (span_a >= (1LL << 31) || span_b >= (1LL << 31)) return 0;
  return rows;
}

hipError_t launch_wgrad_mfma(const WgradProblem& p, float* partial, int split, int* used,
                             hipStream_t s) {
  const int64_t rows = wgrad_mfma_rows(p, split);
  if (rows == 0) return hipErrorNotSupported;
  const int64_t per = ((rows + split - 1) / split + BK - 1) / BK * BK;
  const int ranges = static_cast<int>((rows + per - 1) / per);
  const int ti = static_cast<int>((p.I + BI - 1) / BI), tj = static_cast<int>((p.J + BJ - 1) / BJ);
  const int64_t blocks = static_cast<int64_t>(ti) * tj * ranges;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  WgradArgs a;
  a.A = static_cast<const bf16_t*>(p.A);
  a.B = static_cast<const bf16_t*>(p.B);
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.I = p.I;
  a.J = p.J;
  a.rows_per_split = per;
  a.rows = rows;
  a.ti = ti;
  a.tj = tj;
  a.splits = ranges;
  a.partial = partial;
  hipLaunchKernelGGL(wgrad_mfma_kernel, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0, s, a);
  *used = ranges;
  return hipGetLastError();
}

}  // namespace vitblk
