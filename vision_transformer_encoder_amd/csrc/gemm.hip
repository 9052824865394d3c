// bf16 GEMM on the gfx950 matrix cores with fused epilogues.
//
// C = epi(A @ W) for activations A [M, K] (K contiguous) and a weight given
// out-major, Wt [N, K] (row n holds column n of W, K contiguous), fp32
// accumulation.  It carries the block's four products: the packed Q|K|V
// projection, the output projection + first residual, MLP1 + GELU and
// MLP2 + second residual (crackedaicode.com "ViT Encoder Block",
// "Multi-head attention" and "Feed-forward stage").
//
// Design (gfx950, wave64):
// * v_mfma_f32_32x32x16_bf16.  Each wave owns a (32*TN) x (32*TM) block of
//   C^T: the weight tile is the MFMA's first operand and the activation tile
//   its second, so every accumulator lane holds 4 consecutive output columns
//   of one row (8-byte stores).
// * Both tiles go straight from global memory into LDS with
//   buffer_load_dwordx4 ... lds (no staging registers): each load instruction
//   fills 1 KB of LDS, 16 bytes per lane at consecutive addresses.  The
//   buffer resource (SGPRs) points at the tile's first row, each lane keeps
//   one loop-invariant 32-bit offset per load, and the k offset is scalar.  LDS rows
//   are 64 k (128 B, 8 chunks of 16 B); the chunk index is XOR-swizzled by
//   (row >> 1) & 7, which each lane realises by choosing which global chunk
//   it fetches.  Eight consecutive lanes still read one contiguous 128-B row
//   segment of global memory, and each 16-lane phase of an MFMA operand read
//   covers all 64 banks once.
// * LDS stages: [A0 | A1 | B0 | B1].  A lane's fragment address differs
//   between k-steps only through its swizzled chunk, and between fragments
//   and stages by constants, so a wave keeps one address register per k-step
//   and per operand.
// * Loop: barrier (which also drains this thread's pending LDS loads), then
//   issue the loads of the next k-slice into the other stage, then 4 k-steps
//   of MFMAs on the current one: one barrier per 64-deep k-slice, and the
//   next slice's loads are in flight during the MFMAs.
// * Tile order: workgroups are dispatched round-robin over the 8 XCDs, so the
//   linear workgroup id is remapped to give each XCD a contiguous run of
//   tiles, walked in groups of 8 M-tiles so that the tiles resident at once
//   on an XCD share A and W panels in its L2.
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kBK = 64;     // k per LDS stage (8 chunks of 8 bf16)
constexpr int kGroupM = 8;  // M-tiles per raster group
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies
// Buffer resource word 3 for raw (untyped, stride 0) buffer access on CDNA.
constexpr int kBufferFlags = 0x00020000;

template <int BM_, int BN_, int WM_, int WN_, bool SCHED_ = true>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool SCHED = SCHED_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_LOADS = BM * 8 / NT;  // 16-B chunks per thread per k-slice
  static constexpr int B_LOADS = BN * 8 / NT;
  static constexpr int A_STAGE = BM * 128;     // bytes
  static constexpr int B_STAGE = BN * 128;
  static constexpr int LDS_BYTES = 2 * (A_STAGE + B_STAGE);
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "loads must divide evenly");
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 block");
};

// Linear workgroup id -> (m-tile, n-tile).
// LDS bank swizzle.  gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a
// time over 64 four-byte banks (256 B).  Rows are 128 B, so rows r and r+1
// already fall in different bank halves; XOR-ing the chunk index with
// (row >> 1) & 7 spreads any 16 consecutive rows over all 16 bank groups.
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }

// 16 bytes per lane from a raw buffer straight into LDS at dst + 16 * lane
// (dst must be wave-uniform).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst),
                                           16, voff, soff, 0, 0);
}

__device__ __forceinline__ void tile_of(int bid, int total, int mt, int nt, int* tm, int* tn) {
  const int q = total / kNumXcd, r = total % kNumXcd;
  const int x = bid % kNumXcd, local = bid / kNumXcd;
  const int t = x * q + (x < r ? x : r) + local;
  const int gsz = kGroupM * nt;
  const int first_m = (t / gsz) * kGroupM;
  const int gm = (mt - first_m) < kGroupM ? (mt - first_m) : kGroupM;
  const int w = t % gsz;
  *tm = first_m + w % gm;
  *tn = w / gm;
}

template <class C, int EPI>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16_kernel(GemmProblem p, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
  char* const a_lds = lds;                    // [stage][BM rows][128 B]
  char* const b_lds = lds + 2 * C::A_STAGE;   // [stage][BN rows][128 B]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  int tm, tn;
  tile_of(blockIdx.x, gridDim.x, mt, nt, &tm, &tn);
  const int64_t m0 = static_cast<int64_t>(tm) * C::BM, n0 = static_cast<int64_t>(tn) * C::BN;
  const int64_t M = p.M, N = p.N;

  // Buffer resources at the tiles' first rows, and per-lane byte offsets of
  // the chunks this thread loads (rows past M or N are clamped: their
  // products only reach outputs that are never stored).
  const __amdgpu_buffer_rsrc_t a_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(p.A) + m0 * p.lda * 2), 0, 0x7fffffff,
      kBufferFlags);
  const __amdgpu_buffer_rsrc_t b_rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(static_cast<const char*>(p.B) + n0 * p.ldb * 2), 0, 0x7fffffff,
      kBufferFlags);
  uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
#pragma unroll
  for (int i = 0; i < C::A_LOADS; ++i) {
    const int e = i * C::NT + tid, row = e >> 3, c = (e & 7) ^ swz_key(row);
    const int64_t r = (m0 + row < M) ? row : (M - 1 - m0);
    a_off[i] = static_cast<uint32_t>(r * p.lda * 2 + c * 16);
  }
#pragma unroll
  for (int i = 0; i < C::B_LOADS; ++i) {
    const int e = i * C::NT + tid, row = e >> 3, c = (e & 7) ^ swz_key(row);
    const int64_t r = (n0 + row < N) ? row : (N - 1 - n0);
    b_off[i] = static_cast<uint32_t>(r * p.ldb * 2 + c * 16);
  }
  auto issue = [&](int kt, int st) {
    const int kb = kt * kBK * 2;  // byte offset of the k-slice
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      load_lds16(a_rs, a_lds + st * C::A_STAGE + (i * C::NT + wave * 64) * 16, a_off[i], kb);
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      load_lds16(b_rs, b_lds + st * C::B_STAGE + (i * C::NT + wave * 64) * 16, b_off[i], kb);
  };

  // Fragment addresses: row (lane & 31) of the wave's first 32-row block,
  // logical chunk 2s + (lane >> 5), swizzled.
  const int lrow = lane & 31, lhalf = lane >> 5;
  int a_rd[4], b_rd[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int ch = ((2 * s + lhalf) ^ swz_key(lrow)) * 16;
    a_rd[s] = (wm * C::WTM + lrow) * 128 + ch;
    b_rd[s] = (wn * C::WTN + lrow) * 128 + ch;
  }

  f32x16 acc[C::TN][C::TM];
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  // Fragments of k-step s+1 are read from LDS while the MFMAs of k-step s
  // run; sched_group_barrier pins that interleaving (one LDS read after each
  // of the first MFMAs) so the reads' latency hides behind matrix work.
  auto read_frags = [&](const char* as, const char* bs, int s, bf16x8* af, bf16x8* bf) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(as + a_rd[s] + i * 32 * 128);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      bf[j] = *reinterpret_cast<const bf16x8*>(bs + b_rd[s] + j * 32 * 128);
  };
  auto compute = [&](int st) {
    const char* as = a_lds + st * C::A_STAGE;
    const char* bs = b_lds + st * C::B_STAGE;
    bf16x8 af[2][C::TM], bf[2][C::TN];
    read_frags(as, bs, 0, af[0], bf[0]);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) read_frags(as, bs, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s & 1][j], af[s & 1][i],
                                                              acc[j][i], 0, 0, 0);
      if (C::SCHED && s + 1 < 4) {
#pragma unroll
        for (int r = 0; r < C::TM + C::TN; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, C::TM * C::TN - C::TM - C::TN, 0);
      }
    }
  };

  const int KT = static_cast<int>(p.K / kBK);
  issue(0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();
    if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1);
    compute(kt & 1);
  }

  // Epilogue: accumulator element r of lane l in block (j, i) is
  // C[m0 + wm*WTM + i*32 + (l & 31)][n0 + wn*WTN + j*32 + (r/4)*8 + (l/32)*4 + r%4].
  bf16_t* Cp = static_cast<bf16_t*>(p.C);
  const bf16_t* Rp = static_cast<const bf16_t*>(p.R);
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int64_t m = m0 + wm * C::WTM + i * 32 + lrow;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t n = n0 + wn * C::WTN + j * 32 + rr * 8 + lhalf * 4;
        if (n >= N) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[j][i][rr * 4 + e];
        if (EPI == VITBLK_EPI_RESIDUAL) {
          const uint2 rv = *reinterpret_cast<const uint2*>(Rp + m * p.ldr + n);
          v[0] += __uint_as_float(rv.x << 16);
          v[1] += __uint_as_float(rv.x & 0xffff0000u);
          v[2] += __uint_as_float(rv.y << 16);
          v[3] += __uint_as_float(rv.y & 0xffff0000u);
        }
        if (EPI == VITBLK_EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_fast(v[e]);
        }
        *reinterpret_cast<uint2*>(Cp + m * p.ldc + n) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

using BigTile = Cfg<256, 256, 2, 4>;  // 8 waves (2 per SIMD), 128x64 per wave

template <class C>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t s) {
  const int64_t mt = (p.M + C::BM - 1) / C::BM, nt = (p.N + C::BN - 1) / C::BN;
  const int64_t blocks = mt * nt;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(C::NT);
  const int imt = static_cast<int>(mt), int_nt = static_cast<int>(nt);
  switch (p.epi) {
    case VITBLK_EPI_RESIDUAL:
      hipLaunchKernelGGL((gemm_bf16_kernel<C, VITBLK_EPI_RESIDUAL>), grid, block, 0, s, p, imt,
                         int_nt);
      break;
    case VITBLK_EPI_GELU:
      hipLaunchKernelGGL((gemm_bf16_kernel<C, VITBLK_EPI_GELU>), grid, block, 0, s, p, imt,
                         int_nt);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_kernel<C, VITBLK_EPI_NONE>), grid, block, 0, s, p, imt,
                         int_nt);
      break;
  }
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

// The MFMA kernel needs bf16, K a multiple of 64, N a multiple of 8, 16-byte
// aligned rows, and a 256-row panel of either operand to span < 2 GiB (its
// buffer offsets are 32-bit).  Everything else takes the generic kernel.
bool gemm_fast_ok(const GemmProblem& p) {
  bool ok = p.dtype == VITBLK_BF16 && p.K % kBK == 0 && p.N % 8 == 0 && p.N >= 8 &&
            p.lda % 8 == 0 && p.ldb % 8 == 0 && p.ldc % 8 == 0 && aligned16(p.A) &&
            aligned16(p.B) && aligned16(p.C) && p.lda * 2 * 256 < (1LL << 31) &&
            p.ldb * 2 * 256 < (1LL << 31) && p.K * 2 < (1LL << 31);
  if (p.epi == VITBLK_EPI_RESIDUAL) ok = ok && p.ldr % 8 == 0 && aligned16(p.R);
  return ok;
}

hipError_t launch_gemm(const GemmProblem& p, hipStream_t s) {
  if (!gemm_fast_ok(p)) return launch_gemm_generic(p, s);
  return launch_cfg<BigTile>(p, s);
}

}  // namespace vitblk
