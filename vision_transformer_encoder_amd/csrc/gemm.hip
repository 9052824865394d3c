// bf16 GEMM on the gfx950 matrix cores with fused epilogues.
//
// C = epi(A @ W) for activations A [M, K] (K contiguous) and a weight given
// out-major, Wt [N, K] (row n holds column n of W, K contiguous), fp32
// accumulation.  It carries the block's four products: the packed Q|K|V
// projection, the output projection + first residual, MLP1 + GELU and
// MLP2 + second residual (crackedaicode.com "ViT Encoder Block",
// "Multi-head attention" and "Feed-forward stage"); also the backward's
// data-gradient products and the patch embedding (whose token-row epilogue
// writes each product row into its token row with the position embedding
// added, kEpiEmbed).
//
// Design (gfx950, wave64):
// * v_mfma_f32_32x32x16_bf16.  Each wave owns a (32*TN) x (32*TM) block of
//   C^T: the weight tile is the MFMA's first operand and the activation tile
//   its second, so every accumulator lane holds 4 consecutive output columns
//   of one row; lanes l and l+32 swap halves so each lane stores 16 bytes.
// * Both tiles go straight from global memory into LDS with
//   buffer_load_dwordx4 ... lds (no staging registers): each load instruction
//   fills 1 KB of LDS, 16 bytes per lane at consecutive addresses.  In the
//   256x256 tile only one wave per SIMD issues them (see kSpec).  The
//   buffer resource (SGPRs) points at the tile's first row, each lane keeps
//   one 32-bit offset per load, and the k offset is scalar.  LDS rows are
//   BK k-values; the 16-byte chunk index is XOR-swizzled per row (see
//   swz_key), which each lane realises by choosing which global chunk it
//   fetches, so global reads stay row-contiguous and each 16-lane phase of
//   an MFMA operand read covers all 64 banks once.
// * LDS stages: [A stages | B stages].  A lane's fragment address differs
//   between k-steps only through its swizzled chunk, and between fragments
//   and stages by constants, so a wave keeps one address register per k-step
//   and per operand.
// * k pipeline: NS - 1 k-slices in flight; one s_waitcnt + s_barrier per
//   slice, the next slices' loads issued right after the slice's first
//   fragment reads.  With
//   NSA = 3 A stages (and NS = 2 W stages) the activation slice, the operand
//   that misses L2 most, is issued two slices ahead and the weight slice one.
// * Persistent: the grid is the number of workgroups the device holds at
//   once and each workgroup walks tiles b, b + G, ...  The next tile's first
//   k-slices are issued before the current tile's epilogue, so the load
//   latency at a tile start overlaps the stores of the previous tile, and the
//   epilogue issues all residual loads before its first store.
// * Epilogue reads (residual) are issued before the next tile's first
//   k-slices: loads complete in issue order, so a read issued after them
//   would hold the epilogue until those slices had landed.  A bias is no
//   epilogue work at all: the accumulators start at it (fp32; the products
//   are then added to it), or with the LayerNorm fold the epilogue's rstd
//   scale adds it in the same fma (below).
// * LayerNorm fold (row_stats set): LN(A) @ W = rstd (A @ W - mean colsum W)
//   (crackedaicode.com "ViT Encoder Block", "Normalize before each stage":
//   (x - mean) * rstd per token, multiplied out).  The accumulators start at
//   -mean_m colsum_n instead of 0 and the epilogue scales by rstd_m, so LN's
//   output never goes through memory.
// * Split K (kEpiPartial): the tile index also runs over k-ranges whose
//   unrounded fp32 sums are written out; a second kernel adds them in order.
// * Tiles: 256x256 (8 waves, the default), 192x256 (8 waves, when a product
//   has fewer big tiles than CUs and these fit in one round), 128x128 (4
//   waves, two workgroups per CU: the output projection and the rows past
//   the big tile's whole rounds) and its four-stage variant (one per CU,
//   for a last partial round); launch_gemm chooses.
// * Tile order: workgroups are dispatched round-robin over the 8 XCDs; each
//   XCD is given a contiguous run of tiles per round, walked in groups of 8
//   M-tiles so that the tiles resident at once on an XCD share A and W
//   panels in its L2.
#include <atomic>

#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kGroupM = 8;  // M-tiles per raster group
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies
// Buffer resource word 3 for raw (untyped, stride 0) buffer access on CDNA.
constexpr int kBufferFlags = 0x00020000;

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int NS_ = 2, int NSA_ = NS_,
          bool SCHED_ = true, int WPE_ = 1>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int BK = BK_;    // k per LDS stage
  static constexpr int NS = NS_;    // LDS stages of W (k-slices in flight: NS - 1)
  // LDS stages of A.  NSA = NS + 1 gives the activation operand, whose panels
  // miss L2 far more often than the weights', one more k-slice of lead.
  static constexpr int NSA = NSA_;
  static constexpr bool SCHED = SCHED_;
  static constexpr int WPE = WPE_;  // launch bound: waves per SIMD the registers must allow
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int CPR = BK / 8;                // 16-byte chunks per LDS row
  static constexpr int KSTEPS = BK / 16;            // MFMA k-steps per stage
  static constexpr int A_LOADS = BM * CPR / NT;     // 16-B chunks per thread per k-slice
  static constexpr int B_LOADS = BN * CPR / NT;
  static constexpr int A_STAGE = BM * BK * 2;       // bytes
  static constexpr int B_STAGE = BN * BK * 2;
  static constexpr int LDS_BYTES = NSA * A_STAGE + NS * B_STAGE;
  static_assert(NSA == NS || (NSA == 3 && NS == 2), "A stages: NS, or 3 with NS = 2");
  static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
  static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
  static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "loads must divide evenly");
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 block");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
};

// LDS bank swizzle.  gfx950 serves a 16-byte-per-lane LDS read 16 lanes at a
// time over 64 four-byte banks (256 B).  A row holds CPR chunks of 16 B, so
// 16/CPR consecutive rows fill one 256-B bank row; XOR-ing the chunk index
// with (row / (16/CPR)) % CPR spreads any 16 consecutive rows (one MFMA
// operand read phase) over all 16 bank groups.
template <int CPR>
__device__ __forceinline__ int swz_key(int row) { return (row / (16 / CPR)) % CPR; }

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// 16 bytes per lane from a raw buffer straight into LDS at dst + 16 * lane
// (dst must be wave-uniform).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff,
                                           int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst),
                                           16, voff, soff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff,
                                           kBufferFlags);
}

// Persistent tile order.  Workgroup b processes tiles b, b + G, b + 2G, ...
// The hardware places workgroup b on XCD b % 8, so within each full round of
// G tiles (G a multiple of 8) the XCD-x workgroups get the contiguous logical
// run [rG + x*G/8, rG + (x+1)*G/8); a partial last round keeps t.  Logical
// tiles are walked in groups of kGroupM M-tiles, n fastest within a group.
__device__ __forceinline__ void tile_of(int t, int grid, int total, int mt, int nt, int* tm,
                                        int* tn) {
  const int r = t / grid, b = t - r * grid;
  int logical = t;
  if ((grid % kNumXcd) == 0 && (r + 1) * grid <= total)
    logical = r * grid + (b % kNumXcd) * (grid / kNumXcd) + b / kNumXcd;
  const int gsz = kGroupM * nt;
  const int first_m = (logical / gsz) * kGroupM;
  const int gm = (mt - first_m) < kGroupM ? (mt - first_m) : kGroupM;
  const int w = logical % gsz;
  *tm = first_m + w % gm;
  *tn = w / gm;
}

template <class C, int EPI, bool BIAS, bool NORM>
__global__ __launch_bounds__(C::NT, C::WPE) void gemm_bf16_kernel(GemmProblem p, int mt, int nt) {
  __shared__ __attribute__((aligned(1024))) char lds[C::LDS_BYTES];
  char* const a_lds = lds;                       // [stage][BM rows][BK * 2 B]
  char* const b_lds = lds + C::NSA * C::A_STAGE;  // [stage][BN rows][BK * 2 B]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / C::WN, wn = wave % C::WN;
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int64_t M = p.M, N = p.N;
  // kEpiEmbed: product row m = first + delta (first: the first row of a
  // wave's 32-row block, whose quotient and remainder by row_group, q0 and r0,
  // are taken once per block) goes to C row g + row_skip * (g / row_group + 1)
  // and reads R row row_skip + g % row_group, g = row_base + m (32-bit: the
  // launcher keeps row_base + M below 2^31).  Other epilogues: row m itself.
  auto c_row = [&](int64_t m, uint32_t q0, uint32_t r0, int delta) -> int64_t {
    if (EPI != kEpiEmbed) return m;
    const uint32_t n32 = static_cast<uint32_t>(p.row_group);
    uint32_t idx = r0 + static_cast<uint32_t>(delta), q = q0;
    while (idx >= n32) {  // delta < 32: at most 32 / row_group + 1 steps
      idx -= n32;
      ++q;
    }
    return p.row_base + m + p.row_skip * static_cast<int64_t>(q + 1);
  };
  auto r_row = [&](int64_t m, uint32_t r0, int delta) -> int64_t {
    if (EPI != kEpiEmbed) return m;
    const uint32_t n32 = static_cast<uint32_t>(p.row_group);
    uint32_t idx = r0 + static_cast<uint32_t>(delta);
    while (idx >= n32) idx -= n32;
    return p.row_skip + static_cast<int64_t>(idx);
  };
  // q0, r0 of the 32-row block starting at product row first.
  auto block_div = [&](int64_t first, uint32_t* q0, uint32_t* r0) {
    if (EPI != kEpiEmbed) return;
    const uint32_t g = static_cast<uint32_t>(p.row_base + first);
    const uint32_t n32 = static_cast<uint32_t>(p.row_group);
    *q0 = g / n32;
    *r0 = g - *q0 * n32;
  };
  // Split K (kEpiPartial): the tile index runs over ksplit copies of the
  // mt x nt tiles, copy s covering k-slices [KA * s / ksplit, KA * (s + 1) /
  // ksplit).  Otherwise one copy and the whole of K.
  constexpr bool kSplit = EPI == kEpiPartial;
  const int KA = static_cast<int>(p.K / C::BK);
  const int nsplit = kSplit ? p.ksplit : 1;
  int KT = KA;
  int ks = 0;  // k-range of the current tile
  // Odd rounds walk the k-slices backwards: a tile then starts on the slices
  // its XCD's L2 touched last (the weight panels repeat from round to round).
  bool krev = false;
  const int total = mt * nt * nsplit, grid = gridDim.x;

  // Tile-dependent load state: buffer resources at the tiles' first rows and
  // per-lane byte offsets of the chunks this thread loads (rows past M or N
  // are clamped: their products only reach outputs that are never stored).
  int64_t m0 = 0, n0 = 0;
  __amdgpu_buffer_rsrc_t a_rs, b_rs;
  uint32_t a_off[C::A_LOADS], b_off[C::B_LOADS];
  // 8-wave tiles: the waves of the first half (one per SIMD) issue every
  // global->LDS load, their own chunks and those of wave + NT/128; the second
  // half issue none.  A wave stalls while its LDS-DMA loads are accepted, so
  // with every wave loading, both waves of a SIMD stalled together after each
  // barrier and the matrix core idled; this way the other wave keeps issuing
  // MFMAs meanwhile (measured: MLP1 444.7 -> 422.3 us, Q|K|V 311.4 -> 295.0
  // us at ViT-L/16).
  constexpr bool kSpec = C::NSA > C::NS && C::NT == 512;
  constexpr int HW = C::NT / 128;  // waves per half
  uint32_t a_off2[kSpec ? C::A_LOADS : 1], b_off2[kSpec ? C::B_LOADS : 1];
  auto prepare = [&](int t) {
    int tm, tn;
    tile_of(t, grid, total, mt * nsplit, nt, &tm, &tn);
    krev = ((t / grid) & 1) != 0;
    int64_t kbyte = 0;
    if (kSplit) {
      // The k-ranges are laid out as further M-tiles of the tile order.
      ks = tm / mt;
      tm -= ks * mt;
      const int k0 = KA * ks / nsplit, k1 = KA * (ks + 1) / nsplit;
      KT = k1 - k0;
      kbyte = static_cast<int64_t>(k0) * C::BK * 2;
    }
    m0 = static_cast<int64_t>(tm) * C::BM;
    n0 = static_cast<int64_t>(tn) * C::BN;
    a_rs = make_rsrc(static_cast<const char*>(p.A) + m0 * p.lda * 2 + kbyte);
    b_rs = make_rsrc(static_cast<const char*>(p.B) + n0 * p.ldb * 2 + kbyte);
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i) {
      const int e = i * C::NT + tid, row = e / C::CPR;
      const int c = (e % C::CPR) ^ swz_key<C::CPR>(row);
      const int64_t r = (m0 + row < M) ? row : (M - 1 - m0);
      a_off[i] = static_cast<uint32_t>(r * p.lda * 2 + c * 16);
      if (kSpec) {
        const int e2 = e + HW * 64, row2 = e2 / C::CPR;
        const int c2 = (e2 % C::CPR) ^ swz_key<C::CPR>(row2);
        const int64_t r2 = (m0 + row2 < M) ? row2 : (M - 1 - m0);
        a_off2[kSpec ? i : 0] = static_cast<uint32_t>(r2 * p.lda * 2 + c2 * 16);
      }
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i) {
      const int e = i * C::NT + tid, row = e / C::CPR;
      const int c = (e % C::CPR) ^ swz_key<C::CPR>(row);
      const int64_t r = (n0 + row < N) ? row : (N - 1 - n0);
      b_off[i] = static_cast<uint32_t>(r * p.ldb * 2 + c * 16);
      if (kSpec) {
        const int e2 = e + HW * 64, row2 = e2 / C::CPR;
        const int c2 = (e2 % C::CPR) ^ swz_key<C::CPR>(row2);
        const int64_t r2 = (n0 + row2 < N) ? row2 : (N - 1 - n0);
        b_off2[kSpec ? i : 0] = static_cast<uint32_t>(r2 * p.ldb * 2 + c2 * 16);
      }
    }
  };
  auto issue_a = [&](int kt, int st) {
    const int kb = (krev ? KT - 1 - kt : kt) * C::BK * 2;  // byte offset of the k-slice
    if (kSpec) {
      if (wave < HW) {
#pragma unroll
        for (int i = 0; i < C::A_LOADS; ++i) {
          load_lds16(a_rs, a_lds + st * C::A_STAGE + (i * C::NT + wave * 64) * 16, a_off[i], kb);
          load_lds16(a_rs, a_lds + st * C::A_STAGE + (i * C::NT + (wave + HW) * 64) * 16,
                     a_off2[kSpec ? i : 0], kb);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::A_LOADS; ++i)
      load_lds16(a_rs, a_lds + st * C::A_STAGE + (i * C::NT + wave * 64) * 16, a_off[i], kb);
  };
  auto issue_b = [&](int kt, int st) {
    const int kb = (krev ? KT - 1 - kt : kt) * C::BK * 2;
    if (kSpec) {
      if (wave < HW) {
#pragma unroll
        for (int i = 0; i < C::B_LOADS; ++i) {
          load_lds16(b_rs, b_lds + st * C::B_STAGE + (i * C::NT + wave * 64) * 16, b_off[i], kb);
          load_lds16(b_rs, b_lds + st * C::B_STAGE + (i * C::NT + (wave + HW) * 64) * 16,
                     b_off2[kSpec ? i : 0], kb);
        }
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < C::B_LOADS; ++i)
      load_lds16(b_rs, b_lds + st * C::B_STAGE + (i * C::NT + wave * 64) * 16, b_off[i], kb);
  };
  auto issue = [&](int kt, int st) {
    issue_a(kt, st);
    issue_b(kt, st);
  };
  // Start of a tile: the first k-slices in flight (A(0), W(0) [, A(1)]).
  auto start_tile = [&]() {
    if (C::NSA > C::NS) {
      issue_a(0, 0);
      issue_b(0, 0);
      if (1 < KT) issue_a(1, 1);
    } else {
#pragma unroll
      for (int s = 0; s < C::NS - 1; ++s)
        if (s < KT) issue(s, s);
    }
  };

  // Fragment addresses: row (lane & 31) of the wave's first 32-row block,
  // logical chunk 2s + (lane >> 5), swizzled.
  int a_rd[C::KSTEPS], b_rd[C::KSTEPS];
#pragma unroll
  for (int s = 0; s < C::KSTEPS; ++s) {
    const int ch = ((2 * s + lhalf) ^ swz_key<C::CPR>(lrow)) * 16;
    a_rd[s] = (wm * C::WTM + lrow) * C::BK * 2 + ch;
    b_rd[s] = (wn * C::WTN + lrow) * C::BK * 2 + ch;
  }

  f32x16 acc[C::TN][C::TM];

  // Fragments of k-step s+1 are read from LDS while the MFMAs of k-step s
  // run; sched_group_barrier pins that interleaving (one LDS read after each
  // of the first MFMAs) so the reads' latency hides behind matrix work.
  auto read_frags = [&](const char* as, const char* bs, int s, bf16x8* af, bf16x8* bf) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      af[i] = *reinterpret_cast<const bf16x8*>(as + a_rd[s] + i * 32 * C::BK * 2);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      bf[j] = *reinterpret_cast<const bf16x8*>(bs + b_rd[s] + j * 32 * C::BK * 2);
  };
  auto compute = [&](int sa, int sb, auto&& loads) {
    const char* as = a_lds + sa * C::A_STAGE;
    const char* bs = b_lds + sb * C::B_STAGE;
    bf16x8 af[2][C::TM], bf[2][C::TN];
    // The first fragment reads go out before the next slices' loads, so the
    // matrix cores restart as soon as possible after the barrier.
    read_frags(as, bs, 0, af[0], bf[0]);
    loads();
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      if (s + 1 < C::KSTEPS) read_frags(as, bs, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s & 1][j], af[s & 1][i],
                                                              acc[j][i], 0, 0, 0);
      if (C::SCHED && s + 1 < C::KSTEPS) {
#pragma unroll
        for (int r = 0; r < C::TM + C::TN; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, C::TM * C::TN - C::TM - C::TN, 0);
      }
    }
  };

  int t = blockIdx.x;
  if (t >= total) return;  // whole workgroup
  prepare(t);
  start_tile();

  float rsd[C::TM];  // LayerNorm fold: rstd of the lane's rows of the current tile
  while (true) {
    // The bias of block j's columns for this lane: element r of block (j, i)
    // is column (r/4)*8 + (l/32)*4 + r%4 of block j.  One segment (bias_seg
    // >= N: every bias but the three separate Q, K, V vectors): each run of 4
    // columns is one 8-byte raw buffer load at a 32-bit offset, columns past
    // N read as zero by the buffer's range check.  Otherwise at most three
    // segments (N <= 3 bias_seg), the segment by comparison, columns past N
    // clamped.
    const bool one_seg = p.bias_seg >= N;  // uniform
    auto bias_run = [&](int j, float* bv) {
      if (one_seg) {
        uint2 u[4] = {};
        if (p.bias[0] != nullptr) {
          const __amdgpu_buffer_rsrc_t brs = __builtin_amdgcn_make_buffer_rsrc(
              const_cast<void*>(p.bias[0]), 0, static_cast<int>(static_cast<uint32_t>(N * 2)),
              kBufferFlags);
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const uint32_t n = static_cast<uint32_t>(n0) + wn * C::WTN + j * 32 + g4 * 8 + lhalf * 4;
            const auto v = __builtin_amdgcn_raw_buffer_load_b64(brs, n * 2, 0, 0);
            u[g4] = make_uint2(v[0], v[1]);
          }
        }
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          bv[g4 * 4 + 0] = __uint_as_float(u[g4].x << 16);
          bv[g4 * 4 + 1] = __uint_as_float(u[g4].x & 0xffff0000u);
          bv[g4 * 4 + 2] = __uint_as_float(u[g4].y << 16);
          bv[g4 * 4 + 3] = __uint_as_float(u[g4].y & 0xffff0000u);
        }
        return;
      }
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        int64_t n = n0 + wn * C::WTN + j * 32 + g4 * 8 + lhalf * 4;
        n = n < N ? n : N - 4;
        const bool s1 = n >= p.bias_seg, s2 = n >= 2 * p.bias_seg;
        const void* bs = s2 ? p.bias[2] : (s1 ? p.bias[1] : p.bias[0]);
        const int64_t off = n - (s2 ? 2 * p.bias_seg : (s1 ? p.bias_seg : 0));
        uint2 u = make_uint2(0u, 0u);
        if (bs != nullptr)
          u = *reinterpret_cast<const uint2*>(static_cast<const bf16_t*>(bs) + off);
        bv[g4 * 4 + 0] = __uint_as_float(u.x << 16);
        bv[g4 * 4 + 1] = __uint_as_float(u.x & 0xffff0000u);
        bv[g4 * 4 + 2] = __uint_as_float(u.y << 16);
        bv[g4 * 4 + 3] = __uint_as_float(u.y & 0xffff0000u);
      }
    };
    if (NORM) {
      // LayerNorm fold, mean term: the accumulators start at -mean_m *
      // colsum_n, so after the k loop they hold A @ W - mean colsum and the
      // epilogue only scales by rstd_m (and, with a bias, adds it in the same
      // fma: rstd (A @ W - mean colsum) + b).  The loads (L2-resident) go out
      // before the first k-slice's wait, which they share.  A lane's rows
      // are lrow of each 32-row block i.  Rows and columns past M or N are
      // clamped (never stored).
      float nmu[C::TM];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        int64_t m = m0 + wm * C::WTM + i * 32 + lrow;
        m = m < M ? m : M - 1;
        const float2 st = *reinterpret_cast<const float2*>(p.row_stats + 2 * m);
        nmu[i] = -st.x;
        rsd[i] = st.y;
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        float cs[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          int64_t n = n0 + wn * C::WTN + j * 32 + g4 * 8 + lhalf * 4;
          n = n < N ? n : N - 4;
          const float4 c4 = *reinterpret_cast<const float4*>(p.col_sums + n);
          cs[g4 * 4 + 0] = c4.x;
          cs[g4 * 4 + 1] = c4.y;
          cs[g4 * 4 + 2] = c4.z;
          cs[g4 * 4 + 3] = c4.w;
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][i][r] = nmu[i] * cs[r];
      }
    } else if (BIAS) {
      // Bias without the fold: the accumulators start at the bias, so the
      // epilogue has nothing to add.
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        float bv[16];
        bias_run(j, bv);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][i][r] = bv[r];
      }
    } else {
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
    }

    // Before computing slice kt a wave waits until its own loads of slice kt
    // have landed (newer slices may stay outstanding; vmcnt retires in issue
    // order), then the barrier makes every wave's part visible and
    // guarantees that the stage refilled next (read in the previous
    // iteration) is no longer being read.
    for (int kt = 0; kt < KT; ++kt) {
      if (C::NSA > C::NS) {
        // Iteration j issues W(j+1) then A(j+2); at the top of iteration kt
        // only A(kt+1) is newer than W(kt) (and A(kt) is older); a loading
        // wave of the big tile issues twice the A loads.  Loads retire in
        // issue order; at kt = 0 the previous tile's stores are pending too,
        // so wait for everything.
        if (kt > 0 && kt + 1 < KT)
          wait_vmcnt<(kSpec ? 2 : 1) * C::A_LOADS>();
        else
          wait_vmcnt<0>();
        __builtin_amdgcn_s_barrier();
        compute(kt % C::NSA, kt % C::NS, [&]() {
          if (kt + 1 < KT) issue_b(kt + 1, (kt + 1) % C::NS);
          if (kt + 2 < KT) issue_a(kt + 2, (kt + 2) % C::NSA);
        });
        continue;
      }
      // Loads issued after slice kt's: those of the newer slices (at kt = 0
      // the previous tile's stores are pending too).
      if (kt > 0 && kt + C::NS - 2 < KT)
        wait_vmcnt<(C::NS - 2) * (C::A_LOADS + C::B_LOADS)>();
      else
        wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      compute(kt % C::NS, kt % C::NS, [&]() {
        if (kt + C::NS - 1 < KT) issue(kt + C::NS - 1, (kt + C::NS - 1) % C::NS);
      });
    }

    // The epilogue's global reads (residual, bias) go out before the next
    // tile's first k-slices: loads complete in issue order, so a read issued
    // after those slices would hold the epilogue until they had landed.
    const int64_t cm0 = m0, cn0 = n0;
    const int cks = ks;
    const bf16_t* Rp = static_cast<const bf16_t*>(p.R);
    // R: the residual, or GELU's input z for the GELU-derivative epilogue, in
    // the lanes' store layout (below), rows and columns clamped into range.
    constexpr bool kReadsR = EPI == VITBLK_EPI_RESIDUAL || EPI == VITBLK_EPI_GELU_GRAD ||
                             EPI == kEpiMul || EPI == kEpiResidualStats || EPI == kEpiEmbed;
    uint4 res[C::TM][C::TN][2];
    // With the LayerNorm fold the bias enters in the epilogue's rstd scale
    // (an fma instead of the multiply): read with the other epilogue operands.
    float bve[C::TN][16];
    if (NORM && BIAS) {
#pragma unroll
      for (int j = 0; j < C::TN; ++j) bias_run(j, bve[j]);
    }
    // kEpiEmbed: each wave block's quotient and remainder (see c_row).
    uint32_t bq[C::TM], br[C::TM];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      bq[i] = br[i] = 0;
      block_div(cm0 + wm * C::WTM + i * 32, &bq[i], &br[i]);
    }
    if (kReadsR) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        int64_t m = cm0 + wm * C::WTM + i * 32 + lrow;
        // A row past M reads the block's first row (its product is never stored).
        const int rdelta = m < M ? lrow : 0;
        m = m < M ? m : M - 1;
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            int64_t n = cn0 + wn * C::WTN + j * 32 + q * 16 + lhalf * 8;
            n = n < N ? n : N - 8;
            res[i][j][q] = ld_global16(Rp + r_row(m, br[i], rdelta) * p.ldr + n);
          }
      }
    }

    // Start the next tile's first k-slices before this tile's epilogue (all
    // waves are done reading LDS once past this barrier).
    const int t_next = t + grid;
    const bool more = t_next < total;
    __builtin_amdgcn_s_barrier();
    if (more) {
      prepare(t_next);
      start_tile();
    }

    // Epilogue.  Accumulator element r of lane l in block (j, i) is
    // C[m0 + wm*WTM + i*32 + (l & 31)][n0 + wn*WTN + j*32 + (r/4)*8 + (l/32)*4 + r%4].
    // Lanes l and l+32 hold the two halves of 8 consecutive columns; one
    // v_permlane32_swap per dword hands lane l the columns 16q + 0..7 and lane
    // l+32 the columns 16q + 8..15 (q = 0, 1), so every lane writes 16
    // contiguous bytes.  Residuals are read in that layout, all before the
    // first store (addresses clamped into range), and added in fp32 before
    // the single rounding to bf16.
    bf16_t* Cp = static_cast<bf16_t*>(p.C);
    // LayerNorm fold, scale term: acc = rstd_m * acc (+ b_n).
    if (NORM) {
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[j][i][r] = BIAS ? __builtin_fmaf(acc[j][i][r], rsd[i], bve[j][r])
                                : acc[j][i][r] * rsd[i];
    }
    // The plain and residual epilogues store each 32-row block as whole row
    // lines (rows_to_lines): 8% faster on the fused Q|K|V projection.  The
    // GELU epilogue keeps the direct stores: its exponentials already pace the
    // stores, and the extra exchange work made it 2% slower.
    constexpr bool kLines = (EPI == VITBLK_EPI_NONE || EPI == VITBLK_EPI_RESIDUAL ||
                             EPI == kEpiResidualStats || EPI == kEpiEmbed) &&
                            C::TN == 2;
    // C stores: raw buffer stores at 32-bit offsets from the tile's first
    // row; a lane outside M or N gets an offset past the buffer's range, so
    // the hardware drops its store.  With no branch per store the epilogue
    // is one block the scheduler can interleave (ViT-L/16 Q|K|V 298.8 ->
    // 295.0 us, MLP1 427.5 -> 425.0 us).  Not for the token-row epilogue (its
    // rows are remapped), nor where the big tile would then spill registers:
    // with a bias, and the GELU-derivative and row-statistics epilogues.
    constexpr bool kBufStore =
        EPI != kEpiEmbed && !kSplit && !BIAS &&
        !(C::BM == 256 && (EPI == VITBLK_EPI_GELU_GRAD || EPI == kEpiResidualStats));
    const int64_t c_rows = M - cm0 < C::BM ? M - cm0 : C::BM;
    auto c_rsrc = [&](void* base) {
      return __builtin_amdgcn_make_buffer_rsrc(static_cast<bf16_t*>(base) + cm0 * p.ldc, 0,
                                               static_cast<int>(c_rows * p.ldc * 2),
                                               kBufferFlags);
    };
    const __amdgpu_buffer_rsrc_t c_rs = c_rsrc(p.C);
    auto store_c = [&](const __amdgpu_buffer_rsrc_t& rs, int64_t m, int64_t n, const uint4& v) {
      const uint32_t off = (m < M && n < N) ? static_cast<uint32_t>(((m - cm0) * p.ldc + n) * 2)
                                            : 0x80000000u;
      typedef unsigned v4u __attribute__((ext_vector_type(4)));
      const v4u d = {v.x, v.y, v.z, v.w};
      __builtin_amdgcn_raw_buffer_store_b128(d, rs, off, 0, 0);
    };
    if (kSplit) {
      // Unrounded fp32 sums of this k-range: after the fp32 half exchange a
      // lane holds 8 consecutive columns of one row (32 bytes).
      float* P = static_cast<float*>(p.C) + static_cast<int64_t>(cks) * M * p.ldc;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int64_t m = cm0 + wm * C::WTM + i * 32 + lrow;
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const int64_t n = cn0 + wn * C::WTN + j * 32 + q * 16 + lhalf * 8;
            float x[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const auto r = __builtin_amdgcn_permlane32_swap(
                  __float_as_uint(acc[j][i][(2 * q) * 4 + e]),
                  __float_as_uint(acc[j][i][(2 * q + 1) * 4 + e]), false, false);
              x[e] = __uint_as_float(r[0]);
              y[e] = __uint_as_float(r[1]);
            }
            if (m < M && n < N) {
              float4* d = reinterpret_cast<float4*>(P + m * p.ldc + n);
              d[0] = make_float4(x[0], x[1], x[2], x[3]);
              d[1] = make_float4(y[0], y[1], y[2], y[3]);
            }
          }
      }
    }
#pragma unroll
    for (int i = 0; i < (kSplit ? 0 : C::TM); ++i) {
      const int64_t m = cm0 + wm * C::WTM + i * 32 + lrow;
      uint4 outs[C::TN][2];
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const int64_t n = cn0 + wn * C::WTN + j * 32 + q * 16 + lhalf * 8;
          uint4 out;
          if (kReadsR) {
            // fp32 exchange: lane's 8 columns are x[0..3] then y[0..3].
            float x[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const auto r = __builtin_amdgcn_permlane32_swap(
                  __float_as_uint(acc[j][i][(2 * q) * 4 + e]),
                  __float_as_uint(acc[j][i][(2 * q + 1) * 4 + e]), false, false);
              x[e] = __uint_as_float(r[0]);
              y[e] = __uint_as_float(r[1]);
            }
            const uint4 rv = res[i][j][q];
            const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              v[e] = x[e];
              v[4 + e] = y[e];
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float r0 = __uint_as_float(rw[e] << 16);
              const float r1 = __uint_as_float(rw[e] & 0xffff0000u);
              if (EPI == VITBLK_EPI_GELU_GRAD) {
                v[2 * e] *= gelu_tanh_grad_fast(r0);
                v[2 * e + 1] *= gelu_tanh_grad_fast(r1);
              } else if (EPI == kEpiMul) {
                v[2 * e] *= r0;
                v[2 * e + 1] *= r1;
              } else {
                v[2 * e] += r0;
                v[2 * e + 1] += r1;
              }
            }
            out = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                             pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
          } else {
            // round first, then exchange bf16 pairs (4 dwords per lane).
            uint32_t w[2][2], w2[2][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              float v[4], d[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                v[e] = acc[j][i][(2 * q + h) * 4 + e];
                if (EPI == kEpiGeluDual) d[e] = gelu_tanh_grad_fast(v[e]);
                if (EPI == VITBLK_EPI_GELU || EPI == kEpiGeluDual) v[e] = gelu_tanh_fast(v[e]);
              }
              w[h][0] = pack_bf16x2(v[0], v[1]);
              w[h][1] = pack_bf16x2(v[2], v[3]);
              if (EPI == kEpiGeluDual) {
                w2[h][0] = pack_bf16x2(d[0], d[1]);
                w2[h][1] = pack_bf16x2(d[2], d[3]);
              }
            }
            const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][0], w[1][0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(w[0][1], w[1][1], false, false);
            out = make_uint4(s0[0], s1[0], s0[1], s1[1]);
            if (EPI == kEpiGeluDual) {
              const auto t0 = __builtin_amdgcn_permlane32_swap(w2[0][0], w2[1][0], false, false);
              const auto t1 = __builtin_amdgcn_permlane32_swap(w2[0][1], w2[1][1], false, false);
              const uint4 d2 = make_uint4(t0[0], t1[0], t0[1], t1[1]);
              if constexpr (kBufStore)
                store_c(c_rsrc(p.C2), m, n, d2);
              else if (m < M && n < N)
                st_global16(static_cast<bf16_t*>(p.C2) + m * p.ldc + n, d2);
            }
          }
          outs[j][q] = out;
          if constexpr (!kLines) {
            if constexpr (kBufStore)
              store_c(c_rs, m, n, out);
            else if (m < M && n < N)
              st_global16(Cp + c_row(m, bq[i], br[i], lrow) * p.ldc + n, out);
          }
        }
      }
      if constexpr (EPI == kEpiResidualStats) {
        // Row m's statistics over this wave's WTN columns, from the values as
        // stored (bf16): the lane's 16 * TN values as a sum and a sum of
        // squares (v_dot2_f32_bf16 of each packed pair with (1, 1) and with
        // itself: the bf16 products are exact in fp32), the lane's M2 = S2 -
        // S1^2 / n (relative error about n 2^-24 (1 + mean^2 / var)), then
        // the two lane halves combined (Chan et al.'s pairwise update).
        static_assert(C::WTN == kStatsStrip, "one partial per wave strip");
        constexpr float kCnt = 16.0f * C::TN;
        constexpr bf16x2_t kOne2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint32_t w[4] = {outs[j][q].x, outs[j][q].y, outs[j][q].z, outs[j][q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, w[e]);
              s1 = __builtin_amdgcn_fdot2_f32_bf16(pr, kOne2, s1, false);
              s2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, s2, false);
            }
          }
        const float mu = s1 * (1.0f / kCnt);
        const float m2 = fmaxf(fmaf(-s1, mu, s2), 0.0f);
        const auto ms = __builtin_amdgcn_permlane32_swap(__float_as_uint(mu), __float_as_uint(mu),
                                                         false, false);
        const auto qs = __builtin_amdgcn_permlane32_swap(__float_as_uint(m2), __float_as_uint(m2),
                                                         false, false);
        const float ma = __uint_as_float(ms[0]), mb = __uint_as_float(ms[1]);
        const float delta = mb - ma;
        const float mean = 0.5f * (ma + mb);
        const float m2t = __uint_as_float(qs[0]) + __uint_as_float(qs[1]) +
                          delta * delta * (0.5f * kCnt);
        // A strip lies wholly inside or outside N (N is a multiple of it).
        const int64_t n_strip = cn0 + wn * C::WTN;
        if (lhalf == 0 && m < M && n_strip < N) {
          const int64_t strips = N / kStatsStrip;
          const int64_t strip = n_strip / kStatsStrip;
          p.row_partials[m * strips + strip] = make_float2(mean, m2t);
        }
      }
      if (kLines) {
        uint4 v[4] = {outs[0][0], outs[0][1], outs[C::TN - 1][0], outs[C::TN - 1][1]};
        rows_to_lines(v, lane);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t mr = cm0 + wm * C::WTM + i * 32 + t * 8 + (lane >> 3);
          const int64_t nr = cn0 + wn * C::WTN + (lane & 7) * 8;
          if constexpr (kBufStore)
            store_c(c_rs, mr, nr, v[t]);
          else if (mr < M && nr < N)
            st_global16(Cp + c_row(mr, bq[i], br[i], t * 8 + (lane >> 3)) * p.ldc + nr, v[t]);
        }
      }
    }
    if (!more) break;
    t = t_next;
  }
}

// 8 waves (2 per SIMD), 128x64 per wave, 3 A stages + 2 W stages: 160 KB LDS.
using BigTile = Cfg<256, 256, 2, 4, 64, 2, 3>;
// 4 waves, 64x64 per wave, 80 KB LDS: 2 workgroups per CU.
using SmallTile = Cfg<128, 128, 2, 2, 64, 2, 3>;
// 8 waves, 96x64 per wave, 3 A stages + 2 W stages: 136 KB LDS, one workgroup
// per CU.  Three quarters of a big tile's work, for products whose big tiles
// leave CUs idle in their only round.
using MidTile = Cfg<192, 256, 2, 4, 64, 2, 3>;
// The small tile with four stages of both operands (128 KB LDS, one workgroup
// per CU): three k-slices in flight instead of two (activations) and one
// (weights).  For a last partial round of tiles, where each workgroup runs
// alone on its CU and its time is the latency of its k-slices.
using DeepTile = Cfg<128, 128, 2, 2, 64, 4, 4>;

// Split-K finish: C[m, n] = bf16(((sum_s P[s, m, n]) + b[n]) + R[m, n]), the
// partials summed in order in fp32 (the same order of additions as the
// one-pass residual epilogue: products, then bias, then residual).  One
// thread per 8 consecutive columns; N is a multiple of 8.
__global__ __launch_bounds__(256) void splitk_residual_kernel(const float* __restrict__ P,
                                                              int S, int64_t M, int64_t N,
                                                              const bf16_t* __restrict__ R,
                                                              int64_t ldr,
                                                              const bf16_t* __restrict__ bias,
                                                              bf16_t* __restrict__ Cp,
                                                              int64_t ldc) {
  const int64_t g = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t per_row = N >> 3;
  if (g >= M * per_row) return;
  const int64_t m = g / per_row, n = (g - m * per_row) * 8;
  float v[8];
  {
    const float4* q = reinterpret_cast<const float4*>(P + m * N + n);
    const float4 a = q[0], b = q[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  for (int sp = 1; sp < S; ++sp) {
    const float4* q = reinterpret_cast<const float4*>(P + (sp * M + m) * N + n);
    const float4 a = q[0], b = q[1];
    v[0] += a.x; v[1] += a.y; v[2] += a.z; v[3] += a.w;
    v[4] += b.x; v[5] += b.y; v[6] += b.z; v[7] += b.w;
  }
  if (bias != nullptr) {  // 8-byte aligned
    const uint2 u0 = *reinterpret_cast<const uint2*>(bias + n);
    const uint2 u1 = *reinterpret_cast<const uint2*>(bias + n + 4);
    const uint32_t w[4] = {u0.x, u0.y, u1.x, u1.y};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] += __uint_as_float(w[e] << 16);
      v[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
    }
  }
  const uint4 r = ld_global16(R + m * ldr + n);
  const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] += __uint_as_float(rw[e] << 16);
    v[2 * e + 1] += __uint_as_float(rw[e] & 0xffff0000u);
  }
  st_global16(Cp + m * ldc + n, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])));
}

// Workgroups of this kernel the device holds at once (cached per kernel).
template <class C, int EPI, bool BIAS = false, bool NORM = false>
int resident_workgroups() {
  static std::atomic<int> cached{0};  // computed once, the same value by any thread
  int value = cached.load(std::memory_order_relaxed);
  if (value == 0) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(&gemm_bf16_kernel<C, EPI, BIAS, NORM>), C::NT,
            0) !=
            hipSuccess) {
      (void)hipGetLastError();
      return 0;
    }
    value = cus * (per_cu > 0 ? per_cu : 1);
    cached.store(value, std::memory_order_relaxed);
  }
  return value;
}

template <class C, int EPI, bool BIAS, bool NORM = false>
hipError_t launch_epi(const GemmProblem& p, hipStream_t s) {
  const int64_t mt = (p.M + C::BM - 1) / C::BM, nt = (p.N + C::BN - 1) / C::BN;
  const int64_t tiles = mt * nt * (EPI == kEpiPartial ? p.ksplit : 1);
  if (tiles > 2147483647LL) return hipErrorInvalidValue;
  int64_t grid = resident_workgroups<C, EPI, BIAS, NORM>();
  if (grid <= 0) return hipErrorInvalidValue;
  grid = grid / kNumXcd * kNumXcd;  // keeps the XCD-contiguous mapping exact
  if (grid <= 0 || grid > tiles) grid = tiles;
  hipLaunchKernelGGL((gemm_bf16_kernel<C, EPI, BIAS, NORM>), dim3(static_cast<unsigned>(grid)),
                     dim3(C::NT), 0, s, p, static_cast<int>(mt), static_cast<int>(nt));
  return hipGetLastError();
}

// Epilogue and bias as template arguments: the kernels without a bias carry
// no bias state at all.
template <class C, bool BIAS>
hipError_t launch_bias(const GemmProblem& p, hipStream_t s) {
  switch (p.epi) {
    case VITBLK_EPI_RESIDUAL: return launch_epi<C, VITBLK_EPI_RESIDUAL, BIAS>(p, s);
    case VITBLK_EPI_GELU: return launch_epi<C, VITBLK_EPI_GELU, BIAS>(p, s);
    case VITBLK_EPI_GELU_GRAD: return launch_epi<C, VITBLK_EPI_GELU_GRAD, BIAS>(p, s);
    case kEpiGeluDual: return launch_epi<C, kEpiGeluDual, BIAS>(p, s);
    case kEpiMul: return launch_epi<C, kEpiMul, BIAS>(p, s);
    case kEpiPartial: return launch_epi<C, kEpiPartial, false>(p, s);
    case kEpiResidualStats: return launch_epi<C, kEpiResidualStats, BIAS>(p, s);
    case kEpiEmbed: return launch_epi<C, kEpiEmbed, BIAS>(p, s);
    default: return launch_epi<C, VITBLK_EPI_NONE, BIAS>(p, s);
  }
}

// The LayerNorm-folded products (plain or GELU epilogue only).
template <class C, bool BIAS>
hipError_t launch_norm(const GemmProblem& p, hipStream_t s) {
  if (p.epi == VITBLK_EPI_GELU) return launch_epi<C, VITBLK_EPI_GELU, BIAS, true>(p, s);
  if (p.epi == VITBLK_EPI_NONE) return launch_epi<C, VITBLK_EPI_NONE, BIAS, true>(p, s);
  return hipErrorInvalidValue;
}

template <class C>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t s) {
  if (p.row_stats != nullptr)
    return has_bias(p) ? launch_norm<C, true>(p, s) : launch_norm<C, false>(p, s);
  return has_bias(p) ? launch_bias<C, true>(p, s) : launch_bias<C, false>(p, s);
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

// The MFMA kernel needs bf16, K a multiple of 64, N a multiple of 8, 16-byte
// aligned rows, and a 256-row panel of either operand and of the output to
// span < 2 GiB (its buffer offsets are 32-bit); a bias in segments of a multiple of 8 columns
// (so no lane's run of columns straddles two segments), 8-byte aligned.
// Everything else takes the generic kernel.
bool gemm_fast_ok(const GemmProblem& p) {
  bool ok = p.dtype == VITBLK_BF16 && p.K % 64 == 0 && p.N % 8 == 0 && p.N >= 8 &&
            p.lda % 8 == 0 && p.ldb % 8 == 0 && p.ldc % 8 == 0 && aligned16(p.A) &&
            aligned16(p.B) && aligned16(p.C) && p.lda * 2 * 256 < (1LL << 31) &&
            p.ldb * 2 * 256 < (1LL << 31) && p.ldc * 2 * 256 < (1LL << 31) &&
            p.K * 2 < (1LL << 31);
  if (reads_r(p)) ok = ok && p.ldr % 8 == 0 && aligned16(p.R);
  if (p.row_stats != nullptr)
    ok = ok && aligned16(p.col_sums) && (reinterpret_cast<uintptr_t>(p.row_stats) & 7u) == 0;
  if (p.epi == kEpiGeluDual) ok = ok && aligned16(p.C2);
  if (has_bias(p)) {
    ok = ok && p.bias_seg > 0 && p.bias_seg % 8 == 0 && p.N <= 3 * p.bias_seg;
    for (const void* b : p.bias)
      ok = ok && (reinterpret_cast<uintptr_t>(b) & 7u) == 0;
  }
  return ok;
}

// The row partials ride on the tiles the output projection (a residual
// product with K = D) takes anyway, whose waves cover 64 columns each.
bool gemm_row_partials_ok(const GemmProblem& p) {
  GemmProblem q = p;
  q.epi = kEpiResidualStats;
  return gemm_fast_ok(q) && p.row_partials != nullptr && p.N % kStatsStrip == 0 &&
         (reinterpret_cast<uintptr_t>(p.row_partials) & 7u) == 0;
}

// Rows [r0, r0 + rows) of p as a problem of its own.
GemmProblem row_slice(const GemmProblem& p, int64_t r0, int64_t rows) {
  GemmProblem q = p;
  q.M = rows;
  q.A = static_cast<const char*>(p.A) + r0 * p.lda * 2;
  if (p.epi == kEpiEmbed) {  // C and R rows follow from the absolute product row
    q.row_base = p.row_base + r0;
    return q;
  }
  q.C = static_cast<char*>(p.C) + r0 * p.ldc * 2;
  if (p.R) q.R = static_cast<const char*>(p.R) + r0 * p.ldr * 2;
  if (p.C2) q.C2 = static_cast<char*>(p.C2) + r0 * p.ldc * 2;
  if (p.row_stats) q.row_stats = p.row_stats + 2 * r0;
  return q;
}

constexpr int kMaxSplit = 8;       // k-ranges of a split-K tail
constexpr int kMinSplitSlices = 4;  // k-slices (of 64) per range at least

// The last rows of a product, left over by the big tile's whole rounds.  On
// the 128x128 tile they are few tiles, each alone on its CU, so they run on
// the four-stage variant of that tile (DeepTile) when they fit in one round
// of it (measured: 18.2 -> 17.5 us for the Q|K|V tail at ViT-L/16, 30.0 ->
// 27.3 us for MLP2's split tail and its sum); otherwise on the two-workgroups-
// per-CU small tile.  When K is long each tile runs for a long time while most
// CUs idle.  A residual product (the one kind whose result needs no
// nonlinearity after the sum) then splits K into S ranges, as many as fill the
// resident deep-tile slots: the ranges' unrounded fp32 sums go to the caller's
// scratch memory and a second kernel adds them in order, with the bias and the
// residual, and rounds once.
hipError_t launch_tail(const GemmProblem& p, hipStream_t s) {
  using Small = SmallTile;
  static_assert(DeepTile::BM == Small::BM && DeepTile::BN == Small::BN, "same tile shape");
  const int64_t tiles = ((p.M + Small::BM - 1) / Small::BM) * ((p.N + Small::BN - 1) / Small::BN);
  const int64_t ka = p.K / Small::BK;
  // One workgroup per CU whatever the epilogue (the LDS decides).
  const int64_t deep_slots = resident_workgroups<DeepTile, kEpiPartial>();
  int64_t S = 0;
  if (p.epi == VITBLK_EPI_RESIDUAL && p.scratch != nullptr && p.bias[1] == nullptr &&
      p.bias[2] == nullptr && (p.bias[0] == nullptr || p.bias_seg >= p.N) &&
      p.ldc % 8 == 0 && (reinterpret_cast<uintptr_t>(p.scratch) & 15u) == 0) {
    S = tiles > 0 ? deep_slots / tiles : 0;
    if (S > kMaxSplit) S = kMaxSplit;
    if (S > ka / kMinSplitSlices) S = ka / kMinSplitSlices;
    while (S > 1 && S * p.M * p.N > p.scratch_floats) --S;
  }
  if (S < 2) return tiles <= deep_slots ? launch_cfg<DeepTile>(p, s) : launch_cfg<Small>(p, s);
  GemmProblem q = p;
  q.epi = kEpiPartial;
  q.ksplit = static_cast<int>(S);
  q.C = p.scratch;
  q.ldc = p.N;
  q.R = nullptr;
  q.bias[0] = q.bias[1] = q.bias[2] = nullptr;
  hipError_t e = launch_epi<DeepTile, kEpiPartial, false>(q, s);
  if (e != hipSuccess) return e;
  const int64_t threads = p.M * (p.N / 8);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(splitk_residual_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const float*>(p.scratch), static_cast<int>(S), p.M, p.N,
                     static_cast<const bf16_t*>(p.R), p.ldr,
                     static_cast<const bf16_t*>(p.bias[0]), static_cast<bf16_t*>(p.C), p.ldc);
  return hipGetLastError();
}

// The residual products with K <= 1024 (the output projection) take the small
// tile, except when its tiles need more than one round and the 192-row tiles
// fit in one (ViT-B/16: 594 small tiles for 512 slots, or 198 of 192 rows:
// 29.8 -> 27.8 us with the LayerNorm partials).
bool mid_fits_one_round(const GemmProblem& p) {
  const int64_t nt = (p.N + MidTile::BN - 1) / MidTile::BN;
  const int64_t mid = (p.M + MidTile::BM - 1) / MidTile::BM * nt;
  const int64_t small = ((p.M + SmallTile::BM - 1) / SmallTile::BM) *
                        ((p.N + SmallTile::BN - 1) / SmallTile::BN);
  const int64_t mid_slots = resident_workgroups<MidTile, VITBLK_EPI_NONE>() / kNumXcd * kNumXcd;
  const int64_t small_slots = resident_workgroups<SmallTile, VITBLK_EPI_NONE>();
  return mid_slots > 0 && small_slots > 0 && small > small_slots && mid <= mid_slots;
}

// Tile choice.  With one big-tile workgroup per CU, a tile's epilogue runs
// with the matrix cores idle; when it also reads a residual and K is short
// (the output projection: K = D) that share is large, and the small tile,
// two workgroups per CU, lets one workgroup's epilogue overlap the other's
// main loop.  Otherwise the big tile (half the operand traffic per flop).
//
// Wave quantisation: with G resident big-tile workgroups, the last partial
// round of tiles would run a handful of tiles for a full round's time.  The
// big tile therefore covers the largest block of M-tiles that makes a whole
// number of rounds, and the remaining rows run as a second launch with a
// quarter-size tile, which finishes in a fraction of a round (launch_tail).
hipError_t launch_gemm(const GemmProblem& p, hipStream_t s) {
  if (reads_r(p) && p.R == nullptr) return hipErrorInvalidValue;  // never launch on a null R
  if (p.epi == kEpiGeluDual && p.C2 == nullptr) return hipErrorInvalidValue;
  if (p.row_stats != nullptr &&
      (p.col_sums == nullptr || (p.epi != VITBLK_EPI_NONE && p.epi != VITBLK_EPI_GELU)))
    return hipErrorInvalidValue;
  if (p.epi == kEpiResidualStats) {
    if (!gemm_row_partials_ok(p)) return hipErrorInvalidValue;
    return mid_fits_one_round(p) ? launch_cfg<MidTile>(p, s) : launch_cfg<SmallTile>(p, s);
  }
  if (p.epi == kEpiEmbed && (!gemm_fast_ok(p) || p.row_group <= 0 || p.row_skip < 0 ||
                             p.row_base < 0 || p.row_base + p.M > 2147483647LL))
    return hipErrorInvalidValue;  // the token-row epilogue exists on the MFMA kernel only
  if (!gemm_fast_ok(p)) return launch_gemm_generic(p, s);
  using Big = BigTile;
  using Small = SmallTile;
  if (p.epi == VITBLK_EPI_RESIDUAL && p.K <= 1024)
    return mid_fits_one_round(p) ? launch_cfg<MidTile>(p, s) : launch_cfg<Small>(p, s);
  const int64_t mt = (p.M + Big::BM - 1) / Big::BM, nt = (p.N + Big::BN - 1) / Big::BN;
  int64_t grid = 0;
  switch (p.epi) {
    case VITBLK_EPI_RESIDUAL: grid = resident_workgroups<Big, VITBLK_EPI_RESIDUAL>(); break;
    case VITBLK_EPI_GELU: grid = resident_workgroups<Big, VITBLK_EPI_GELU>(); break;
    case VITBLK_EPI_GELU_GRAD: grid = resident_workgroups<Big, VITBLK_EPI_GELU_GRAD>(); break;
    case kEpiGeluDual: grid = resident_workgroups<Big, kEpiGeluDual>(); break;
    case kEpiMul: grid = resident_workgroups<Big, kEpiMul>(); break;
    default: grid = resident_workgroups<Big, VITBLK_EPI_NONE>(); break;
  }
  grid = grid / kNumXcd * kNumXcd;
  if (grid > 0 && mt * nt < grid) {
    // Fewer big tiles than CUs: each CU holds at most one tile, so the time
    // is one tile's; 192-row tiles take 3/4 of it when they too fit in one
    // round (ViT-B/16's MLP2: 150 big tiles or 198 of these, 72.3 -> 60.3 us).
    const int64_t mt_mid = (p.M + MidTile::BM - 1) / MidTile::BM;
    if (mt_mid * nt <= grid) return launch_cfg<MidTile>(p, s);
  }
  if (grid <= 0 || mt * nt <= grid) return launch_cfg<Big>(p, s);
  int64_t g = grid, b = nt;  // gcd(grid, nt)
  while (b) {
    const int64_t r = g % b;
    g = b;
    b = r;
  }
  const int64_t step = grid / g;     // M-tiles per whole number of rounds
  int64_t m_main = mt / step * step;  // M-tiles done with the big tile
  if ((mt * nt) % grid == 0) return launch_cfg<Big>(p, s);
  if (m_main == 0) {
    // No row split gives whole rounds (nt shares few factors with the grid):
    // the big tile takes the rows of floor(tiles / grid) nearly full rounds
    // and the small tile the rest, when that is estimated to be shorter than
    // a last partial round of big tiles.  A round of the small tile (a
    // quarter of the work per tile, two workgroups per CU) is counted as half
    // a big-tile round.
    const int64_t rounds = mt * nt / grid;
    const int64_t m_try = rounds * grid / nt;
    if (m_try > 0 && m_try < mt) {
      const int64_t small_tiles = ((p.M - m_try * Big::BM + SmallTile::BM - 1) / SmallTile::BM) *
                                  ((p.N + SmallTile::BN - 1) / SmallTile::BN);
      int64_t small_slots = resident_workgroups<SmallTile, VITBLK_EPI_NONE>();
      if (small_slots <= 0) small_slots = 2 * grid;
      const int64_t small_rounds = (small_tiles + small_slots - 1) / small_slots;
      const int64_t whole_rounds = (mt * nt + grid - 1) / grid;
      if (2 * ((m_try * nt + grid - 1) / grid) + small_rounds < 2 * whole_rounds) m_main = m_try;
    }
  }
  if (m_main == 0 || m_main == mt) return launch_cfg<Big>(p, s);
  const int64_t rows_main = m_main * Big::BM;
  const hipError_t e = launch_cfg<Big>(row_slice(p, 0, rows_main), s);
  if (e != hipSuccess) return e;
  return launch_tail(row_slice(p, rows_main, p.M - rows_main), s);
}

}  // namespace vitblk
