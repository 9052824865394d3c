// bf16 GEMM on the gfx950 matrix cores with fused epilogues.
//
// C = epi(A @ B) for A [M, K] (activations, K contiguous) and B [K, N]
// (weights stored (in, out), N contiguous), fp32 accumulation.  It carries
// the block's four products: the Q/K/V projections (three problems sharing
// A in one launch), the output projection + first residual, MLP1 + GELU and
// MLP2 + second residual (crackedaicode.com "ViT Encoder Block",
// "Multi-head attention" and "Feed-forward stage").
//
// Design (gfx950, wave64):
// * v_mfma_f32_32x32x16_bf16: each wave owns a (32*TN) x (32*TM) block of
//   C^T, i.e. the weight tile is the MFMA's first operand and the activation
//   tile its second, so every accumulator lane holds 4 consecutive output
//   columns of one row and stores 8 contiguous bytes.
// * Both operands are staged in LDS as [row][64 k] bf16 with the 16-byte
//   chunk index XOR-swizzled by (row & 7), so the 32 rows a wave reads for
//   one MFMA operand spread over all banks.
// * The weights arrive N-major; each thread loads an 8 (k) x 8 (n) block with
//   eight 16-byte loads and transposes it in registers, so LDS holds both
//   operands K-contiguous and no separate transpose pass over HBM is needed.
// * Two LDS stages: the next k-slice is fetched into registers while the
//   MFMAs run on the current one, then written to the other stage; one
//   workgroup barrier per k-slice.
// * Tile order: workgroups are dispatched round-robin over the 8 XCDs, so the
//   linear workgroup id is remapped to give each XCD a contiguous run of
//   tiles, and that run is walked in groups of 8 M-tiles so that concurrently
//   resident tiles share A and B panels in the XCD's L2.
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kBK = 64;      // k per LDS stage (8 chunks of 8 bf16)
constexpr int kGroupM = 8;   // M-tiles per raster group
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies

template <int BM_, int BN_, int WM_, int WN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = WM * WN * 64;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;
  static constexpr int A_CHUNKS = BM * 8 / NT;       // 16-B chunks per thread per stage
  static constexpr int B_BLOCKS = (BN + NT - 1) / NT;  // 8x8 blocks per thread per stage
  static constexpr int LDS_A = BM * 8;               // uint4 per stage
  static constexpr int LDS_B = BN * 8;
  static_assert(BM * 8 % NT == 0, "A staging must divide evenly");
  static_assert(TM >= 1 && TN >= 1, "wave tile must hold at least one 32x32 block");
};

// Linear workgroup id -> (problem, m-tile, n-tile).
__device__ __forceinline__ void tile_of(int64_t bid, int64_t total, int64_t mt, int64_t nt,
                                        int* prob, int64_t* tm, int64_t* tn) {
  const int64_t q = total / kNumXcd, r = total % kNumXcd;
  const int64_t x = bid % kNumXcd, local = bid / kNumXcd;
  const int64_t b2 = x * q + (x < r ? x : r) + local;
  const int64_t per = mt * nt;
  *prob = static_cast<int>(b2 / per);
  const int64_t t = b2 % per;
  const int64_t gsz = static_cast<int64_t>(kGroupM) * nt;
  const int64_t first_m = (t / gsz) * kGroupM;
  const int64_t gm = (mt - first_m) < kGroupM ? (mt - first_m) : kGroupM;
  const int64_t w = t % gsz;
  *tm = first_m + w % gm;
  *tn = w / gm;
}

__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }

template <class C, int EPI>
__global__ __launch_bounds__(C::NT, 1) void gemm_bf16_kernel(GemmProblem p, int64_t mt,
                                                             int64_t nt) {
  // Stage st: A tile at lds + st*STAGE, B tile right after it.
  __shared__ uint4 lds[2 * (C::LDS_A + C::LDS_B)];
  constexpr int STAGE = C::LDS_A + C::LDS_B;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / C::WN, wn = wave % C::WN;
  int prob;
  int64_t tm, tn;
  tile_of(blockIdx.x, static_cast<int64_t>(gridDim.x), mt, nt, &prob, &tm, &tn);
  const int64_t m0 = tm * C::BM, n0 = tn * C::BN;

  const bf16_t* A = static_cast<const bf16_t*>(p.A);
  const bf16_t* B = static_cast<const bf16_t*>(p.B[prob]);
  const int64_t M = p.M, N = p.N, K = p.K;

  // Per-thread global source pointers (rows/columns clamped into range: the
  // values loaded for out-of-range rows or columns only reach outputs that
  // are never stored).
  const bf16_t* a_src[C::A_CHUNKS];
  int a_dst[C::A_CHUNKS];
#pragma unroll
  for (int i = 0; i < C::A_CHUNKS; ++i) {
    const int e = tid + i * C::NT;
    const int row = e >> 3, ch = e & 7;
    int64_t gm = m0 + row;
    gm = gm < M ? gm : M - 1;
    a_src[i] = A + gm * p.lda + ch * 8;
    a_dst[i] = swz(row, ch);
  }
  const bf16_t* b_src[C::B_BLOCKS];
  int b_nc[C::B_BLOCKS], b_kb[C::B_BLOCKS];
  bool b_on[C::B_BLOCKS];
#pragma unroll
  for (int i = 0; i < C::B_BLOCKS; ++i) {
    const int blk = tid + i * C::NT;
    b_on[i] = blk < C::BN;
    const int nc = blk % (C::BN / 8), kb = blk / (C::BN / 8);
    b_nc[i] = nc;
    b_kb[i] = kb;
    int64_t gn = n0 + nc * 8;
    gn = gn < N ? gn : N - 8;
    b_src[i] = B + static_cast<int64_t>(kb * 8) * p.ldb + gn;
  }

  uint4 ra[C::A_CHUNKS];
  uint4 rb[C::B_BLOCKS][8];

  auto fetch = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) ra[i] = ld_global16(a_src[i] + k0);
#pragma unroll
    for (int i = 0; i < C::B_BLOCKS; ++i) {
      if (!b_on[i]) continue;
#pragma unroll
      for (int r = 0; r < 8; ++r) rb[i][r] = ld_global16(b_src[i] + (k0 + r) * p.ldb);
    }
  };
  auto stash = [&](int st) {
#pragma unroll
    for (int i = 0; i < C::A_CHUNKS; ++i) lds[st * STAGE + a_dst[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < C::B_BLOCKS; ++i) {
      if (!b_on[i]) continue;
      uint4 tr[8];
      transpose8x8_b16(rb[i], tr);
#pragma unroll
      for (int j = 0; j < 8; ++j) lds[st * STAGE + C::LDS_A + swz(b_nc[i] * 8 + j, b_kb[i])] = tr[j];
    }
  };

  f32x16 acc[C::TN][C::TM];
#pragma unroll
  for (int j = 0; j < C::TN; ++j)
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  const int64_t KT = K / kBK;
  fetch(0);
  stash(0);
  __syncthreads();

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int64_t kt = 0; kt < KT; ++kt) {
    const int st = static_cast<int>(kt & 1);
    if (kt + 1 < KT) fetch((kt + 1) * kBK);
    const uint4* as = lds + st * STAGE;
    const uint4* bs = as + C::LDS_A;
#pragma unroll
    for (int s = 0; s < kBK / 16; ++s) {
      const int ch = 2 * s + lhalf;
      bf16x8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        const int row = wm * C::WTM + i * 32 + lrow;
        const uint4 u = as[swz(row, ch)];
        af[i] = __builtin_bit_cast(bf16x8, u);
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
        const int row = wn * C::WTN + j * 32 + lrow;
        const uint4 u = bs[swz(row, ch)];
        bf[j] = __builtin_bit_cast(bf16x8, u);
      }
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
          acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[j], af[i], acc[j][i], 0, 0, 0);
    }
    if (kt + 1 < KT) stash(st ^ 1);
    __syncthreads();
  }

  // Epilogue: accumulator element r of lane l in block (j, i) is
  // C[m0 + wm*WTM + i*32 + (l & 31)][n0 + wn*WTN + j*32 + (r/4)*8 + (l/32)*4 + r%4].
  bf16_t* Cp = static_cast<bf16_t*>(p.C);
  const bf16_t* Rp = static_cast<const bf16_t*>(p.R);
  const int64_t coff = p.col_off[prob];
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
          const uint2 rv = *reinterpret_cast<const uint2*>(Rp + m * p.ldr + coff + n);
          v[0] += __uint_as_float(rv.x << 16);
          v[1] += __uint_as_float(rv.x & 0xffff0000u);
          v[2] += __uint_as_float(rv.y << 16);
          v[3] += __uint_as_float(rv.y & 0xffff0000u);
        }
        if (EPI == VITBLK_EPI_GELU) {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = gelu_tanh_fast(v[e]);
        }
        *reinterpret_cast<uint2*>(Cp + m * p.ldc + coff + n) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

using BigTile = Cfg<256, 256, 2, 2>;  // 4 waves, 128x128 per wave

template <class C>
hipError_t launch_cfg(const GemmProblem& p, hipStream_t s) {
  const int64_t mt = (p.M + C::BM - 1) / C::BM, nt = (p.N + C::BN - 1) / C::BN;
  const int64_t blocks = mt * nt * p.nprob;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks)), block(C::NT);
  switch (p.epi) {
    case VITBLK_EPI_RESIDUAL:
      hipLaunchKernelGGL((gemm_bf16_kernel<C, VITBLK_EPI_RESIDUAL>), grid, block, 0, s, p, mt,
                         nt);
      break;
    case VITBLK_EPI_GELU:
      hipLaunchKernelGGL((gemm_bf16_kernel<C, VITBLK_EPI_GELU>), grid, block, 0, s, p, mt, nt);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_kernel<C, VITBLK_EPI_NONE>), grid, block, 0, s, p, mt, nt);
      break;
  }
  return hipGetLastError();
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

}  // namespace

hipError_t launch_gemm(const GemmProblem& p, hipStream_t s) {
  bool fast = p.dtype == VITBLK_BF16 && p.K % kBK == 0 && p.N % 8 == 0 && p.N >= 8 &&
              p.lda % 8 == 0 && p.ldb % 8 == 0 && p.ldc % 8 == 0 && aligned16(p.A) &&
              aligned16(p.C);
  if (p.epi == VITBLK_EPI_RESIDUAL) fast = fast && p.ldr % 8 == 0 && aligned16(p.R);
  for (int i = 0; i < p.nprob; ++i)
    fast = fast && aligned16(p.B[i]) && p.col_off[i] % 8 == 0;
  if (!fast) return launch_gemm_generic(p, s);
  return launch_cfg<BigTile>(p, s);
}

}  // namespace vitblk
