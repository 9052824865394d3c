// fp32 products on the gfx950 matrix cores: C = epi(A @ B^T) with A [M, K]
// and B [N, K] both K-contiguous (the packed weight layout), fp32 in, fp32
// out, every product and sum in fp32 (v_mfma_f32_32x32x2_f32 multiplies and
// accumulates in full fp32; the fp32 tolerance rules out bf16 operands).
//
// The block's products (crackedaicode.com "ViT Encoder Block": the Q, K, V
// projections, the output projection, the two MLP layers) in fp32 mode, and
// the backward's data-gradient products, with the same epilogues as the
// any-shape VALU kernel (generic.hip), applied in the same order: LayerNorm
// fold, bias, residual or derivative factor, GELU.
//
// 128 x 128 output tile per workgroup, 4 waves of 64 x 64 (2 x 2 blocks of
// 32 x 32), k-slices of 32 staged through two LDS stages: each thread
// requests its share of the next slice into registers before the current
// slice's MFMAs and writes it to the other stage after them; one barrier per
// slice.  LDS rows are padded to 36 floats so the 16-byte fragment reads of
// any 16 consecutive rows cover all 64 banks once.  A lane's 16-byte read
// holds 4 consecutive k of one row; MFMA step s of a read pairs k = 8q + s
// (lanes 0-31) with k = 8q + 4 + s (lanes 32-63), the same pairing for both
// operands, so every k is summed exactly once.
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kBM = 128, kBN = 128, kBK = 32;
constexpr int kThreads = 256;                      // 4 waves, 2 x 2
constexpr int kRow = kBK + 4;                      // LDS row stride, floats
constexpr int kStage = (kBM + kBN) * kRow;         // floats per stage
constexpr int kLoads = kBM * (kBK / 4) / kThreads;  // 16-byte chunks per thread per operand
static_assert(kBM == kBN && kLoads * kThreads * 4 == kBM * kBK, "load split");

template <int EPI, bool BIAS, bool NORM>
__global__ __launch_bounds__(kThreads, 2) void gemm_f32_mfma_kernel(GemmProblem p, int nt) {
  __shared__ __attribute__((aligned(16))) float lds[2 * kStage];  // 73,728 B
  const int64_t tile = blockIdx.x;
  const int64_t m0 = (tile / nt) * kBM, n0 = (tile % nt) * kBN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const float* A = static_cast<const float*>(p.A);
  const float* B = static_cast<const float*>(p.B);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lh = lane >> 5;

  // Loads: chunk e = tid + 256 i is row e / 8, floats 4 (e % 8) .. +3 of the
  // slice.  Rows past M or N are clamped (they only reach outputs that are
  // never stored); chunks past K are zero (K is a multiple of 4).
  const float* a_src[kLoads];
  const float* b_src[kLoads];
  const int c4 = 4 * (tid & 7);
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int row = (tid + i * kThreads) >> 3;
    const int64_t ra = m0 + row < M ? m0 + row : M - 1;
    const int64_t rb = n0 + row < N ? n0 + row : N - 1;
    a_src[i] = A + ra * p.lda + c4;
    b_src[i] = B + rb * p.ldb + c4;
  }
  f32x4 ra[kLoads], rb[kLoads];
  auto fetch = [&](int kt) {
    const int64_t k = static_cast<int64_t>(kt) * kBK;
    const bool in = k + c4 < K;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      ra[i] = in ? *reinterpret_cast<const f32x4*>(a_src[i] + k) : f32x4{0.f, 0.f, 0.f, 0.f};
      rb[i] = in ? *reinterpret_cast<const f32x4*>(b_src[i] + k) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto stash = [&](int st) {
    float* as = lds + st * kStage;
    float* bs = as + kBM * kRow;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int row = (tid + i * kThreads) >> 3;
      *reinterpret_cast<f32x4*>(as + row * kRow + c4) = ra[i];
      *reinterpret_cast<f32x4*>(bs + row * kRow + c4) = rb[i];
    }
  };

  // acc[j][i]: n-block j, m-block i of the wave.  Element r of lane l is
  // C[m0 + 64 wm + 32 i + (l & 31)][n0 + 64 wn + 32 j + 8 (r / 4) + 4 (l / 32) + r % 4].
  f32x16 acc[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  const int KT = static_cast<int>((K + kBK - 1) / kBK);
  const int a_rd = (wm * 64 + l32) * kRow + 4 * lh;
  const int b_rd = (wn * 64 + l32) * kRow + 4 * lh;
  if (KT > 0) {
    fetch(0);
    stash(0);
  }
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt & 1;
    if (kt + 1 < KT) fetch(kt + 1);
    const float* as = lds + st * kStage;
    const float* bs = as + kBM * kRow;
#pragma unroll
    for (int q = 0; q < kBK / 8; ++q) {
      f32x4 af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const f32x4*>(as + a_rd + i * 32 * kRow + 8 * q);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const f32x4*>(bs + b_rd + j * 32 * kRow + 8 * q);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x2f32(bf[j][s], af[i][s], acc[j][i], 0,
                                                              0, 0);
    }
    if (kt + 1 < KT) stash(st ^ 1);
    __syncthreads();
  }

  // Epilogue, per run of 4 columns (N is a multiple of 4, so a run is wholly
  // inside or outside N).
  float* C = static_cast<float*>(p.C);
  const float* R = static_cast<const float*>(p.R);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t m = m0 + wm * 64 + i * 32 + l32;
    if (m >= M) continue;
    float mu = 0.f, rs = 1.f;
    if (NORM) {
      const float2 st = *reinterpret_cast<const float2*>(p.row_stats + 2 * m);
      mu = st.x;
      rs = st.y;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int64_t n = n0 + wn * 64 + j * 32 + 8 * b + 4 * lh;
        if (n >= N) continue;
        float v[4] = {acc[j][i][4 * b], acc[j][i][4 * b + 1], acc[j][i][4 * b + 2],
                      acc[j][i][4 * b + 3]};
        if (NORM) {  // LN(A) @ W = rstd (A @ W - mean colsum)
          const f32x4 cs = *reinterpret_cast<const f32x4*>(p.col_sums + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = rs * (v[e] - mu * cs[e]);
        }
        if (BIAS) {
          const int64_t seg = n / p.bias_seg;
          const void* bp = seg == 0 ? p.bias[0] : (seg == 1 ? p.bias[1] : p.bias[2]);
          if (bp != nullptr) {
            const f32x4 bv =
                *reinterpret_cast<const f32x4*>(static_cast<const float*>(bp) + (n - seg * p.bias_seg));
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += bv[e];
          }
        }
        f32x4 rv = {0.f, 0.f, 0.f, 0.f};
        if (EPI == VITBLK_EPI_RESIDUAL || EPI == VITBLK_EPI_GELU_GRAD || EPI == kEpiMul)
          rv = *reinterpret_cast<const f32x4*>(R + m * p.ldr + n);
        f32x4 d2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (EPI == VITBLK_EPI_RESIDUAL) v[e] += rv[e];
          if (EPI == VITBLK_EPI_GELU_GRAD) v[e] *= gelu_tanh_grad_precise(rv[e]);
          if (EPI == kEpiMul) v[e] *= rv[e];
          if (EPI == kEpiGeluDual) {
            d2[e] = gelu_tanh_grad_precise(v[e]);
            v[e] = gelu_tanh_precise(v[e]);
          }
          if (EPI == VITBLK_EPI_GELU) v[e] = gelu_tanh_precise(v[e]);
        }
        if (EPI == kEpiGeluDual)
          *reinterpret_cast<f32x4*>(static_cast<float*>(p.C2) + m * p.ldc + n) = d2;
        *reinterpret_cast<f32x4*>(C + m * p.ldc + n) = f32x4{v[0], v[1], v[2], v[3]};
      }
  }
}

bool al16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

template <int EPI, bool BIAS, bool NORM>
hipError_t launch_f32(const GemmProblem& p, int64_t mt, int64_t nt, hipStream_t s) {
  hipLaunchKernelGGL((gemm_f32_mfma_kernel<EPI, BIAS, NORM>), dim3(static_cast<unsigned>(mt * nt)),
                     dim3(kThreads), 0, s, p, static_cast<int>(nt));
  return hipGetLastError();
}

template <bool BIAS, bool NORM>
hipError_t launch_f32_epi(const GemmProblem& p, int64_t mt, int64_t nt, hipStream_t s) {
  switch (p.epi) {
    case VITBLK_EPI_RESIDUAL: return launch_f32<VITBLK_EPI_RESIDUAL, BIAS, NORM>(p, mt, nt, s);
    case VITBLK_EPI_GELU: return launch_f32<VITBLK_EPI_GELU, BIAS, NORM>(p, mt, nt, s);
    case VITBLK_EPI_GELU_GRAD: return launch_f32<VITBLK_EPI_GELU_GRAD, BIAS, NORM>(p, mt, nt, s);
    case kEpiGeluDual: return launch_f32<kEpiGeluDual, BIAS, NORM>(p, mt, nt, s);
    case kEpiMul: return launch_f32<kEpiMul, BIAS, NORM>(p, mt, nt, s);
    default: return launch_f32<VITBLK_EPI_NONE, BIAS, NORM>(p, mt, nt, s);
  }
}

}  // namespace

// The fp32 matrix-core product.  Needs 16-byte-aligned operands and rows
// (K, N, every leading dimension a multiple of 4 floats), a bias in segments
// of a multiple of 4 columns, and one of the epilogues above; otherwise it
// launches nothing and returns hipErrorNotSupported (the caller then takes
// the any-shape VALU kernel).
hipError_t launch_gemm_f32_mfma(const GemmProblem& p, hipStream_t s) {
  if (p.dtype != VITBLK_FP32 || p.M <= 0 || p.N <= 0 || p.K < 0) return hipErrorNotSupported;
  const bool known = p.epi == VITBLK_EPI_NONE || p.epi == VITBLK_EPI_RESIDUAL ||
                     p.epi == VITBLK_EPI_GELU || p.epi == VITBLK_EPI_GELU_GRAD ||
                     p.epi == kEpiGeluDual || p.epi == kEpiMul;
  bool ok = known && p.K % 4 == 0 && p.N % 4 == 0 && p.lda % 4 == 0 && p.ldb % 4 == 0 &&
            p.ldc % 4 == 0 && al16(p.A) && al16(p.B) && al16(p.C);
  if (reads_r(p)) ok = ok && p.R != nullptr && p.ldr % 4 == 0 && al16(p.R);
  if (p.epi == kEpiGeluDual) ok = ok && p.C2 != nullptr && al16(p.C2);
  const bool norm = p.row_stats != nullptr;
  if (norm)
    ok = ok && p.col_sums != nullptr && (p.epi == VITBLK_EPI_NONE || p.epi == VITBLK_EPI_GELU) &&
         (reinterpret_cast<uintptr_t>(p.row_stats) & 7u) == 0 && al16(p.col_sums);
  const bool bias = has_bias(p);
  if (bias) {
    ok = ok && p.bias_seg > 0 && p.bias_seg % 4 == 0 && p.N <= 3 * p.bias_seg;
    for (const void* b : p.bias) ok = ok && (b == nullptr || al16(b));
  }
  const int64_t mt = (p.M + kBM - 1) / kBM, nt = (p.N + kBN - 1) / kBN;
  if (!ok || mt * nt > 2147483647LL) return hipErrorNotSupported;
  if (norm) {  // epilogues NONE and GELU only (checked above)
    if (p.epi == VITBLK_EPI_GELU)
      return bias ? launch_f32<VITBLK_EPI_GELU, true, true>(p, mt, nt, s)
                  : launch_f32<VITBLK_EPI_GELU, false, true>(p, mt, nt, s);
    return bias ? launch_f32<VITBLK_EPI_NONE, true, true>(p, mt, nt, s)
                : launch_f32<VITBLK_EPI_NONE, false, true>(p, mt, nt, s);
  }
  return bias ? launch_f32_epi<true, false>(p, mt, nt, s) : launch_f32_epi<false, false>(p, mt, nt, s);
}

}  // namespace vitblk
