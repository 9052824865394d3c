// The ViT front end: patch extraction and token assembly around one GEMM
// (mlgrind.dev "E2E: Tiny Vision Transformer", "Architecture": patchify,
// @ W_patch + b_patch, prepend the class token, add position embeddings;
// "Details": patches row-major over the (H/P, W/P) grid, each flattened as
// (p1, p2, c)).
//
// patchify_band_kernel (or, for image rows that are not whole 16-byte
// vectors, patchify_kernel) writes the patches as GEMM rows [B*N, Kp] (Kp =
// P*P*C rounded up to 64 with zero columns, so the MFMA GEMM's k-slices tile it);
// the GEMM (bias epilogue) then embeds them into [B*N, D]; tokens_kernel
// writes the sequences [B, N (+1), D]: the class token (if any) as token 0,
// then the embedded patches, each plus its position embedding (if any).  With
// position embeddings and the MFMA GEMM, the GEMM's token epilogue writes the
// patch tokens (position embedding added) and tokens_kernel only the class
// tokens.
// All three are HBM-bound except the GEMM (MFMA).
#include "device.h"
#include "kernels.h"
#include "vitblk.h"

namespace vitblk {
namespace {

// Patch matrix a[row][k], row = b * N + cell, k = (p1 * P + p2) * C + c
// (< K) or a zero pad column (K <= k < Kp).  Each thread writes VEC = 16 /
// sizeof(T) consecutive k as one 16-byte store (Kp is a multiple of 64);
// it decodes (p1, p2, c) of its first k once and steps through the rest.
// Its reads fall in at most two image rows per channel, which the
// neighbouring threads of the same patch row also read (cache hits).
template <typename T>
__global__ __launch_bounds__(256) void patchify_kernel(const T* __restrict__ x,
                                                       T* __restrict__ a, int64_t total_vec,
                                                       int C, int H, int W, int P, int K,
                                                       int Kp) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= total_vec) return;
  const int vpr = Kp / VEC;  // vectors per row
  const int64_t row = e / vpr;
  const int k0 = static_cast<int>(e - row * vpr) * VEC;
  const int gw = W / P, cells = (H / P) * gw;
  const int64_t b = row / cells;
  const int cell = static_cast<int>(row - b * cells);
  const int gi = cell / gw, gj = cell - gi * gw;
  // pixel (p1, p2) of channel c of this patch: x + ((b*C + c)*H + gi*P + p1)*W + gj*P + p2
  const T* base = x + (b * C * H + static_cast<int64_t>(gi) * P) * W + static_cast<int64_t>(gj) * P;
  const int64_t plane = static_cast<int64_t>(H) * W;
  int c = k0 % C, pix = k0 / C;
  int p1 = pix / P, p2 = pix - p1 * P;
  T v[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    v[i] = (k0 + i < K) ? base[c * plane + static_cast<int64_t>(p1) * W + p2] : T(0);
    if (++c == C) {
      c = 0;
      if (++p2 == P) {
        p2 = 0;
        ++p1;
      }
    }
  }
  *reinterpret_cast<uint4*>(a + row * Kp + k0) = *reinterpret_cast<const uint4*>(v);
}

// The same patch matrix, one workgroup per band of P image rows (every
// channel) of one image: the band is read into LDS with 16-byte loads that
// follow the image rows, then its W/P patches leave as W/P consecutive rows of
// the patch matrix (one contiguous block), one 16-byte store per thread and
// vector.  Needs W a multiple of VEC, 16-byte-aligned images and C*P*W
// elements of LDS (at most 64 KB).
template <typename T>
__global__ __launch_bounds__(256) void patchify_band_kernel(const T* __restrict__ x,
                                                            T* __restrict__ a, int C, int H,
                                                            int W, int P, int K, int Kp) {
  constexpr int VEC = 16 / sizeof(T);
  extern __shared__ __attribute__((aligned(16))) char band_raw[];
  T* const band = reinterpret_cast<T*>(band_raw);  // [C][P][W]
  const int gh = H / P, gw = W / P;
  const int64_t b = blockIdx.x / gh;
  const int gi = static_cast<int>(blockIdx.x % gh);
  const int vrow = W / VEC;  // 16-byte vectors per image row
  for (int e = threadIdx.x; e < C * P * vrow; e += 256) {
    const int r = e / vrow, v = e - r * vrow;  // r = c * P + p1
    const int c = r / P, p1 = r - c * P;
    const T* src = x + ((b * C + c) * H + static_cast<int64_t>(gi) * P + p1) * W + v * VEC;
    *reinterpret_cast<uint4*>(band + r * W + v * VEC) = *reinterpret_cast<const uint4*>(src);
  }
  __syncthreads();
  const int vpr = Kp / VEC;  // vectors per patch row
  T* const dst = a + (b * gh + gi) * static_cast<int64_t>(gw) * Kp;  // the band's first patch
  for (int e = threadIdx.x; e < gw * vpr; e += 256) {
    const int gj = e / vpr, k0 = (e - gj * vpr) * VEC;
    int c = k0 % C, pix = k0 / C;
    int p1 = pix / P, p2 = pix - p1 * P;
    T v[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      v[i] = (k0 + i < K) ? band[(c * P + p1) * W + gj * P + p2] : T(0);
      if (++c == C) {
        c = 0;
        if (++p2 == P) {
          p2 = 0;
          ++p1;
        }
      }
    }
    *reinterpret_cast<uint4*>(dst + static_cast<int64_t>(gj) * Kp + k0) =
        *reinterpret_cast<const uint4*>(v);
  }
}

// Zero columns [K, Kp) of every row of w_t [rows, Kp] (the packed weight's
// padding; the pack kernel writes columns [0, K)).
template <typename T>
__global__ __launch_bounds__(256) void zero_pad_kernel(T* __restrict__ w, int64_t rows, int K,
                                                       int Kp) {
  const int pad = Kp - K;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= rows * pad) return;
  const int64_t r = e / pad;
  w[r * Kp + K + (e - r * pad)] = T(0);
}

// Token rows: out[b, t, :] = (t < HC ? cls : emb[b * N + t - HC]) + pos[t], for
// t < t_end (N + HC: every row; HC: the class-token rows only, when the
// embedding product wrote the others), VEC consecutive features per thread
// (VEC = 8 needs D % 8 == 0).
template <typename T, int VEC>
__global__ __launch_bounds__(256) void tokens_kernel(const T* __restrict__ emb,
                                                     const T* __restrict__ cls,
                                                     const T* __restrict__ pos,
                                                     T* __restrict__ out, int64_t B, int N,
                                                     int HC, int D, int t_end) {
  const int Tn = N + HC;
  const int per_row = D / VEC;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= B * t_end * per_row) return;
  const int64_t r = e / per_row;
  const int d0 = static_cast<int>(e - r * per_row) * VEC;
  const int64_t b = r / t_end;
  const int t = static_cast<int>(r - b * t_end);
  const int64_t row = b * Tn + t;
  const T* src = t < HC ? cls + d0 : emb + (b * N + t - HC) * D + d0;
  float v[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) v[i] = load_f32(src + i);
  if (pos != nullptr) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v[i] += load_f32(pos + static_cast<int64_t>(t) * D + d0 + i);
  }
#pragma unroll
  for (int i = 0; i < VEC; ++i) store_f32(out + row * D + d0 + i, v[i]);
}

unsigned blocks_for(int64_t n) { return static_cast<unsigned>((n + 255) / 256); }

template <typename T>
hipError_t launch_typed(const PatchEmbedArgs& p, hipStream_t s) {
  const int K = static_cast<int>(p.P * p.P * p.C), Kp = static_cast<int>(p.Kp);
  const int N = static_cast<int>((p.H / p.P) * (p.W / p.P));
  const int64_t rows = p.B * N;
  // W_patch [K, D] -> out-major [D, Kp], pad columns zero.
  const PackJob job{p.w_patch, K, p.D, p.w_t, Kp};
  hipError_t e = launch_pack(&job, 1, p.dtype, s);
  if (e != hipSuccess) return e;
  if (Kp > K) {
    hipLaunchKernelGGL(zero_pad_kernel<T>, dim3(blocks_for(p.D * (Kp - K))), dim3(256), 0, s,
                       static_cast<T*>(p.w_t), p.D, K, Kp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  constexpr int VEC = 16 / sizeof(T);
  const int64_t band_bytes = p.C * p.P * p.W * static_cast<int64_t>(sizeof(T));
  const bool banded = p.W % VEC == 0 && band_bytes <= 64 * 1024 &&
                      (reinterpret_cast<uintptr_t>(p.images) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.patches) & 15u) == 0 &&
                      p.B * (p.H / p.P) <= 2147483647LL;
  if (banded)
    hipLaunchKernelGGL(patchify_band_kernel<T>, dim3(static_cast<unsigned>(p.B * (p.H / p.P))),
                       dim3(256), static_cast<size_t>(band_bytes), s,
                       static_cast<const T*>(p.images), static_cast<T*>(p.patches),
                       static_cast<int>(p.C), static_cast<int>(p.H), static_cast<int>(p.W),
                       static_cast<int>(p.P), K, Kp);
  else
    hipLaunchKernelGGL(patchify_kernel<T>, dim3(blocks_for(rows * Kp / VEC)), dim3(256), 0, s,
                       static_cast<const T*>(p.images), static_cast<T*>(p.patches),
                       rows * Kp / VEC,
                       static_cast<int>(p.C), static_cast<int>(p.H), static_cast<int>(p.W),
                       static_cast<int>(p.P), K, Kp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  GemmProblem g{};
  g.M = rows;
  g.N = p.D;
  g.K = Kp;
  g.A = p.patches;
  g.lda = Kp;
  g.B = p.w_t;
  g.ldb = Kp;
  g.C = p.embedded;
  g.ldc = p.D;
  g.epi = VITBLK_EPI_NONE;
  g.dtype = p.dtype;
  g.bias[0] = p.b_patch;
  g.bias_seg = p.D;
  const int HC = p.cls != nullptr ? 1 : 0;
  // With position embeddings on the MFMA kernel, the product writes the patch
  // tokens itself (each row into its token row, the position embedding added
  // before the one rounding) and only the class-token rows remain.
  GemmProblem gt = g;
  gt.epi = kEpiEmbed;
  gt.C = p.tokens;
  gt.R = p.pos;
  gt.ldr = p.D;
  gt.row_group = N;
  gt.row_base = 0;
  gt.row_skip = HC;
  const bool fused = p.pos != nullptr && gemm_fast_ok(gt);
  if ((e = launch_gemm(fused ? gt : g, s)) != hipSuccess) return e;
  const int t_end = fused ? HC : N + HC;
  if (t_end == 0) return hipSuccess;
  const int64_t toks = p.B * t_end;
  if (p.D % 8 == 0)
    hipLaunchKernelGGL((tokens_kernel<T, 8>), dim3(blocks_for(toks * (p.D / 8))), dim3(256), 0,
                       s, static_cast<const T*>(p.embedded), static_cast<const T*>(p.cls),
                       static_cast<const T*>(p.pos), static_cast<T*>(p.tokens), p.B, N, HC,
                       static_cast<int>(p.D), t_end);
  else
    hipLaunchKernelGGL((tokens_kernel<T, 1>), dim3(blocks_for(toks * p.D)), dim3(256), 0, s,
                       static_cast<const T*>(p.embedded), static_cast<const T*>(p.cls),
                       static_cast<const T*>(p.pos), static_cast<T*>(p.tokens), p.B, N, HC,
                       static_cast<int>(p.D), t_end);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_patch_embed(const PatchEmbedArgs& p, hipStream_t s) {
  return p.dtype == VITBLK_BF16 ? launch_typed<bf16_t>(p, s) : launch_typed<float>(p, s);
}

}  // namespace vitblk
