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
// position embeddings and the MFMA GEMM, pos_bias_kernel writes the class
// tokens and a table of position embedding plus bias, and the GEMM's token
// epilogue writes the patch tokens with that table added.
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
// VEC consecutive features per thread (VEC = 8 needs D % 8 == 0).
template <typename T, int VEC>
__global__ __launch_bounds__(256) void tokens_kernel(const T* __restrict__ emb,
                                                     const T* __restrict__ cls,
                                                     const T* __restrict__ pos,
                                                     T* __restrict__ out, int64_t B, int N,
                                                     int HC, int D) {
  const int Tn = N + HC;
  const int per_row = D / VEC;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e >= B * Tn * per_row) return;
  const int64_t row = e / per_row;
  const int d0 = static_cast<int>(e - row * per_row) * VEC;
  const int64_t b = row / Tn;
  const int t = static_cast<int>(row - b * Tn);
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

// Before the fused embedding product (bf16, D % 8 == 0, one 16-byte vector
// per thread): the position embedding plus patch bias, rounded once, pb[t] =
// pos[t] + b (b null: pos) for t < rows, and, if cls is given, the class-token
// rows out[i * Tn] = cls + pos[0] of the B images.
__global__ __launch_bounds__(256) void pos_bias_kernel(const bf16_t* __restrict__ pos,
                                                       const bf16_t* __restrict__ b,
                                                       bf16_t* __restrict__ pb, int64_t rows,
                                                       int D, const bf16_t* __restrict__ cls,
                                                       bf16_t* __restrict__ out, int64_t B,
                                                       int64_t Tn) {
  int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int per_row = D / 8;
  if (e >= rows * per_row) {  // a class-token row
    e -= rows * per_row;
    if (cls == nullptr || e >= B * per_row) return;
    const int64_t i = e / per_row;
    const int d0 = static_cast<int>(e - i * per_row) * 8;
    const uint4 cv = ld_global16(cls + d0), pv = ld_global16(pos + d0);
    const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w}, pw[4] = {pv.x, pv.y, pv.z, pv.w};
    uint32_t o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      o[k] = pack_bf16x2(__uint_as_float(cw[k] << 16) + __uint_as_float(pw[k] << 16),
                         __uint_as_float(cw[k] & 0xffff0000u) + __uint_as_float(pw[k] & 0xffff0000u));
    st_global16(out + i * Tn * D + d0, make_uint4(o[0], o[1], o[2], o[3]));
    return;
  }
  const int64_t t = e / per_row;
  const int d0 = static_cast<int>(e - t * per_row) * 8;
  const uint4 pv = ld_global16(pos + t * D + d0);
  const uint4 bv = b != nullptr ? ld_global16(b + d0) : make_uint4(0, 0, 0, 0);
  const uint32_t pw[4] = {pv.x, pv.y, pv.z, pv.w}, bw[4] = {bv.x, bv.y, bv.z, bv.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf16x2(__uint_as_float(pw[i] << 16) + __uint_as_float(bw[i] << 16),
                       __uint_as_float(pw[i] & 0xffff0000u) + __uint_as_float(bw[i] & 0xffff0000u));
  st_global16(pb + t * D + d0, make_uint4(o[0], o[1], o[2], o[3]));
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
  // tokens itself (each row into its token row) and only the class-token rows
  // remain.  Its epilogue adds one bf16 table, the position embeddings plus
  // the patch bias (their sum rounded once, into the then unused embedding
  // buffer, which holds it when B*N >= N + HC rows), so it carries no bias.
  GemmProblem gt = g;
  gt.epi = kEpiEmbed;
  gt.C = p.tokens;
  gt.R = p.embedded;
  gt.ldr = p.D;
  gt.bias[0] = nullptr;
  gt.row_group = N;
  gt.row_base = 0;
  gt.row_skip = HC;
  const bool fused = p.dtype == VITBLK_BF16 && p.pos != nullptr && p.D % 8 == 0 &&
                     rows >= N + HC && gemm_fast_ok(gt) &&
                     (reinterpret_cast<uintptr_t>(p.pos) & 15u) == 0 &&
                     (reinterpret_cast<uintptr_t>(p.b_patch) & 15u) == 0;
  if (fused) {  // the table, and the class-token rows (they do not need the product)
    hipLaunchKernelGGL(pos_bias_kernel, dim3(blocks_for((N + HC + HC * p.B) * (p.D / 8))),
                       dim3(256), 0, s, static_cast<const bf16_t*>(p.pos),
                       static_cast<const bf16_t*>(p.b_patch), static_cast<bf16_t*>(p.embedded),
                       static_cast<int64_t>(N + HC), static_cast<int>(p.D),
                       static_cast<const bf16_t*>(p.cls), static_cast<bf16_t*>(p.tokens), p.B,
                       static_cast<int64_t>(N + HC));
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_gemm(gt, s);
  }
  if ((e = launch_gemm(g, s)) != hipSuccess) return e;
  const int64_t toks = p.B * (N + HC);
  if (p.D % 8 == 0)
    hipLaunchKernelGGL((tokens_kernel<T, 8>), dim3(blocks_for(toks * (p.D / 8))), dim3(256), 0,
                       s, static_cast<const T*>(p.embedded), static_cast<const T*>(p.cls),
                       static_cast<const T*>(p.pos), static_cast<T*>(p.tokens), p.B, N, HC,
                       static_cast<int>(p.D));
  else
    hipLaunchKernelGGL((tokens_kernel<T, 1>), dim3(blocks_for(toks * p.D)), dim3(256), 0, s,
                       static_cast<const T*>(p.embedded), static_cast<const T*>(p.cls),
                       static_cast<const T*>(p.pos), static_cast<T*>(p.tokens), p.B, N, HC,
                       static_cast<int>(p.D));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_patch_embed(const PatchEmbedArgs& p, hipStream_t s) {
  return p.dtype == VITBLK_BF16 ? launch_typed<bf16_t>(p, s) : launch_typed<float>(p, s);
}

}  // namespace vitblk
