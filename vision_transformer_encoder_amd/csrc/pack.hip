// Weight packing: (in, out) weights -> out-major copies, dst[c][r] = src[r][c],
// and the fused prologue of a block call (the transposes, the LayerNorm
// fold's column sums and the first LayerNorm's row statistics in one launch).
//
// The block's weights are applied as x @ W with W stored (in_features,
// out_features) (crackedaicode.com "ViT Encoder Block", "Inputs and output").
// The GEMM kernels want both operands contiguous along the reduction axis,
// so each call first writes W^T once (an HBM-bound transpose of all six
// weights, one launch).
// bf16 weights whose sides are multiples of 8: each lane moves one 8 x 8
// block, eight 16-byte row loads, an in-register transpose, eight 16-byte
// column stores; a wave covers a 64 x 64 tile, so each group of 8 lanes
// reads and writes whole 128-byte segments.  Other shapes and fp32: 64 x 64
// tiles through LDS (padded by one element so the column-wise reads fall in
// distinct banks).
#include "device.h"
#include "kernels.h"
#include "row_stats.h"
#include "vitblk.h"

namespace vitblk {
namespace {

constexpr int kMaxJobs = 6;

struct PackArgs {
  PackJob job[kMaxJobs];
  int64_t tiles_c[kMaxJobs];  // 64-wide column tiles per job
};

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  __shared__ T tile[64][65];
  const PackJob& j = a.job[blockIdx.y];
  const int64_t tc = a.tiles_c[blockIdx.y];
  const int64_t b = blockIdx.x;
  const int64_t r0 = (b / tc) * 64, c0 = (b % tc) * 64;
  if (r0 >= j.rows) return;  // whole workgroup: this job has fewer tiles
  const T* src = static_cast<const T*>(j.src);
  T* dst = static_cast<T*>(j.dst);
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = tid + i * 256, r = e >> 6, c = e & 63;
    if (r0 + r < j.rows && c0 + c < j.cols) tile[r][c] = src[(r0 + r) * j.cols + c0 + c];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int e = tid + i * 256, c = e >> 6, r = e & 63;
    if (r0 + r < j.rows && c0 + c < j.cols) dst[(c0 + c) * j.ldd + r0 + r] = tile[r][c];
  }
}

// One wave per 64 x 64 tile, four tiles per workgroup; lane (br, bc) =
// (lane / 8, lane % 8) moves rows br*8..+7, columns bc*8..+7.
__global__ __launch_bounds__(256) void pack_blocks_kernel(PackArgs a) {
  const PackJob& j = a.job[blockIdx.y];
  const int64_t tc = a.tiles_c[blockIdx.y];
  const int64_t b = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int64_t r0 = (b / tc) * 64, c0 = (b % tc) * 64;
  if (r0 >= j.rows) return;  // this job has fewer tiles
  const int lane = threadIdx.x & 63;
  const int64_t r = r0 + (lane >> 3) * 8, c = c0 + (lane & 7) * 8;
  if (r >= j.rows || c >= j.cols) return;  // sides are multiples of 8: whole blocks
  const bf16_t* src = static_cast<const bf16_t*>(j.src) + r * j.cols + c;
  uint4 in[8], out[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) in[k] = ld_global16(src + k * j.cols);
  transpose8x8_b16(in, out);
  bf16_t* dst = static_cast<bf16_t*>(j.dst) + c * j.ldd + r;
#pragma unroll
  for (int k = 0; k < 8; ++k) st_global16(dst + k * j.ldd, out[k]);
}

// Row sums of the packed out-major weights, sums[r] = sum_c src[r][c]: the
// column sums of the (in, out) weights that the LayerNorm fold needs.  One
// wave per row, four rows per workgroup.  bf16 rows whose length is a
// multiple of 8 (16-byte aligned) are read 8 elements per lane and load:
// lane l adds chunks l, l + 64, ... in order; otherwise single elements.
// The wave reduction is a fixed tree, so every call gives the same bits.
struct RowSumArgs {
  RowSumJob job[2];
};

template <typename T, bool VEC>
__global__ __launch_bounds__(256) void row_sums_kernel(RowSumArgs a) {
  const RowSumJob& j = a.job[blockIdx.y];
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= j.rows) return;  // whole wave
  const int lane = threadIdx.x & 63;
  const T* src = static_cast<const T*>(j.src) + r * j.cols;
  float s = 0.f;
  if (VEC) {
    for (int64_t c = lane * 8; c < j.cols; c += 512) {
      const uint4 u = ld_global16(src + c);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
        s += __uint_as_float(w[e] << 16) + __uint_as_float(w[e] & 0xffff0000u);
    }
  } else {
    for (int64_t c = lane; c < j.cols; c += 64) s += load_f32(src + c);
  }
  s = wave_sum(s);
  if (lane == 0) j.sums[r] = s;
}

bool blocks_ok(const PackJob& j) {
  return j.rows % 8 == 0 && j.cols % 8 == 0 && j.ldd % 8 == 0 &&
         (reinterpret_cast<uintptr_t>(j.src) & 15u) == 0 &&
         (reinterpret_cast<uintptr_t>(j.dst) & 15u) == 0;
}

// ---------------------------------------------------------------- fused prologue
//
// The transposes, the column sums and the first LayerNorm's statistics are
// independent HBM-bound passes (the column sums are taken from the source
// weights, not the transposed copies); as three launches each pays its own
// fill and drain, with few bytes in flight at its start and end.  One launch
// gives every workgroup one role by its index: the column sums first (few
// workgroups, each a long loop), then the transposes, then the statistics
// rows, so the long work starts early and the many short statistics
// workgroups fill the end.
//
// Column sums: a workgroup owns 64 columns; thread t adds rows t/8, t/8 + 32,
// ... of columns 8 (t % 8) .. + 7 (16-byte loads: a wave reads 8 rows x 128
// contiguous bytes per step), then the 32 partial sums of each column are
// added in order through LDS.  Fixed order: every call gives the same bits.
constexpr int kColsPerBlock = 64;
constexpr int kColSlices = 32;  // rows handled in parallel per column group

struct PrologueArgs {
  PackJob job[kMaxJobs];
  int64_t tiles_c[kMaxJobs];
  int64_t tile_end[kMaxJobs];  // 64 x 64 tiles of jobs 0 .. i
  int njobs;
  ColSumJob cs[4];
  int64_t cs_end[4];  // column-sum workgroups of jobs 0 .. i
  int ncs;
  const bf16_t* x;
  int64_t ld, rows;
  float2* stats;
  int D;
  float eps;
  int64_t cs_blocks, pack_blocks;  // role boundaries (workgroups)
};

__device__ __forceinline__ void colsum_block(const PrologueArgs& a, int64_t b) {
  __shared__ float part[kColSlices][kColsPerBlock];
  int j = 0;
  while (j + 1 < a.ncs && b >= a.cs_end[j]) ++j;
  const ColSumJob& c = a.cs[j];
  const int64_t c0 = (b - (j > 0 ? a.cs_end[j - 1] : 0)) * kColsPerBlock;
  const int t = threadIdx.x, cg = t & 7, ks = t >> 3;
  const int64_t col = c0 + cg * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (col < c.cols) {  // cols is a multiple of 8: whole groups
    const bf16_t* src = static_cast<const bf16_t*>(c.src) + col;
    int64_t r = ks;
    for (; r + 3 * kColSlices < c.rows; r += 4 * kColSlices) {
      uint4 u[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) u[k] = ld_global16(src + (r + k * kColSlices) * c.cols);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t w[4] = {u[k].x, u[k].y, u[k].z, u[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(w[e] << 16);
          acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
        }
      }
    }
    for (; r < c.rows; r += kColSlices) {
      const uint4 u = ld_global16(src + r * c.cols);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(w[e] << 16);
        acc[2 * e + 1] += __uint_as_float(w[e] & 0xffff0000u);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[ks][cg * 8 + e] = acc[e];
  __syncthreads();  // every thread of the workgroup reaches it (role is per workgroup)
  if (t < kColsPerBlock && c0 + t < c.cols) {
    float sum = 0.f;
#pragma unroll
    for (int k = 0; k < kColSlices; ++k) sum += part[k][t];
    c.sums[c0 + t] = sum;
  }
}

__device__ __forceinline__ void pack_wave(const PrologueArgs& a, int64_t w, int lane) {
  int j = 0;
  while (j + 1 < a.njobs && w >= a.tile_end[j]) ++j;
  if (w >= a.tile_end[j]) return;  // past the last job's tiles
  const PackJob& jb = a.job[j];
  const int64_t b = w - (j > 0 ? a.tile_end[j - 1] : 0);
  const int64_t tc = a.tiles_c[j];
  const int64_t r = (b / tc) * 64 + (lane >> 3) * 8, c = (b % tc) * 64 + (lane & 7) * 8;
  if (r >= jb.rows || c >= jb.cols) return;  // sides are multiples of 8: whole blocks
  const bf16_t* src = static_cast<const bf16_t*>(jb.src) + r * jb.cols + c;
  uint4 in[8], out[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) in[k] = ld_global16(src + k * jb.cols);
  transpose8x8_b16(in, out);
  bf16_t* dst = static_cast<bf16_t*>(jb.dst) + c * jb.ldd + r;
#pragma unroll
  for (int k = 0; k < 8; ++k) st_global16(dst + k * jb.ldd, out[k]);
}

template <int NCH>
__global__ __launch_bounds__(256) void prologue_kernel(PrologueArgs a) {
  const int64_t b = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (b < a.cs_blocks) {
    colsum_block(a, b);
  } else if (b < a.cs_blocks + a.pack_blocks) {
    pack_wave(a, (b - a.cs_blocks) * 4 + wave, lane);
  } else {
    const int64_t row = (b - a.cs_blocks - a.pack_blocks) * 4 + wave;
    if (row < a.rows) stats_of_row<bf16_t, NCH>(a.x, a.ld, a.stats, row, a.D, a.eps, lane);
  }
}

}  // namespace

hipError_t launch_pack(const PackJob* jobs, int njobs, int dtype, hipStream_t s) {
  if (njobs < 1 || njobs > kMaxJobs) return hipErrorInvalidValue;
  PackArgs a{};
  int64_t max_tiles = 0;
  for (int i = 0; i < njobs; ++i) {
    a.job[i] = jobs[i];
    a.tiles_c[i] = (jobs[i].cols + 63) / 64;
    const int64_t t = a.tiles_c[i] * ((jobs[i].rows + 63) / 64);
    max_tiles = t > max_tiles ? t : max_tiles;
  }
  if (max_tiles > 2147483647LL) return hipErrorInvalidValue;
  bool blocks = dtype == VITBLK_BF16;
  for (int i = 0; i < njobs; ++i) blocks = blocks && blocks_ok(jobs[i]);
  if (blocks) {
    const dim3 grid(static_cast<unsigned>((max_tiles + 3) / 4), static_cast<unsigned>(njobs));
    hipLaunchKernelGGL(pack_blocks_kernel, grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>(max_tiles), static_cast<unsigned>(njobs));
  if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL(pack_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_row_sums(const RowSumJob* jobs, int njobs, int dtype, hipStream_t s) {
  if (njobs < 1 || njobs > 2) return hipErrorInvalidValue;
  RowSumArgs a{};
  int64_t max_rows = 0;
  for (int i = 0; i < njobs; ++i) {
    a.job[i] = jobs[i];
    max_rows = jobs[i].rows > max_rows ? jobs[i].rows : max_rows;
  }
  const int64_t blocks = (max_rows + 3) / 4;
  if (blocks > 2147483647LL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(blocks), static_cast<unsigned>(njobs));
  bool vec = dtype == VITBLK_BF16;
  for (int i = 0; i < njobs; ++i)
    vec = vec && jobs[i].cols % 8 == 0 && (reinterpret_cast<uintptr_t>(jobs[i].src) & 15u) == 0;
  if (vec)
    hipLaunchKernelGGL((row_sums_kernel<bf16_t, true>), grid, dim3(256), 0, s, a);
  else if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL((row_sums_kernel<bf16_t, false>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((row_sums_kernel<float, false>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_prologue(const PackJob* jobs, int njobs, const ColSumJob* cs, int ncs,
                           const StatsJob* st, int dtype, hipStream_t s) {
  if (dtype != VITBLK_BF16 || njobs < 1 || njobs > kMaxJobs || ncs < 0 || ncs > 4)
    return hipErrorNotSupported;
  PrologueArgs a{};
  a.njobs = njobs;
  int64_t tiles = 0;
  for (int i = 0; i < njobs; ++i) {
    if (!blocks_ok(jobs[i])) return hipErrorNotSupported;
    a.job[i] = jobs[i];
    a.tiles_c[i] = (jobs[i].cols + 63) / 64;
    tiles += a.tiles_c[i] * ((jobs[i].rows + 63) / 64);
    a.tile_end[i] = tiles;
  }
  a.ncs = ncs;
  int64_t csb = 0;
  for (int i = 0; i < ncs; ++i) {
    if (cs[i].cols % 8 != 0 || (reinterpret_cast<uintptr_t>(cs[i].src) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(cs[i].sums) & 3u) != 0)
      return hipErrorNotSupported;
    a.cs[i] = cs[i];
    csb += (cs[i].cols + kColsPerBlock - 1) / kColsPerBlock;
    a.cs_end[i] = csb;
  }
  int nch = 1;
  int64_t stats_blocks = 0;
  if (st != nullptr && st->rows > 0) {
    if (st->D % 8 != 0 || st->ld % 8 != 0 || st->D > 64 * 8 * 8 ||
        (reinterpret_cast<uintptr_t>(st->x) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(st->stats) & 7u) != 0)
      return hipErrorNotSupported;
    a.x = static_cast<const bf16_t*>(st->x);
    a.ld = st->ld;
    a.rows = st->rows;
    a.stats = reinterpret_cast<float2*>(st->stats);
    a.D = static_cast<int>(st->D);
    a.eps = st->eps;
    stats_blocks = (st->rows + 3) / 4;
    const int cpl = static_cast<int>((st->D / 8 + 63) / 64);
    nch = cpl <= 1 ? 1 : cpl <= 2 ? 2 : cpl <= 4 ? 4 : 8;
  }
  a.cs_blocks = csb;
  a.pack_blocks = (tiles + 3) / 4;
  const int64_t blocks = a.cs_blocks + a.pack_blocks + stats_blocks;
  if (blocks > 2147483647LL) return hipErrorNotSupported;
  const dim3 grid(static_cast<unsigned>(blocks)), block(256);
  switch (nch) {
    case 1: hipLaunchKernelGGL(prologue_kernel<1>, grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL(prologue_kernel<2>, grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL(prologue_kernel<4>, grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL(prologue_kernel<8>, grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

}  // namespace vitblk
