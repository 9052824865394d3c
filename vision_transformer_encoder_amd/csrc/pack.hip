// Weight packing: (in, out) weights -> out-major copies, dst[c][r] = src[r][c].
//
// The block's weights are applied as x @ W with W stored (in_features,
// out_features) (crackedaicode.com "ViT Encoder Block", "Inputs and output").
// The GEMM kernels want both operands contiguous along the reduction axis,
// so each call first writes W^T once (an HBM-bound transpose of all six
// weights, one launch).  64 x 64 tiles go through LDS so that reads and
// writes are both coalesced; the LDS tile is padded by one element so the
// column-wise reads fall in distinct banks.
#include "device.h"
#include "kernels.h"
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
  const dim3 grid(static_cast<unsigned>(max_tiles), static_cast<unsigned>(njobs));
  if (dtype == VITBLK_BF16)
    hipLaunchKernelGGL(pack_kernel<bf16_t>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(pack_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace vitblk
