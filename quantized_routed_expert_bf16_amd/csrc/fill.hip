// Zero fill of a workspace (moe_workspace_init), for gfx950.  A plain kernel
// rather than hipMemsetAsync, so that it can sit inside a captured graph.
#include "moe_internal.h"

namespace moe {
namespace {

__global__ void fill_zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = blockIdx.x * size_t(blockDim.x) + threadIdx.x; i < n16;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

}  // namespace

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t s) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                     static_cast<uint4 *>(p), n16);
  return hipGetLastError();
}

}  // namespace moe
