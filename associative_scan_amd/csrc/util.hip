// Small utility kernels of libmscan.
#include "mscan_launch.hpp"

namespace mscan {

// Zero `words` 32-bit words; used instead of hipMemsetAsync so the call can sit
// inside a captured HIP graph.
__global__ __launch_bounds__(256) void k_zero(uint32_t* p, size_t words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < words; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t launch_zero(void* p, size_t bytes, hipStream_t st) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const size_t want = (words + 255) / 256;
  const unsigned blocks = (unsigned)(want < 1024 ? want : 1024);
  hipLaunchKernelGGL(k_zero, dim3(blocks), dim3(256), 0, st, (uint32_t*)p, words);
  return hipGetLastError();
}

}  // namespace mscan
