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

// Streaming diagnostic: NS arrays read and ND arrays written, n4 16-byte units
// each, with the scan kernels' access type (non-temporal dwordx4 loads and
// stores); every lane keeps four units of each source in flight before it
// stores. It moves the bytes of a scan kernel with the same read:write mix and
// nothing else, so its rate is the practical ceiling for that kernel.
typedef float sv4 __attribute__((ext_vector_type(4)));
struct StreamArgs {
  const sv4* src[4];
  sv4* dst[4];
  size_t n4;
};

template <int NS, int ND>
__global__ __launch_bounds__(256) void k_stream(const StreamArgs a) {
  constexpr int U = 4;  // units per lane per round
  const size_t step = (size_t)gridDim.x * 256 * U;
  for (size_t base = (size_t)blockIdx.x * 256 * U + threadIdx.x; base < a.n4; base += step) {
    sv4 acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) acc[u] = sv4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * 256;
        if (i < a.n4) acc[u] += __builtin_nontemporal_load(a.src[s] + i);
      }
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const size_t i = base + (size_t)u * 256;
        if (i < a.n4) __builtin_nontemporal_store(acc[u], a.dst[d] + i);
      }
  }
}

template <int NS, int ND>
static hipError_t launch_stream_nd(const StreamArgs& a, hipStream_t st) {
  // one workgroup per 1024 units (16 KiB of every array), as the scan
  // kernels take one tile per workgroup; a grid beyond 2^20 workgroups loops
  const size_t want = (a.n4 + 1023) / 1024;
  const unsigned blocks = (unsigned)(want < (1u << 20) ? (want ? want : 1) : (1u << 20));
  hipLaunchKernelGGL((k_stream<NS, ND>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_stream(const float* const* src, int nsrc, float* const* dst, int ndst, size_t n4, hipStream_t st) {
  StreamArgs a{};
  for (int i = 0; i < nsrc; ++i) a.src[i] = (const sv4*)src[i];
  for (int i = 0; i < ndst; ++i) a.dst[i] = (sv4*)dst[i];
  a.n4 = n4;
#define MSCAN_STREAM_CASE(S, D) \
  if (nsrc == S && ndst == D) return launch_stream_nd<S, D>(a, st);
  MSCAN_STREAM_CASE(1, 1) MSCAN_STREAM_CASE(2, 1) MSCAN_STREAM_CASE(3, 1) MSCAN_STREAM_CASE(1, 2)
  MSCAN_STREAM_CASE(2, 2) MSCAN_STREAM_CASE(3, 2) MSCAN_STREAM_CASE(4, 2) MSCAN_STREAM_CASE(4, 3)
#undef MSCAN_STREAM_CASE
  return hipErrorInvalidValue;
}

// Copy the workspace header's error word to *dst (device-accessible memory).
// The word is written with agent-scope atomics by the scan kernels, so it is
// read the same way.
__global__ __launch_bounds__(64) void k_read_error(const uint32_t* hdr, int32_t* dst) {
  if (threadIdx.x == 0) {
    const uint32_t e = __hip_atomic_load(hdr + kHdrErrorWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *dst = e ? 5 : 0;  // MSCAN_ERR_TIMEOUT or MSCAN_OK
  }
}

hipError_t launch_read_error(const void* ws, int32_t* dst, hipStream_t st) {
  hipLaunchKernelGGL(k_read_error, dim3(1), dim3(64), 0, st, (const uint32_t*)ws, dst);
  return hipGetLastError();
}

}  // namespace mscan
