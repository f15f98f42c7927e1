// Read-only HBM stream for the benchmark: the attainable read bandwidth of
// the device, reported next to the nominal peak beside the HBM-bound
// kernels' rooflines.  Not part of the HSA library: it is built into its own
// small library (libhsa_attn_stream.so) and only the benchmark loads it.
//
// Every 16-byte word of the buffer is loaded once (nontemporal loads, U
// independent loads in flight per thread, grid-stride over the buffer); the
// XOR of all the words a thread loaded is stored only when it equals a fixed
// constant, so the compiler cannot drop a load and the kernel writes
// (practically) nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ p, uint64_t n,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const uint64_t step = (uint64_t)gridDim.x * 256 * U;
  for (uint64_t i = (uint64_t)blockIdx.x * 256 * U + threadIdx.x; i < n; i += step) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint64_t j = i + (uint64_t)u * 256;
      v[u] = j < n ? __builtin_nontemporal_load(p + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// buf: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned);
// sink: device buffer of blocks * 256 uint32 (almost never written);
// unroll: 4 or 8; blocks > 0.  Launches on `stream` and returns the HIP
// status of the launch (hipErrorInvalidValue for bad arguments).
extern "C" int hsa_attn_stream_read(const void* buf, uint64_t bytes, int blocks, int unroll, uint32_t* sink,
                                    hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || blocks <= 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0 || (unroll != 4 && unroll != 8))
    return (int)hipErrorInvalidValue;
  const u32x4* p = static_cast<const u32x4*>(buf);
  const uint64_t n = bytes / 16;
  if (unroll == 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, sink);
  else
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3((unsigned)blocks), dim3(256), 0, stream, p, n, sink);
  return (int)hipGetLastError();
}
