// Streaming yardsticks for the benchmark (not part of the codec or decode
// path, and not declared in the library's public header): plain HIP kernels
// that move bytes with the traffic mix of each benchmarked kernel and do no
// other work, so that each kernel's bandwidth can be read against what the
// memory system delivers for the same mix, next to the 8 TB/s peak.
//
//   kind 0  read only      (every byte of `src` read once)
//   kind 1  write only     (every byte of `dst` written once)
//   kind 2  read 4 : write 1   (16 bytes read, 4 written per lane step: the
//                               encoder's mix, bf16 pages in, NVFP4 out)
//   kind 3  read 1 : write 4   (4 bytes read, 16 written: the decoder's mix)
//
// Each lane moves 16-byte vectors with several in flight; the launch shapes
// are the fastest of a sweep on MI355X (grid 1024 to 8192 workgroups of 256).
// Built into its own library, loaded only by bench.py.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

template <int U>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ src, size_t n,
                                                        uint32_t* __restrict__ sink) {
  size_t i = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads * U;
  uint32_t acc = 0;
  for (; i + (size_t)(U - 1) * kThreads < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // keeps the loads live; the condition is never met for the fill the
  // benchmark uses, so nothing is written
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

template <int U>
__global__ __launch_bounds__(kThreads) void write_kernel(u32x4* __restrict__ dst, size_t n) {
  size_t i = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads * U;
  for (; i + (size_t)(U - 1) * kThreads < n; i += stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * kThreads] = (u32x4){(uint32_t)i, 1u, 2u, (uint32_t)u};
  }
}

// n: 16-byte vectors read; one 4-byte word written per vector
template <int U>
__global__ __launch_bounds__(kThreads) void read4_write1_kernel(const u32x4* __restrict__ src,
                                                                uint32_t* __restrict__ dst,
                                                                size_t n) {
  size_t i = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads * U;
  for (; i + (size_t)(U - 1) * kThreads < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * kThreads] = v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
}

// n: 16-byte vectors written; one 4-byte word read per vector
template <int U>
__global__ __launch_bounds__(kThreads) void read1_write4_kernel(const uint32_t* __restrict__ src,
                                                                u32x4* __restrict__ dst,
                                                                size_t n) {
  size_t i = (size_t)blockIdx.x * kThreads * U + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kThreads * U;
  for (; i + (size_t)(U - 1) * kThreads < n; i += stride) {
    uint32_t v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kThreads);
#pragma unroll
    for (int u = 0; u < U; ++u) dst[i + u * kThreads] = (u32x4){v[u], v[u] + 1u, v[u] + 2u, v[u] + 3u};
  }
}

}  // namespace

// Moves `bytes` of the kind's reference stream on `stream` (the read side for
// kinds 0 and 2, the write side for kinds 1 and 3); `src` and `dst` are
// device buffers of at least `bytes` bytes (16-byte aligned), `sink` at
// least 1 KiB.  `bytes` must be a multiple of 16 x 256 x 8 x the grid.
// Returns the HIP error of the launch, or hipErrorInvalidValue for a bad
// kind, size or pointer.  The caller times it.
extern "C" int kvfp4_yardstick(int kind, const void* src, void* dst, void* sink, size_t bytes,
                               hipStream_t stream) {
  constexpr int kGridRead = 2048, kGridWrite = 8192, kGridMix = 8192;
  const size_t n = bytes / 16;
  const size_t quantum = (size_t)kThreads * 8 * kGridWrite;  // vectors per full sweep, largest
  if (bytes == 0 || bytes % 16 != 0 || n % quantum != 0) return (int)hipErrorInvalidValue;
  if (((uintptr_t)src & 15) != 0 || ((uintptr_t)dst & 15) != 0) return (int)hipErrorInvalidValue;
  switch (kind) {
    case 0:
      if (!src || !sink) return (int)hipErrorInvalidValue;
      hipLaunchKernelGGL((read_kernel<8>), dim3(kGridRead), dim3(kThreads), 0, stream,
                         static_cast<const u32x4*>(src), n, static_cast<uint32_t*>(sink));
      break;
    case 1:
      if (!dst) return (int)hipErrorInvalidValue;
      hipLaunchKernelGGL((write_kernel<4>), dim3(kGridWrite), dim3(kThreads), 0, stream,
                         static_cast<u32x4*>(dst), n);
      break;
    case 2:
      if (!src || !dst) return (int)hipErrorInvalidValue;
      hipLaunchKernelGGL((read4_write1_kernel<8>), dim3(kGridMix), dim3(kThreads), 0, stream,
                         static_cast<const u32x4*>(src), static_cast<uint32_t*>(dst), n);
      break;
    case 3:
      if (!src || !dst) return (int)hipErrorInvalidValue;
      hipLaunchKernelGGL((read1_write4_kernel<4>), dim3(kGridMix), dim3(kThreads), 0, stream,
                         static_cast<const uint32_t*>(src), static_cast<u32x4*>(dst), n);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
