// Streaming probes: the rate at which this device reads (and copies) a large
// buffer in HBM. They measure the bandwidth ceiling the decode kernels work
// against; they are not part of the attention path.
//
// Every thread keeps `depth` (4, 8 or 16) 16-byte non-temporal loads in
// flight, grid-strided so that one pass of the grid covers a contiguous span of
// the buffer (consecutive lanes read consecutive 16-byte words). On MI355X the
// read rate peaks with about 16-32 KiB in flight per compute unit (one or two
// 256-thread workgroups per CU at depth 4-8) and falls with more: the sweep
// over grid and depth is left to the caller. The read probe folds
// what it read into one XOR word per wave and XORs that into *sink with one
// device-scope atomic, so the loads cannot be dropped and the result can be
// checked (the XOR of every 32-bit word of the buffer).
#include "da_device.h"
#include "da_internal.h"

namespace da {
namespace {

constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int kUnroll>
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                               int64_t n16, uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

template <int kUnroll>
__global__ __launch_bounds__(kThreads) void stream_copy_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst,
                                                               int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, int32_t blocks, int32_t depth,
                              uint32_t* sink, hipStream_t st) {
  const auto* p = static_cast<const u32x4*>(src);
  const int64_t n16 = bytes / 16;
  if (depth == 4)
    hipLaunchKernelGGL(stream_read_kernel<4>, dim3(blocks), dim3(kThreads), 0, st, p, n16, sink);
  else if (depth == 8)
    hipLaunchKernelGGL(stream_read_kernel<8>, dim3(blocks), dim3(kThreads), 0, st, p, n16, sink);
  else if (depth == 16)
    hipLaunchKernelGGL(stream_read_kernel<16>, dim3(blocks), dim3(kThreads), 0, st, p, n16, sink);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, int64_t bytes, int32_t blocks,
                              int32_t depth, hipStream_t st) {
  const auto* p = static_cast<const u32x4*>(src);
  auto* q = static_cast<u32x4*>(dst);
  const int64_t n16 = bytes / 16;
  if (depth == 4)
    hipLaunchKernelGGL(stream_copy_kernel<4>, dim3(blocks), dim3(kThreads), 0, st, p, q, n16);
  else if (depth == 8)
    hipLaunchKernelGGL(stream_copy_kernel<8>, dim3(blocks), dim3(kThreads), 0, st, p, q, n16);
  else if (depth == 16)
    hipLaunchKernelGGL(stream_copy_kernel<16>, dim3(blocks), dim3(kThreads), 0, st, p, q, n16);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace da
