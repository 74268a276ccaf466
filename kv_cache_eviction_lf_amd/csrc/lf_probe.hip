// HBM probes: a streaming copy and a streaming read with 16-byte lanes, one
// contiguous 4 KiB run per workgroup load step, grid-stride over the buffer.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/lf_probe.h"

namespace {

constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 256 * 8;  // 8 workgroups per CU on 256 CUs
constexpr int kUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) dst[i + k * stride] = v[k];
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ src, size_t n,
                                                                    uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kProbeThreads;
  size_t i = (size_t)blockIdx.x * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) v[k] = src[i + k * stride];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
  for (; i < n; i += stride) x ^= src[i].x ^ src[i].y ^ src[i].z ^ src[i].w;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t s[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

bool bad(const void* p) { return !p || reinterpret_cast<uintptr_t>(p) % 16; }

}  // namespace

extern "C" {

int32_t lf_probe_read_sink_words(void) { return kProbeBlocks; }

lf_status lf_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bad(src) || bad(dst) || bytes % 16) return LF_ERR_ARG;
  if (!bytes) return LF_OK;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), static_cast<uint4*>(dst),
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? LF_OK : LF_ERR_HIP;
}

lf_status lf_probe_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bad(src) || !sink || bytes % 16) return LF_ERR_ARG;
  if (!bytes) return LF_OK;
  hipLaunchKernelGGL(probe_read_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? LF_OK : LF_ERR_HIP;
}

}  // extern "C"
