// HBM probes: a streaming copy and a streaming read with 16-byte lanes, each
// workgroup sweeping one contiguous slice of the buffer.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/lf_probe.h"

namespace {

// Each workgroup streams one contiguous slice of the buffer with 8 16-byte
// loads per lane in flight; 1024 workgroups of 256 threads.
constexpr int kProbeThreads = 256;
constexpr int kProbeBlocks = 1024;
constexpr int kUnroll = 8;

__device__ __forceinline__ void slice(size_t n, size_t& lo, size_t& hi) {
  const size_t per = (n + gridDim.x - 1) / gridDim.x;
  lo = per * blockIdx.x;
  hi = lo + per < n ? lo + per : n;
}

__global__ __launch_bounds__(kProbeThreads) void probe_copy_kernel(const uint4* __restrict__ src,
                                                                    uint4* __restrict__ dst, size_t n) {
  size_t lo, hi;
  slice(n, lo, hi);
  for (size_t i = lo + threadIdx.x; i < hi; i += (size_t)kProbeThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const size_t j = i + (size_t)k * kProbeThreads;
      v[k] = j < hi ? src[j] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const size_t j = i + (size_t)k * kProbeThreads;
      if (j < hi) dst[j] = v[k];
    }
  }
}

__global__ __launch_bounds__(kProbeThreads) void probe_read_kernel(const uint4* __restrict__ src, size_t n,
                                                                    uint32_t* __restrict__ sink) {
  size_t lo, hi;
  slice(n, lo, hi);
  uint32_t x = 0;
  for (size_t i = lo + threadIdx.x; i < hi; i += (size_t)kProbeThreads * kUnroll) {
    uint4 v[kUnroll];
#pragma unroll
    for (int k = 0; k < kUnroll; ++k) {
      const size_t j = i + (size_t)k * kProbeThreads;
      v[k] = src[j < hi ? j : hi - 1];
    }
#pragma unroll
    for (int k = 0; k < kUnroll; ++k)
      if (i + (size_t)k * kProbeThreads < hi) x ^= v[k].x ^ v[k].y ^ v[k].z ^ v[k].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t s[kProbeThreads / 64];
  if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

// A workgroup that does nothing: a graph of these measures the per-launch
// floor (dispatch, workgroup start and retirement, the gap between nodes).
__global__ __launch_bounds__(kProbeThreads) void probe_empty_kernel() {}

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

lf_status lf_probe_empty(int32_t n_blocks, void* stream) {
  if (n_blocks < 1) return LF_ERR_ARG;
  hipLaunchKernelGGL(probe_empty_kernel, dim3(n_blocks), dim3(kProbeThreads), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? LF_OK : LF_ERR_HIP;
}

}  // extern "C"
