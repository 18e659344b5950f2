// Stream-read ceiling: the rate at which this GPU can read a buffer from HBM
// with the same loads the weight-streaming kernels issue (16-byte
// non-temporal loads, 1 KiB contiguous per wave instruction).  It does no
// arithmetic beyond an XOR that keeps the loads alive, so its time is the
// floor for reading the same number of bytes.  [gemma-cuda-hybrid README,
// "Why it's NVIDIA-only": the kernels are tuned against the bandwidth the
// memory actually delivers, not the datasheet's.]
#include <hip/hip_runtime.h>

#include "q4mi_tiles.h"

namespace q4mi {
namespace {
using namespace dev;

constexpr int kCeilThreads = 256;

// XOR over the wave (one LDS atomic per wave afterwards, not one per lane:
// atomics on one LDS word serialize)
__device__ __forceinline__ unsigned wave_xor(unsigned x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  return x;
}

// Lane work: words i0, i0 + stride, ... below end, in batches of U loads,
// the next batch issued before the previous one is consumed (two batches in
// flight per lane).
// MODE 0: grid-stride; consecutive waves read consecutive KiB.
// MODE 1: workgroup b reads one contiguous chunk (as a GEMM workgroup reads
//         its own panels).
template <int MODE, int U>
__global__ __launch_bounds__(kCeilThreads) void stream_read_kernel(const uint8_t* __restrict__ src, size_t n16,
                                                                   unsigned* __restrict__ out) {
  __shared__ unsigned sx;
  const size_t tid = threadIdx.x;
  size_t i, end, stride;
  if constexpr (MODE == 0) {
    i = static_cast<size_t>(blockIdx.x) * kCeilThreads + tid;
    stride = static_cast<size_t>(gridDim.x) * kCeilThreads;
    end = n16;
  } else {
    const size_t chunk = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t b0 = static_cast<size_t>(blockIdx.x) * chunk;
    i = b0 + tid;
    stride = kCeilThreads;
    end = b0 + chunk < n16 ? b0 + chunk : n16;
  }
  if (tid == 0) sx = 0u;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t span = (U - 1) * stride;  // a batch at i is whole while i + span < end
  if (i + span < end) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = ld_nt16(src + (i + u * stride) * 16);
    i += U * stride;
    for (; i + span < end; i += U * stride) {
      u32x4 nv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) nv[u] = ld_nt16(src + (i + u * stride) * 16);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        acc ^= v[u];
        v[u] = nv[u];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  for (; i < end; i += stride) acc ^= ld_nt16(src + i * 16);
  __syncthreads();
  const unsigned x = wave_xor(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if ((tid & 63) == 0) atomicXor(&sx, x);
  __syncthreads();
  if (tid == 0) out[blockIdx.x] = sx;
}

// MODE 2 (one batch): 512-thread workgroups; workgroup b reads the b-th of
// `grid` contiguous chunks (whole KiB per wave instruction), every lane
// issuing all its loads (at most kOnceMax) before the first is used, as a
// GEMM wave issues its tiles.
constexpr int kOnceMax = 32;
__global__ __launch_bounds__(512) void stream_read_once_kernel(const uint8_t* __restrict__ src, size_t n16,
                                                              size_t per, unsigned* __restrict__ out) {
  __shared__ unsigned sx;
  const size_t b0 = static_cast<size_t>(blockIdx.x) * per;
  const size_t end = b0 + per < n16 ? b0 + per : n16;
  if (threadIdx.x == 0) sx = 0u;
  u32x4 v[kOnceMax];
#pragma unroll
  for (int u = 0; u < kOnceMax; ++u) {
    const size_t i = b0 + static_cast<size_t>(u) * 512 + threadIdx.x;
    v[u] = i < end ? ld_nt16(src + i * 16) : u32x4{0u, 0u, 0u, 0u};
  }
  u32x4 acc = v[0];
#pragma unroll
  for (int u = 1; u < kOnceMax; ++u) acc ^= v[u];
  __syncthreads();
  const unsigned x = wave_xor(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if ((threadIdx.x & 63) == 0) atomicXor(&sx, x);
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = sx;
}

template <int MODE, int U>
int launch_u(const uint8_t* p, size_t bytes, int grid, unsigned* out, hipStream_t s) {
  hipLaunchKernelGGL((stream_read_kernel<MODE, U>), dim3(grid), dim3(kCeilThreads), 0, s, p, bytes / 16, out);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

// depth: loads per batch (1, 2, 4 or 8; the host checks); mode 2 ignores it
int launch_stream_read(const void* src, size_t bytes, int grid, int mode, int depth, unsigned* out, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const uint8_t* p = static_cast<const uint8_t*>(src);
  if (mode == 2) {
    const size_t n16 = bytes / 16;
    const size_t per = (n16 + grid - 1) / grid;
    hipLaunchKernelGGL(stream_read_once_kernel, dim3(grid), dim3(512), 0, s, p, n16, per, out);
    return static_cast<int>(hipGetLastError());
  }
  if (mode == 0) {
    switch (depth) {
      case 1: return launch_u<0, 1>(p, bytes, grid, out, s);
      case 2: return launch_u<0, 2>(p, bytes, grid, out, s);
      case 4: return launch_u<0, 4>(p, bytes, grid, out, s);
      default: return launch_u<0, 8>(p, bytes, grid, out, s);
    }
  }
  switch (depth) {
    case 1: return launch_u<1, 1>(p, bytes, grid, out, s);
    case 2: return launch_u<1, 2>(p, bytes, grid, out, s);
    case 4: return launch_u<1, 4>(p, bytes, grid, out, s);
    default: return launch_u<1, 8>(p, bytes, grid, out, s);
  }
}

}  // namespace q4mi
