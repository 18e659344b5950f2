// The Gemma-4 MoE block around the expert kernels: the input RMSNorms and
// the combine.  (The router's normalization, softmax and top-k run in the
// last workgroup of the router kernel.)
//
// [DOC 3.2 "Per-layer (MoE)"], [DOC 4.6 "MoE"]: from the residual r,
//   h1 = RMSNorm(r; ffn_norm), h2 = RMSNorm(r; pre_ffw_norm_2)
//   z  = RMSNorm(h2 . W_r; unit weights) * ffn_gate_inp.scale, p = softmax(z),
//        top-k of p; [DOC 14 "Completed"]: ffn_down_exps.scale folded into
//        the kept weights
//   b1 = dense FFN(h1), b2 = sum_j w_j FFN_idx_j(h2)   (the expert kernels;
//        their per-slot outputs are summed by the combine here)
//   r += RMSNorm(RMSNorm(b1; post_ffw_norm_1) + RMSNorm(b2; post_ffw_norm_2);
//                post_ffw_norm)
// with RMSNorm(v; w) = v / sqrt(mean(v^2) + eps) * w.  The rows are few (one
// per token) and short, so each kernel takes one token per workgroup; every
// sum is reduced in a fixed order (deterministic).
#include <hip/hip_runtime.h>

#include <cmath>

#include "q4mi_internal.h"

namespace q4mi {
namespace {

typedef _Float16 f16;

// sum over the 256 threads: butterfly within each wave (lane 0's result),
// then the four waves in order
__device__ __forceinline__ float block_sum256(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();  // red may still be read from a previous sum
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return ((red[0] + red[1]) + red[2]) + red[3];
}
__device__ __forceinline__ float inv_rms(float sum_sq, int n, float eps) {
  return 1.0f / sqrtf(sum_sq / static_cast<float>(n) + eps);
}

// A row of D <= 256 * kRowRegs values lives in registers, thread t holding
// elements t + 256 j: every load of the row is issued before the first use.
constexpr int kRowRegs = 16;
__device__ __forceinline__ void load_row(float (&v)[kRowRegs], const float* __restrict__ row, int D) {
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    const int i = static_cast<int>(threadIdx.x) + 256 * j;
    v[j] = i < D ? row[i] : 0.f;
  }
}
__device__ __forceinline__ float sum_sq(const float (&v)[kRowRegs]) {
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) ss = fmaf(v[j], v[j], ss);
  return ss;
}

// h1 = RMSNorm(r; w1), h2 = RMSNorm(r; w2) as f16 (the expert GEMMs' input)
__global__ __launch_bounds__(256) void block_norm_in_kernel(const float* __restrict__ res, int D,
                                                            const float* __restrict__ w1,
                                                            const float* __restrict__ w2, float eps,
                                                            f16* __restrict__ h1, f16* __restrict__ h2) {
  __shared__ float red[4];
  float v[kRowRegs], a[kRowRegs], b[kRowRegs];
  load_row(v, res + static_cast<size_t>(blockIdx.x) * D, D);
  load_row(a, w1, D);
  load_row(b, w2, D);
  const float r = inv_rms(block_sum256(sum_sq(v), red), D, eps);
  f16* o1 = h1 + static_cast<size_t>(blockIdx.x) * D;
  f16* o2 = h2 + static_cast<size_t>(blockIdx.x) * D;
#pragma unroll
  for (int j = 0; j < kRowRegs; ++j) {
    const int i = static_cast<int>(threadIdx.x) + 256 * j;
    if (i < D) {
      const float x = v[j] * r;
      o1[i] = static_cast<f16>(x * a[j]);
      o2[i] = static_cast<f16>(x * b[j]);
    }
  }
}

// r += RMSNorm(RMSNorm(b1; p1) + RMSNorm(b2; p2); p), the branches read
// straight from the expert kernels' per-slot outputs: b1 = o1[t][0] (the
// dense layer, one slot of two per token), b2 = the sum over slots s < k of
// o2[t][s] whose pair has a row (rowof2[t][s] >= 0), added in slot order.
// 1024 threads per token, thread i holding elements i + 1024 j; each batch of
// 8 slots is loaded (with the row map) before any is added.
constexpr int kCombRegs = 4;  // D <= 4096
__device__ __forceinline__ float block_sum1024(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();  // red may still be read from a previous sum
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 16; ++w) s += red[w];
  return s;
}
__global__ __launch_bounds__(1024) void block_combine_kernel(const float* __restrict__ o1,
                                                             const float* __restrict__ o2,
                                                             const int32_t* __restrict__ rowof2, int k, int D,
                                                             const float* __restrict__ p1,
                                                             const float* __restrict__ p2,
                                                             const float* __restrict__ p, float eps,
                                                             float* __restrict__ res) {
  __shared__ float red[16];
  const int t = blockIdx.x, tid = threadIdx.x;
  float x1[kCombRegs], x2[kCombRegs], q1[kCombRegs], q2[kCombRegs], q[kCombRegs], xr[kCombRegs];
  const float* r1p = o1 + static_cast<size_t>(t) * 2 * D;
  const float* r2p = o2 + static_cast<size_t>(t) * (k + 1) * D;
#pragma unroll
  for (int j = 0; j < kCombRegs; ++j) {
    const int i = tid + 1024 * j;
    const bool in = i < D;
    x1[j] = in ? r1p[i] : 0.f;
    q1[j] = in ? p1[i] : 0.f;
    q2[j] = in ? p2[i] : 0.f;
    q[j] = in ? p[i] : 0.f;
    xr[j] = in ? res[static_cast<size_t>(t) * D + i] : 0.f;
    x2[j] = 0.f;
  }
  for (int s0 = 0; s0 < k; s0 += 8) {
    float v[8][kCombRegs];
    int pos[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sl = min(s0 + u, k - 1);
      pos[u] = s0 + u < k ? rowof2[t * k + sl] : -1;
#pragma unroll
      for (int j = 0; j < kCombRegs; ++j) {
        const int i = tid + 1024 * j;
        v[u][j] = i < D ? r2p[static_cast<size_t>(sl) * D + i] : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (pos[u] >= 0) {
#pragma unroll
        for (int j = 0; j < kCombRegs; ++j) x2[j] += v[u][j];
      }
  }
  float ss1 = 0.f, ss2 = 0.f;
#pragma unroll
  for (int j = 0; j < kCombRegs; ++j) {
    ss1 = fmaf(x1[j], x1[j], ss1);
    ss2 = fmaf(x2[j], x2[j], ss2);
  }
  const float r1 = inv_rms(block_sum1024(ss1, red), D, eps);
  const float r2 = inv_rms(block_sum1024(ss2, red), D, eps);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kCombRegs; ++j) {
    x1[j] = (x1[j] * r1) * q1[j] + (x2[j] * r2) * q2[j];  // the branches' sum
    ss = fmaf(x1[j], x1[j], ss);
  }
  const float r3 = inv_rms(block_sum1024(ss, red), D, eps);
  float* out = res + static_cast<size_t>(t) * D;
#pragma unroll
  for (int j = 0; j < kCombRegs; ++j) {
    const int i = tid + 1024 * j;
    if (i < D) out[i] = xr[j] + (x1[j] * r3) * q[j];
  }
}

}  // namespace

int launch_block_norm_in(const float* res, int T, int D, const float* w1, const float* w2, float eps, void* h1,
                         void* h2, void* stream) {
  hipLaunchKernelGGL(block_norm_in_kernel, dim3(T), dim3(256), 0, static_cast<hipStream_t>(stream), res, D, w1, w2,
                     eps, static_cast<f16*>(h1), static_cast<f16*>(h2));
  return static_cast<int>(hipGetLastError());
}

int launch_block_combine(const float* o1, const float* o2, const int32_t* rowof2, int k, int T, int D,
                         const float* p1, const float* p2, const float* p, float eps, float* res, void* stream) {
  hipLaunchKernelGGL(block_combine_kernel, dim3(T), dim3(1024), 0, static_cast<hipStream_t>(stream), o1, o2, rowof2,
                     k, D, p1, p2, p, eps, res);
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
