// NVFP4 quantizer on the device: fp32 weights -> codes and scales, written
// straight into the packed layout the GEMMs stream.
//
// [gemma-cuda-hybrid README]: an NVFP4 quantization kernel sits beside the
// FP4 GEMM in its kernel list; "Why it's NVIDIA-only": E2M1 codes, an E4M3
// scale per 16 values, an fp32 global scale.  Recipe: g = amax / (448 * 6);
// group scale s = E4M3(group amax / 6 / g), round to nearest even, saturating
// at 448; codes = E2M1(w / (e4m3(s) * g)), nearest even, saturating at 6; a
// group whose decoded scale is 0 gets +0 codes.  Every step is one fp32
// operation in that order (the codes are integers that floating point
// decides, here in fp32).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "q4mi_internal.h"

namespace q4mi {
namespace {

__global__ void quant_zero_kernel(unsigned* word) { *word = 0u; }

// max |w| over n values into *amax (fp32 bits; non-negative floats order as
// unsigned integers); NaN values are skipped by fmaxf
__global__ __launch_bounds__(256) void quant_amax_kernel(const float* __restrict__ w, size_t n, unsigned* amax) {
  float m = 0.f;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += static_cast<size_t>(gridDim.x) * 256)
    m = fmaxf(m, fabsf(w[i]));
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) atomicMax(amax, __float_as_uint(m));
}

// E4M3FN byte of t >= 0: nearest value, ties to the even code, >= 448 -> 0x7E
__device__ __forceinline__ unsigned e4m3_encode(float t) {
  if (!(t > 0.f)) return 0u;
  if (t >= 448.f) return 0x7Eu;
  int e = static_cast<int>(__float_as_uint(t) >> 23) - 127;  // t in [2^e, 2^(e+1)) for normal fp32
  e = e < -6 ? -6 : e;                                       // E4M3 subnormals share the 2^-6 binade's quantum
  const int m = static_cast<int>(rintf(ldexpf(t, 3 - e)));  // t / 2^(e-3), exact scaling, then nearest even
  const int code = ((e + 7) << 3) + (m - 8);                 // m == 16 carries into the exponent field
  return static_cast<unsigned>(code < 0x7E ? code : 0x7E);
}
__device__ __forceinline__ float e4m3_decode(unsigned b) {
  const unsigned ex = (b >> 3) & 15u, mt = b & 7u;
  return ex == 0 ? static_cast<float>(mt) * 0x1p-9f : ldexpf(1.0f + static_cast<float>(mt) * 0.125f, int(ex) - 7);
}
// E2M1 code of x: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even
// index (midpoints .25 and 1.25, 2.5, 5 go down; .75, 1.75, 3.5 go up),
// saturating at 6; bit 3 is the sign bit of x
__device__ __forceinline__ unsigned e2m1_encode(float x) {
  const float a = fabsf(x);
  const unsigned mag = (a > 0.25f ? 1u : 0u) + (a >= 0.75f ? 1u : 0u) + (a > 1.25f ? 1u : 0u) + (a >= 1.75f ? 1u : 0u) +
                       (a > 2.5f ? 1u : 0u) + (a >= 3.5f ? 1u : 0u) + (a > 5.0f ? 1u : 0u);
  return mag | ((__float_as_uint(x) >> 28) & 8u);
}

// One wave per (tile t, panel p): lane (o, c) quantizes row n = 16 p + c,
// k = 128 t + 32 i + 8 o + 0..7 for each MFMA step i, and writes the code
// dword where the GEMM's lane reads it; the group amax is shared with lane
// o ^ 1 (lane ^ 16), and lanes with even o write the group's scale byte.
__global__ __launch_bounds__(64) void quant_pack_kernel(const float* __restrict__ w, int K, int nfull, int64_t pb,
                                                        float g_in, const unsigned* amax, uint8_t* __restrict__ packed,
                                                        float* g_out, int64_t tail_off, int tail_bytes) {
  const int t = blockIdx.y, p = blockIdx.x;
  const int lane = threadIdx.x, o = lane >> 4, c = lane & 15;
  const float g = g_in > 0.f ? g_in : __uint_as_float(*amax) / 2688.0f;
  if (t == 0 && p == 0) {
    if (lane == 0 && g_out) *g_out = g;
    for (int i = lane; i < tail_bytes; i += 64) packed[tail_off + i] = 0;  // zero guard behind the last panel
  }
  const bool is_half = t == nfull;
  const int steps = is_half ? 2 : 4;
  const int64_t n = static_cast<int64_t>(p) * 16 + c;
  uint8_t* base = packed + static_cast<int64_t>(p) * pb + static_cast<int64_t>(t) * kTileBytes;
  uint8_t* sbase = base + (is_half ? kHalfCodeBytes : kTileCodeBytes);
  for (int i = 0; i < steps; ++i) {
    const int k0 = t * kTileK + 32 * i + 8 * o;
    float v[8];
    if (k0 < K) {  // K % 16 == 0: all 8 inside
      const float4 a = *reinterpret_cast<const float4*>(w + n * K + k0);
      const float4 b = *reinterpret_cast<const float4*>(w + n * K + k0 + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = 0.f;
    }
    float la = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) la = fmaxf(la, fabsf(v[j]));
    const float gamax = fmaxf(la, __shfl_xor(la, 16));
    const unsigned s = g > 0.f ? e4m3_encode((gamax / 6.0f) / g) : 0u;
    const float S = e4m3_decode(s) * g;
    unsigned dword = 0u;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const unsigned q = S > 0.f ? e2m1_encode(v[j] / S) : 0u;
      dword |= q << (4 * j);  // byte b = codes of k0 + 2b (low nibble) and k0 + 2b + 1
    }
    *reinterpret_cast<unsigned*>(base + lane * (steps * 4) + i * 4) = dword;
    if ((o & 1) == 0) sbase[(c * 2 + (o >> 1)) * steps + i] = static_cast<uint8_t>(s);
  }
}

}  // namespace

int launch_quantize(const float* w, int64_t N, int64_t K, float g_in, unsigned* amax, uint8_t* packed, float* g_out,
                    void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(g_in > 0.f)) {
    hipLaunchKernelGGL(quant_zero_kernel, dim3(1), dim3(1), 0, s, amax);
    const size_t n = static_cast<size_t>(N) * static_cast<size_t>(K);
    const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n + 255) / 256, 4096));
    hipLaunchKernelGGL(quant_amax_kernel, dim3(blocks), dim3(256), 0, s, w, n, amax);
  }
  const int nfull = static_cast<int>(full_tiles(K));
  const int ntiles = nfull + (has_half_tile(K) ? 1 : 0);
  hipLaunchKernelGGL(quant_pack_kernel, dim3(static_cast<unsigned>(N / 16), static_cast<unsigned>(ntiles)), dim3(64), 0,
                     s, w, static_cast<int>(K), nfull, panel_bytes(K), g_in, amax, packed, g_out,
                     static_cast<int64_t>(N / 16) * panel_bytes(K), static_cast<int>(packed_tail(K)));
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
