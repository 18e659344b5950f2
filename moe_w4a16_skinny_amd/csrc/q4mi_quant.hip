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

// max |w| over n4 float4 values into *amax (fp32 bits; non-negative floats
// order as unsigned integers); NaN values are skipped by fmaxf, so the
// result does not depend on the order of the maxima.  A grid-stride range
// with two batches of kAmaxU 16-byte non-temporal loads in flight per lane
// (the next batch is issued before the current one is reduced), one wave
// maximum and one atomicMax per wave.
__device__ __forceinline__ float amax4(float m, float4 v) {
  return fmaxf(fmaxf(m, fmaxf(fabsf(v.x), fabsf(v.y))), fmaxf(fabsf(v.z), fabsf(v.w)));
}
constexpr int kAmaxU = 8;
constexpr unsigned kAmaxGrid = 256;  // one workgroup a CU: measured 1073 us a step against 1117 at 512 and 1185 at 1024
typedef float nf32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ld_nt_f4(const float4* p) {
  const nf32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nf32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__global__ __launch_bounds__(256) void quant_amax_kernel(const float4* __restrict__ w, size_t n4, unsigned* amax) {
  const size_t stride = static_cast<size_t>(gridDim.x) * 256;
  size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  float m[4] = {0.f, 0.f, 0.f, 0.f};
  const size_t span = (kAmaxU - 1) * stride;  // a batch at i is whole while i + span < n4
  if (i + span < n4) {
    float4 v[kAmaxU];
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) v[u] = ld_nt_f4(w + i + u * stride);
    i += kAmaxU * stride;
    for (; i + span < n4; i += kAmaxU * stride) {
      float4 nv[kAmaxU];
#pragma unroll
      for (int u = 0; u < kAmaxU; ++u) nv[u] = ld_nt_f4(w + i + u * stride);
#pragma unroll
      for (int u = 0; u < kAmaxU; ++u) {
        m[u & 3] = amax4(m[u & 3], v[u]);
        v[u] = nv[u];
      }
    }
#pragma unroll
    for (int u = 0; u < kAmaxU; ++u) m[u & 3] = amax4(m[u & 3], v[u]);
  }
  for (; i < n4; i += stride) m[0] = amax4(m[0], w[i]);
  float mm = fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3]));
  for (int off = 32; off > 0; off >>= 1) mm = fmaxf(mm, __shfl_xor(mm, off));
  if ((threadIdx.x & 63) == 0) atomicMax(amax, __float_as_uint(mm));
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
// E2M1 codes of eight values into one dword (value j at nibble j) by the
// hardware conversion with unit scale: nearest of {0, .5, 1, 1.5, 2, 3, 4, 6},
// ties to the even code, saturating at 6, the sign bit of the value in bit 3.
__device__ __forceinline__ unsigned e2m1_x8(const float* q) {
  unsigned d = 0u;
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[0], q[1], 1.0f, 0);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[2], q[3], 1.0f, 1);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[4], q[5], 1.0f, 2);
  d = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(d, q[6], q[7], 1.0f, 3);
  return d;
}

// The codes of x[0..7] / S, the quotients correctly rounded.  For S in
// [2^-60, 2^60] each quotient takes one multiply by r = RN(1/S) and one
// correction: e = |x| - q0 S is exact (q0 is within an ulp and nothing
// underflows where the code depends on it), and RN(q0 + e r) = RN(|x| / S)
// because r is the correctly rounded reciprocal (Markstein's theorem).  The
// sign is copied from x afterwards, so -0 keeps its sign bit.  Quotients are
// capped at 8 first (beyond 6 every value saturates; an overflow of q0 to
// inf makes the correction NaN, which fminf drops).  Outside that range of S
// the quotients come from the IEEE division.
__device__ __forceinline__ unsigned e2m1_div8(const float* x, float S) {
  float q[8];
  if (S >= 0x1p-60f && S <= 0x1p60f) {
    const float r = 1.0f / S;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float a = fabsf(x[j]);
      const float q0 = a * r;
      const float e = fmaf(-q0, S, a);
      q[j] = copysignf(fminf(fmaf(e, r, q0), 8.0f), x[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = copysignf(fminf(fabsf(x[j] / S), 8.0f), x[j]);
  }
  return e2m1_x8(q);
}

// One tile (STEPS = 4 MFMA k-steps of 32, or 2 for a half tile) of panel
// rows n0..n0+15 by one wave: lane (o, c) quantizes row n0 + c at
// k = kb + 32 i + 8 o + 0..7 for each step i and writes the code dwords where
// the GEMM's lane reads them (one 16- or 8-byte store); the group amax is
// shared with lane o ^ 1 (lane ^ 16), and lanes with even o write the scale
// bytes of their groups (one store).
template <int STEPS>
__device__ __forceinline__ void quant_tile(const float* __restrict__ wrow, int K, int kb, int lane, float g,
                                           uint8_t* __restrict__ base) {
  const int o = lane >> 4, c = lane & 15;
  float4 v[STEPS][2];
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {  // every load first: K % 16 == 0, so a chunk of 8 is all inside or all padding
    const int k0 = kb + 32 * i + 8 * o;
    if (k0 < K) {
      v[i][0] = *reinterpret_cast<const float4*>(wrow + k0);
      v[i][1] = *reinterpret_cast<const float4*>(wrow + k0 + 4);
    } else {
      v[i][0] = make_float4(0.f, 0.f, 0.f, 0.f);
      v[i][1] = v[i][0];
    }
  }
  unsigned dw[STEPS], sc = 0u;
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    const float x[8] = {v[i][0].x, v[i][0].y, v[i][0].z, v[i][0].w, v[i][1].x, v[i][1].y, v[i][1].z, v[i][1].w};
    float la = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) la = fmaxf(la, fabsf(x[j]));
    const float gamax = fmaxf(la, __shfl_xor(la, 16));
    const unsigned s = g > 0.f ? e4m3_encode((gamax / 6.0f) / g) : 0u;
    const float S = e4m3_decode(s) * g;
    dw[i] = S > 0.f ? e2m1_div8(x, S) : 0u;  // low nibble: even k
    sc |= s << (8 * i);
  }
  uint8_t* sbase = base + STEPS * 256;  // the scales follow the 64 lanes' code dwords
  if constexpr (STEPS == 4) {
    *reinterpret_cast<uint4*>(base + lane * 16) = make_uint4(dw[0], dw[1], dw[2], dw[3]);
    if ((o & 1) == 0) *reinterpret_cast<unsigned*>(sbase + (c * 2 + (o >> 1)) * 4) = sc;
  } else {
    *reinterpret_cast<uint2*>(base + lane * 8) = make_uint2(dw[0], dw[1]);
    if ((o & 1) == 0) *reinterpret_cast<unsigned short*>(sbase + (c * 2 + (o >> 1)) * 2) = static_cast<unsigned short>(sc);
  }
}

// One workgroup of 4 waves per 16-row panel; wave q takes tiles q, q + 4, ...
// so that the four waves read 2 KiB of each row side by side.
__global__ __launch_bounds__(256) void quant_pack_kernel(const float* __restrict__ w, int K, int nfull, int ntiles,
                                                         int64_t pb, float g_in, const unsigned* amax,
                                                         uint8_t* __restrict__ packed, float* g_out, int64_t tail_off,
                                                         int tail_bytes) {
  const int p = blockIdx.x, q = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float g = g_in > 0.f ? g_in : __uint_as_float(*amax) / 2688.0f;
  if (p == 0) {
    if (threadIdx.x == 0 && g_out) *g_out = g;
    for (int i = threadIdx.x; i < tail_bytes; i += 256) packed[tail_off + i] = 0;  // zero guard behind the last panel
  }
  const float* wrow = w + (static_cast<int64_t>(p) * 16 + (lane & 15)) * K;
  uint8_t* pbase = packed + static_cast<int64_t>(p) * pb;
  for (int t = q; t < nfull; t += 4) quant_tile<4>(wrow, K, t * kTileK, lane, g, pbase + static_cast<int64_t>(t) * kTileBytes);
  if (nfull < ntiles && q == nfull % 4)
    quant_tile<2>(wrow, K, nfull * kTileK, lane, g, pbase + static_cast<int64_t>(nfull) * kTileBytes);
}

}  // namespace

int launch_quantize(const float* w, int64_t N, int64_t K, float g_in, unsigned* amax, uint8_t* packed, float* g_out,
                    void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!(g_in > 0.f)) {
    hipLaunchKernelGGL(quant_zero_kernel, dim3(1), dim3(1), 0, s, amax);
    const size_t n4 = static_cast<size_t>(N) * static_cast<size_t>(K) / 4;  // N * K % 256 == 0
    const unsigned blocks = static_cast<unsigned>(std::min<size_t>((n4 + 255) / 256, kAmaxGrid));
    hipLaunchKernelGGL(quant_amax_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const float4*>(w), n4, amax);
  }
  const int nfull = static_cast<int>(full_tiles(K));
  const int ntiles = nfull + (has_half_tile(K) ? 1 : 0);
  hipLaunchKernelGGL(quant_pack_kernel, dim3(static_cast<unsigned>(N / 16)), dim3(256), 0, s, w, static_cast<int>(K),
                     nfull, ntiles, panel_bytes(K), g_in, amax, packed, g_out, static_cast<int64_t>(N / 16) * panel_bytes(K),
                     static_cast<int>(packed_tail(K)));
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
