// MLX-style affine W{2,3,5,6,8}A16 skinny GEMM (M <= 16):
//   y[m][n] = sum_k a[m][k] * (q[n][k] * s[n][k / 64] + b[n][k / 64])
//
// [README "Everything it has"]: MLX affine weights at 2, 3, 4, 5, 6 and 8
// bits in groups of 64 (the 4-bit width has its own kernel).  Packed layout
// (q4_affine_bits_repack): per 16-row panel, 128-k tiles of 256 * BITS code
// bytes and 128 scale/bias bytes.  Lane (c, o) of a wave owns 4 * BITS
// code bytes holding, as one little-endian bit stream, the 32 codes of row
// c at k = 32 i + 8 o + j (i = 0..3, j = 0..7), code (i, j) at bit
// 8 BITS i + BITS j; the scale/bias words (bf16 scale low, bf16 bias high)
// of row c's two groups sit at 8 c.  K is padded to 128 with zero codes and
// zero scale/bias.
//
// A code q < 128 becomes the exact bf16 128 + q by OR-ing it under the
// exponent of 128, so sum_k a (128 + q) runs on the bf16 MFMA and the group
// sum sum_k a on the same MFMA against ones; per group
//   sum_k a w = s * sum a (128 + q) + (b - 128 s) * sum a.
// 8-bit codes are split in nibbles, q = 16 qh + ql, each on its own MFMA:
//   sum_k a w = s * (16 sum a (128 + qh) + sum a (128 + ql)) + (b - 2176 s) * sum a.
// A workgroup of 4 waves computes 2 panels; its waves split the tiles and
// their partial sums are added in LDS in wave order (deterministic).
#include <hip/hip_runtime.h>

#include "q4mi_tiles.h"

namespace q4mi {
using namespace dev;
namespace {

constexpr int kAbP = 2;  // panels per workgroup

template <int BITS>
struct AffB {
  static constexpr int kLaneBytes = 4 * BITS;
  static constexpr int kCodeBytes = 64 * kLaneBytes;
  static constexpr int kTileBytes = kCodeBytes + 128;
};

template <int BITS>
__device__ __forceinline__ void load_codes(unsigned (&d)[BITS], const uint8_t* p) {
  if constexpr (BITS % 4 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 4; ++j) {
      const u32x4 v = ld_nt16(p + 16 * j);
      d[4 * j] = v.x, d[4 * j + 1] = v.y, d[4 * j + 2] = v.z, d[4 * j + 3] = v.w;
    }
  } else if constexpr (BITS % 2 == 0) {
#pragma unroll
    for (int j = 0; j < BITS / 2; ++j) {
      const u32x2 v = ld_nt8(p + 8 * j);
      d[2 * j] = v.x, d[2 * j + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int j = 0; j < BITS; ++j) d[j] = ld_nt4(p + 4 * j);
  }
}

// code j of step i from the lane's bit stream
template <int BITS>
__device__ __forceinline__ unsigned code_at(const unsigned (&d)[BITS], int i, int j) {
  const int p = 8 * BITS * i + BITS * j;
  const int w = p >> 5, sh = p & 31;
  unsigned v = d[w] >> sh;
  if (sh + BITS > 32) v |= d[w + 1] << (32 - sh);
  return v & ((1u << BITS) - 1u);
}

// 8 values (128 + x_j) as bf16, x_j < 128, element j = k offset j
__device__ __forceinline__ bf16x8 bf16_128_plus(const unsigned (&x)[8]) {
  u32x4 r;
  r.x = (x[0] | 0x4300u) | ((x[1] | 0x4300u) << 16);
  r.y = (x[2] | 0x4300u) | ((x[3] | 0x4300u) << 16);
  r.z = (x[4] | 0x4300u) | ((x[5] | 0x4300u) << 16);
  r.w = (x[6] | 0x4300u) | ((x[7] | 0x4300u) << 16);
  return __builtin_bit_cast(bf16x8, r);
}

template <int BITS>
__global__ __launch_bounds__(256) void qgemm_affineb_kernel(const uint8_t* __restrict__ w, int64_t pb, int ntiles,
                                                            const uint16_t* __restrict__ a, int M, int K, int N,
                                                            void* __restrict__ out, int out_dtype) {
  using L = AffB<BITS>;
  __shared__ f32x4 part[4][kAbP][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, o = lane >> 4;
  const int p0 = blockIdx.x * kAbP;
  const int npanels = N / 16;
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc[kAbP];
#pragma unroll
  for (int p = 0; p < kAbP; ++p) acc[p] = z;
  const uint16_t* arow = a + static_cast<int64_t>(c < M ? c : 0) * K;
  // the waves take tiles w, w + 4, ...
  for (int t = wave; t < ntiles; t += 4) {
    const int kb = t * kTileK;
    u32x4 af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k0 = kb + 32 * i + 8 * o;
      af[i] = (c < M && k0 < K) ? *reinterpret_cast<const u32x4*>(arow + k0) : u32x4{0u, 0u, 0u, 0u};
    }
    unsigned d[kAbP][BITS];
    u32x2 sb[kAbP];
#pragma unroll
    for (int p = 0; p < kAbP; ++p) {
      const int pn = min(p0 + p, npanels - 1);  // a panel past N re-reads the last one (never stored)
      const uint8_t* tb = w + static_cast<int64_t>(pn) * pb + static_cast<int64_t>(t) * L::kTileBytes;
      load_codes<BITS>(d[p], tb + lane * L::kLaneBytes);
      sb[p] = ld_nt8(tb + L::kCodeBytes + c * 8);
    }
    f32x4 as0 = mfma_bf16(af[0], ones, z);
    as0 = mfma_bf16(af[1], ones, as0);
    f32x4 as1 = mfma_bf16(af[2], ones, z);
    as1 = mfma_bf16(af[3], ones, as1);
#pragma unroll
    for (int p = 0; p < kAbP; ++p) {
      f32x4 q0, q1;
      if constexpr (BITS == 8) {
        f32x4 h[2] = {z, z}, l[2] = {z, z};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned xh[8], xl[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const unsigned v = code_at<BITS>(d[p], i, j);
            xh[j] = v >> 4;
            xl[j] = v & 15u;
          }
          h[i >> 1] = mfma_bf16(af[i], bf16_128_plus(xh), h[i >> 1]);
          l[i >> 1] = mfma_bf16(af[i], bf16_128_plus(xl), l[i >> 1]);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          q0[r] = fmaf(16.0f, h[0][r], l[0][r]);
          q1[r] = fmaf(16.0f, h[1][r], l[1][r]);
        }
      } else {
        f32x4 q[2] = {z, z};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          unsigned x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) x[j] = code_at<BITS>(d[p], i, j);
          q[i >> 1] = mfma_bf16(af[i], bf16_128_plus(x), q[i >> 1]);
        }
        q0 = q[0];
        q1 = q[1];
      }
      const float off = BITS == 8 ? -2176.0f : -128.0f;  // the 128 (and 16 * 128) under each code
      const float s0 = bf16_lo(sb[p].x), b0 = bf16_hi(sb[p].x);
      const float s1 = bf16_lo(sb[p].y), b1 = bf16_hi(sb[p].y);
      const float c0 = fmaf(off, s0, b0), c1 = fmaf(off, s1, b1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[p][r];
        v = fmaf(s0, q0[r], v);
        v = fmaf(c0, as0[r], v);
        v = fmaf(s1, q1[r], v);
        v = fmaf(c1, as1[r], v);
        acc[p][r] = v;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < kAbP; ++p) part[wave][p][lane] = acc[p];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int p = 0; p < kAbP; ++p) {
    const f32x4 v = ((part[0][p][lane] + part[1][p][lane]) + part[2][p][lane]) + part[3][p][lane];
    const int pn = p0 + p;
    if (pn >= npanels) continue;
    const int n = pn * 16 + c;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * o + r;
      if (m < M) store_out(out, out_dtype, static_cast<size_t>(m) * N + n, v[r]);
    }
  }
}

template <int BITS>
int launch_bits(const uint8_t* w, int64_t N, int64_t K, const uint16_t* a, int M, void* out, int out_dtype,
                void* stream) {
  const int ntiles = static_cast<int>((K + kTileK - 1) / kTileK);
  const int64_t pb = static_cast<int64_t>(ntiles) * AffB<BITS>::kTileBytes;
  const int64_t blocks = (N / 16 + kAbP - 1) / kAbP;
  hipLaunchKernelGGL(qgemm_affineb_kernel<BITS>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), w, pb, ntiles, a, M, static_cast<int>(K), static_cast<int>(N),
                     out, out_dtype);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

int launch_affine_bits(int bits, const uint8_t* w, int64_t N, int64_t K, const uint16_t* a, int M, void* out,
                       int out_dtype, void* stream) {
  switch (bits) {
    case 2: return launch_bits<2>(w, N, K, a, M, out, out_dtype, stream);
    case 3: return launch_bits<3>(w, N, K, a, M, out, out_dtype, stream);
    case 5: return launch_bits<5>(w, N, K, a, M, out, out_dtype, stream);
    case 6: return launch_bits<6>(w, N, K, a, M, out, out_dtype, stream);
    case 8: return launch_bits<8>(w, N, K, a, M, out, out_dtype, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace q4mi
