// Device building blocks shared by the GEMM and MoE kernels of libq4mi
// (included only by .hip sources).  See q4mi_internal.h for the packed
// tile geometry.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

#include "q4mi.h"
#include "q4mi_internal.h"

namespace q4mi {
namespace dev {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x4 ld_nt16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld_nt8(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ unsigned ld_nt4(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned*>(p));
}
__device__ __forceinline__ unsigned ld_nt2(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const unsigned short*>(p));
}

// 8 NVFP4 codes (one MFMA step of one lane) -> 8 f16 = e2m1 * e4m3 (exact)
__device__ __forceinline__ f16x8 nvfp4_operand(unsigned cw, f16 s) {
  const f16x2 ss = {s, s};
  const f16x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 0) * ss;
  const f16x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 1) * ss;
  const f16x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 2) * ss;
  const f16x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(cw, 1.0f, 3) * ss;
  return f16x8{v0[0], v0[1], v1[0], v1[1], v2[0], v2[1], v3[0], v3[1]};
}

// E4M3 scale bytes 0,1 (word_sel false) or 2,3 (true) -> two f16
__device__ __forceinline__ f16x2 e4m3_pair(unsigned sw, bool hi) {
  return hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)
            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false);
}

// 8 affine codes -> 8 bf16 of value 128 + q (element 2s at nibble s, 2s+1 at nibble s+4)
__device__ __forceinline__ bf16x8 affine_operand(unsigned d) {
  const unsigned mk = 0x000F000Fu, mg = 0x43004300u;
  u32x4 r;
  r.x = (d & mk) | mg;
  r.y = ((d >> 4) & mk) | mg;
  r.z = ((d >> 8) & mk) | mg;
  r.w = ((d >> 12) & mk) | mg;
  return __builtin_bit_cast(bf16x8, r);
}

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}


// fp32 -> output element
__device__ __forceinline__ float store_out(void* out, int dtype, size_t off, float v) {
  if (dtype == Q4_F32) {
    static_cast<float*>(out)[off] = v;
    return v;
  } else if (dtype == Q4_F16) {
    const f16 h = (f16)v;
    static_cast<f16*>(out)[off] = h;
    return (float)h;
  } else {
    const __bf16 h = (__bf16)v;
    static_cast<__bf16*>(out)[off] = h;
    return (float)h;
  }
}

// Cross-workgroup handoff without cache-wide invalidation: the producer's
// stores reach the coherence point through one agent-scope release fence
// (issued by one thread after a workgroup barrier has drained every wave's
// stores to L2), then an arrival counter is bumped; the consumer reads the
// published data with agent-scope loads, which bypass stale L2 lines, so no
// acquire fence (L2 invalidation) is needed.
__device__ __forceinline__ unsigned arrive(unsigned* counter) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ordered 64-bit key: larger value first, then lower index; 0 = "no value"
__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
  if (v != v) return 0ull;
  if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
  const unsigned b = __float_as_uint(v);
  const unsigned ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<unsigned long long>(ord) << 32) | static_cast<unsigned>(0xFFFFFFFFu - unsigned(n));
}

__device__ __forceinline__ unsigned long long max_key_16(unsigned long long k) {
  // max over the 16 lanes of a row group (lanes sharing lane >> 4)
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) {
    const unsigned lo = __shfl_xor(static_cast<unsigned>(k), off, 16);
    const unsigned hi = __shfl_xor(static_cast<unsigned>(k >> 32), off, 16);
    const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}


// One MFMA tile step: P panels of codes/scales in `c`/`s`, activation
// operands a[0..3] (the four 32-k steps of the tile).
template <int FMT, int P>
__device__ __forceinline__ void tile_math(f32x4 (&acc)[P][2], const u32x4 (&a)[4], const u32x4 (&c)[P],
                                          const typename std::conditional<FMT == kNvfp4, unsigned, u32x2>::type (&s)[P]) {
  if constexpr (FMT == kNvfp4) {
    f16x2 sv[P][2];
#pragma unroll
    for (int p = 0; p < P; ++p) {
      sv[p][0] = e4m3_pair(s[p], false);
      sv[p][1] = e4m3_pair(s[p], true);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < P; ++p)
        acc[p][i & 1] = mfma_f16(a[i], nvfp4_operand(c[p][i], sv[p][i >> 1][i & 1]), acc[p][i & 1]);
  } else {
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 as0 = mfma_bf16(a[0], ones, z);
    as0 = mfma_bf16(a[1], ones, as0);
    f32x4 as1 = mfma_bf16(a[2], ones, z);
    as1 = mfma_bf16(a[3], ones, as1);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      f32x4 q0 = mfma_bf16(a[0], affine_operand(c[p][0]), z);
      q0 = mfma_bf16(a[1], affine_operand(c[p][1]), q0);
      f32x4 q1 = mfma_bf16(a[2], affine_operand(c[p][2]), z);
      q1 = mfma_bf16(a[3], affine_operand(c[p][3]), q1);
      const float s0 = bf16_lo(s[p].x), b0 = bf16_hi(s[p].x);
      const float s1 = bf16_lo(s[p].y), b1 = bf16_hi(s[p].y);
      const float c0 = fmaf(-128.0f, s0, b0), c1 = fmaf(-128.0f, s1, b1);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[p][0][r];
        v = fmaf(s0, q0[r], v);
        v = fmaf(c0, as0[r], v);
        v = fmaf(s1, q1[r], v);
        v = fmaf(c1, as1[r], v);
        acc[p][0][r] = v;
      }
    }
  }
}

// Where a wave's activation operands come from.
//  * ALDS: the workgroup staged the k-range in LDS as [tile][step i][octet o]
//    [row c] 16-byte blocks (rows >= M and k >= K zero), so that lane l of
//    step i of local tile t reads block (t * 4 + i) * 64 + l: one
//    conflict-free ds_read_b128 per step.
//  * global: lane reads a[row][k0 .. k0 + 8) from its row pointer, zeros for
//    rows it does not own or k0 >= K (the only bound check of the loop).
template <int FMT, int P, bool ALDS>
struct StreamStage {
  u32x4 c[P];
  typename std::conditional<FMT == kNvfp4, unsigned, u32x2>::type s[P];
  u32x4 a[ALDS ? 1 : 4];
};

// Stage the activation k-range [kt0, kt0 + nt) tiles of rows 0..M-1 into LDS
// in the ALDS layout (whole workgroup; caller synchronizes).  a is [M][K].
__device__ __forceinline__ void stage_a_lds(u32x4* alds, const uint16_t* a, int M, int K, int kt0, int nt) {
  const int nblk = nt * 16;  // 16-byte blocks per row in the range
  for (int q = threadIdx.x; q < 16 * nblk; q += blockDim.x) {
    const int c = q / nblk, b = q - c * nblk;         // row, block along k (8 k each)
    const int t = b >> 4, i = (b >> 2) & 3, o = b & 3;
    const int k0 = (kt0 + t) * kTileK + 32 * i + 8 * o;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (c < M && k0 < K) v = *reinterpret_cast<const u32x4*>(a + static_cast<size_t>(c) * K + k0);
    alds[(t * 4 + i) * 64 + o * 16 + c] = v;
  }
}

// Stream ng groups of P panels over the tiles [kt0, kt0 + KRg) of each group
// (global packed tile indices; tile `half_t` is the 576-byte half tile, -1 if
// none), keeping D tiles of weight loads in flight across group boundaries.
// gbase(g, p): packed base of panel p of the wave's g-th group.  After the
// last tile of group g, epi(g, acc) consumes the accumulators, which restart
// at zero.  pre() runs once after the first loads are issued (the workgroup
// stages its activations there, so that the LDS fill overlaps the first HBM
// round trip; every wave must reach it).  All arguments except the
// lane-dependent A row are wave-uniform.
template <int FMT, int P, int D, bool ALDS, class GBase, class Pre, class Epi>
__device__ __forceinline__ void stream_groups(int ng, int KRg, int kt0, int half_t, const u32x4* alds,
                                              const uint16_t* arow, bool arow_ok, int K, GBase gbase, Pre pre,
                                              Epi epi) {
  const int lane = threadIdx.x & 63;
  const int o = lane >> 4;
  const int c = lane & 15;
  const int F = ng * KRg;
  using St = StreamStage<FMT, P, ALDS>;

  auto load = [&](St& st, int g, int t) {
    const int tg = kt0 + t;
    const bool half = tg == half_t;
    if constexpr (!ALDS) {
      const int kb = tg * kTileK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k0 = kb + 32 * i + 8 * o;
        st.a[i] = (arow_ok && k0 < K) ? *reinterpret_cast<const u32x4*>(arow + k0) : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint8_t* tb = gbase(g, p) + static_cast<size_t>(tg) * kTileBytes;
      if (!half) {
        st.c[p] = ld_nt16(tb + lane * 16);
        if constexpr (FMT == kNvfp4)
          st.s[p] = ld_nt4(tb + kTileCodeBytes + (c * 2 + (lane >> 5)) * 4);
        else
          st.s[p] = ld_nt8(tb + kTileCodeBytes + c * 8);
      } else {
        const u32x2 cc = ld_nt8(tb + lane * 8);
        st.c[p] = u32x4{cc.x, cc.y, 0u, 0u};
        if constexpr (FMT == kNvfp4)
          st.s[p] = ld_nt2(tb + kHalfCodeBytes + (c * 2 + (lane >> 5)) * 2);
        else
          st.s[p] = u32x2{ld_nt4(tb + kHalfCodeBytes + c * 4), 0u};  // 2nd group s = b = 0 adds 0
      }
    }
  };

  f32x4 acc[P][2];
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  St st[D];
  // load cursor (group, tile) and compute cursor
  int lg = 0, lt = 0;
#pragma unroll
  for (int d = 0; d < D; ++d) {
    if (d < F) {
      load(st[d], lg, lt);
      if (++lt == KRg) { lt = 0; ++lg; }
    }
  }
  pre();
  int cg = 0, ct = 0;
  for (int f0 = 0; f0 < F; f0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (f0 + d < F) {
        u32x4 a[4];
        if constexpr (ALDS) {
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = alds[(ct * 4 + i) * 64 + lane];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) a[i] = st[d].a[i];
        }
        tile_math<FMT, P>(acc, a, st[d].c, st[d].s);
        if (f0 + d + D < F) {
          load(st[d], lg, lt);
          if (++lt == KRg) { lt = 0; ++lg; }
        }
        if (++ct == KRg) {
          epi(cg, acc);
#pragma unroll
          for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
          ct = 0;
          ++cg;
        }
      }
    }
  }
}

// Split of a K range into the checked-free tiles and an optional tail tile.
struct KSplit {
  int nmain;  // full tiles entirely inside K
  int tail;   // 0 none, 1 half tile, 2 full tile crossing K
};
__host__ __device__ inline KSplit ksplit(int K) {
  const int Kp = (K + 63) / 64 * 64;
  const int nfull = Kp / kTileK;
  const bool half = (Kp % kTileK) != 0;
  const int full_in = K / kTileK;
  if (half) return {nfull, 1};
  if (full_in < nfull) return {full_in, 2};
  return {nfull, 0};
}

}  // namespace dev
}  // namespace q4mi
