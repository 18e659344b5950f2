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
// (mk = 0x000F000F and mg = 0x43004300 come in registers, so that each
// dword is one v_and_or_b32, which takes no literal on gfx9)
__device__ __forceinline__ bf16x8 affine_operand(unsigned d, unsigned mk, unsigned mg) {
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

// Cross-workgroup handoff without any cache-wide write-back or invalidation.
// Data meant for another workgroup (possibly on another XCD, whose L2 is not
// coherent with this one) is written with agent-scope atomic stores, which
// write through to the device coherence point; every wave waits for its own
// stores to complete (wait_stores) before the workgroup barrier, after which
// one thread bumps an arrival counter with an agent-scope atomic.  The
// workgroup that sees the final count reads the data with agent-scope loads,
// which fetch from the coherence point instead of a possibly stale L2 line.
__device__ __forceinline__ void store_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent4(float* p, f32x4 v) {
  unsigned long long* q = reinterpret_cast<unsigned long long*>(p);
  const unsigned long long lo = (static_cast<unsigned long long>(__float_as_uint(v[1])) << 32) | __float_as_uint(v[0]);
  const unsigned long long hi = (static_cast<unsigned long long>(__float_as_uint(v[3])) << 32) | __float_as_uint(v[2]);
  __hip_atomic_store(q, lo, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 1, hi, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this wave's stores and atomics have completed (stores count in vmcnt here)
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ unsigned count_arrival(unsigned* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ f32x4 load_coherent4(const float* p) {
  const unsigned long long* q = reinterpret_cast<const unsigned long long*>(p);
  const unsigned long long lo = __hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const unsigned long long hi = __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return f32x4{__uint_as_float(static_cast<unsigned>(lo)), __uint_as_float(static_cast<unsigned>(lo >> 32)),
               __uint_as_float(static_cast<unsigned>(hi)), __uint_as_float(static_cast<unsigned>(hi >> 32))};
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


// Park a finished group's accumulators in LDS: lane l writes its P f32x4
// (rows 4 (l >> 4) + r of column l & 15 of each panel) to
// wout[((g * P + p) * 64 + l)].  The streaming loop must issue no vector-
// memory instruction other than its loads (the compiler's wait counting
// across a loop with stores in it degenerates to waiting for everything), so
// the epilogues write results to global memory only after the stream.
template <int P>
__device__ __forceinline__ void stash(f32x4* wout, int g, const f32x4 (&acc)[P][2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < P; ++p) wout[(g * P + p) * 64 + lane] = acc[p][0] + acc[p][1];
}

// Per-format tile layout, the registers one lane holds for a tile of one
// panel, and the loads that fill them.  A half tile (K % 128 == 64) of the
// NVFP4 and 4-bit affine layouts is packed on its own (8 code bytes a lane);
// the b-bit widths pad K to whole tiles, so their last tile is loaded like
// any other (the streaming code zeroes its activations past K).
template <int FMT>
struct Fm;
template <>
struct Fm<kNvfp4> {
  using Codes = u32x4;
  using Scales = unsigned;
  using HalfCodes = u32x2;
  static constexpr int kTile = kTileBytes;
  __device__ static void load(Codes& c, Scales& s, const uint8_t* tb, int lane) {
    c = ld_nt16(tb + lane * 16);
    s = ld_nt4(tb + kTileCodeBytes + ((lane & 15) * 2 + (lane >> 5)) * 4);
  }
  __device__ static void load_half(HalfCodes& c, Scales& s, const uint8_t* tb, int lane) {
    c = ld_nt8(tb + lane * 8);
    s = ld_nt2(tb + kHalfCodeBytes + ((lane & 15) * 2 + (lane >> 5)) * 2);
  }
  __device__ static Codes widen(HalfCodes h) { return u32x4{h.x, h.y, 0u, 0u}; }
  __device__ static unsigned first_word(const Codes& c) { return c.x; }  // of the tile's first load
  // A full tile, or (hf, wave-uniform) the half tile, with the same two
  // loads either way so that the stream's waits stay exact: the half tile's
  // 16-byte code load covers this lane's 8 bytes and its neighbour's, its
  // scale load the word holding this lane's 2 bytes; the unused parts are
  // dropped and steps 2 and 3 (k >= 64) get zero codes and zero scales.
  __device__ static void load_any(Codes& c, Scales& s, const uint8_t* tb, int lane, bool hf) {
    const int cc = lane & 15, h = lane >> 5;
    const unsigned coff = hf ? static_cast<unsigned>(lane & ~1) * 8u : static_cast<unsigned>(lane) * 16u;
    const unsigned soff = hf ? kHalfCodeBytes + 4u * cc : kTileCodeBytes + 4u * (2 * cc + h);
    const u32x4 v = ld_nt16(tb + coff);
    const unsigned sv = ld_nt4(tb + soff);
    if (hf) {
      c = (lane & 1) ? u32x4{v.z, v.w, 0u, 0u} : u32x4{v.x, v.y, 0u, 0u};
      s = h ? sv >> 16 : sv & 0xFFFFu;
    } else {
      c = v;
      s = sv;
    }
  }
};
template <>
struct Fm<kAffine> {
  using Codes = u32x4;
  using Scales = u32x2;
  using HalfCodes = u32x2;
  static constexpr int kTile = kTileBytes;
  __device__ static void load(Codes& c, Scales& s, const uint8_t* tb, int lane) {
    c = ld_nt16(tb + lane * 16);
    s = ld_nt8(tb + kTileCodeBytes + (lane & 15) * 8);
  }
  __device__ static void load_half(HalfCodes& c, Scales& s, const uint8_t* tb, int lane) {
    c = ld_nt8(tb + lane * 8);
    s = u32x2{ld_nt4(tb + kHalfCodeBytes + (lane & 15) * 4), 0u};  // 2nd group s = b = 0 adds 0
  }
  __device__ static Codes widen(HalfCodes h) { return u32x4{h.x, h.y, 0u, 0u}; }
  __device__ static unsigned first_word(const Codes& c) { return c.x; }
};
// 8 values (128 + x_j) as bf16, x_j < 128, element j = k offset j (exact)
__device__ __forceinline__ bf16x8 bf16_128_plus(const unsigned (&x)[8]) {
  u32x4 r;
  r.x = (x[0] | 0x4300u) | ((x[1] | 0x4300u) << 16);
  r.y = (x[2] | 0x4300u) | ((x[3] | 0x4300u) << 16);
  r.z = (x[4] | 0x4300u) | ((x[5] | 0x4300u) << 16);
  r.w = (x[6] | 0x4300u) | ((x[7] | 0x4300u) << 16);
  return __builtin_bit_cast(bf16x8, r);
}

// b-bit affine: lane (c, o) owns 4 b code bytes, the 32 codes of row c at
// k = 32 i + 8 o + j as one little-endian bit stream (code (i, j) at bit
// 8 b i + b j), stored in pieces of the widest load that divides them (see
// load); the scale/bias words of row c's two groups at 8 c.
template <int B>
struct BitsCodes {
  unsigned w[B];
};
template <int B>
struct FmBits {
  using Codes = BitsCodes<B>;
  using Scales = u32x2;
  using HalfCodes = Codes;
  static constexpr int kTile = 256 * B + 128;
  // piece j of the lane's bit stream (16, 8 or 4 bytes) at j * 64 * piece +
  // lane * piece: each load of the wave reads one contiguous block
  __device__ static void load(Codes& c, Scales& s, const uint8_t* tb, int lane) {
    if constexpr (B % 4 == 0) {
#pragma unroll
      for (int j = 0; j < B / 4; ++j) {
        const u32x4 v = ld_nt16(tb + 1024 * j + lane * 16);
        c.w[4 * j] = v.x, c.w[4 * j + 1] = v.y, c.w[4 * j + 2] = v.z, c.w[4 * j + 3] = v.w;
      }
    } else if constexpr (B % 2 == 0) {
#pragma unroll
      for (int j = 0; j < B / 2; ++j) {
        const u32x2 v = ld_nt8(tb + 512 * j + lane * 8);
        c.w[2 * j] = v.x, c.w[2 * j + 1] = v.y;
      }
    } else {
#pragma unroll
      for (int j = 0; j < B; ++j) c.w[j] = ld_nt4(tb + 256 * j + lane * 4);
    }
    s = ld_nt8(tb + 256 * B + (lane & 15) * 8);
  }
  __device__ static void load_half(HalfCodes& c, Scales& s, const uint8_t* tb, int lane) { load(c, s, tb, lane); }
  __device__ static Codes widen(HalfCodes h) { return h; }
  __device__ static unsigned first_word(const Codes& c) { return c.w[0]; }
  // code j of MFMA step i
  __device__ static unsigned code(const Codes& c, int i, int j) {
    const int p = 8 * B * i + B * j;
    const int wd = p >> 5, sh = p & 31;
    unsigned v = c.w[wd] >> sh;
    if (sh + B > 32) v |= c.w[wd + 1] << (32 - sh);
    return v & ((1u << B) - 1u);
  }
  // The MFMA operand of step i: the 8 bf16 values 128 + q_j (q_j itself
  // for B = 8; element j in the low half of dword j / 2 for even j, the
  // high half for odd j).
  // B = 2: step i is the 16-bit field i & 1 of word i / 2, codes 2 bits
  // apart; masking the even and the odd codes and one byte permute put
  // q_2m and q_2m+1 16 bits apart at bit 4 m, so each dword is a shift, a
  // mask and the exponent of 128.  Other widths: bitfield extracts.
  // mk, mg: 0x00030003 and 0x43004300 in registers (one v_and_or_b32 a dword)
  __device__ static bf16x8 operand(const Codes& c, int i, unsigned mk, unsigned mg) {
    if constexpr (B == 2) {
      const unsigned d = c.w[i >> 1];
      const unsigned x = d & 0x33333333u, y = (d >> 2) & 0x33333333u;
      // bytes of step i's fields: x in the low half, y in the high half
      const unsigned z = __builtin_amdgcn_perm(y, x, (i & 1) ? 0x07060302u : 0x05040100u);
      u32x4 r;
      r.x = (z & mk) | mg;
      r.y = ((z >> 4) & mk) | mg;
      r.z = ((z >> 8) & mk) | mg;
      r.w = ((z >> 12) & mk) | mg;
      return __builtin_bit_cast(bf16x8, r);
    } else if constexpr (B == 8) {
      // the codes themselves: a byte converts to fp32 exactly
      // (v_cvt_f32_ubyte*), and an integer below 256 keeps 8 significant
      // bits, so the fp32 value's high half is its exact bf16
      u32x4 r;
      unsigned* rr = reinterpret_cast<unsigned*>(&r);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const unsigned d = c.w[2 * i + h];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const unsigned lo = __float_as_uint(static_cast<float>((d >> (16 * j)) & 0xFFu));
          const unsigned hi = __float_as_uint(static_cast<float>((d >> (16 * j + 8)) & 0xFFu));
          rr[2 * h + j] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);
        }
      }
      return __builtin_bit_cast(bf16x8, r);
    } else {
      unsigned x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = code(c, i, j);
      return bf16_128_plus(x);
    }
  }
};
template <>
struct Fm<kAffineBits + 2> : FmBits<2> {};
template <>
struct Fm<kAffineBits + 3> : FmBits<3> {};
template <>
struct Fm<kAffineBits + 5> : FmBits<5> {};
template <>
struct Fm<kAffineBits + 6> : FmBits<6> {};
template <>
struct Fm<kAffineBits + 8> : FmBits<8> {};

// One MFMA tile step: P panels of codes/scales in `c`/`s`, activation
// operands a[0..3] (the four 32-k steps of the tile).
// Affine widths: a code q < 128 becomes the exact bf16 128 + q, so that
// sum_k a (128 + q) runs on the bf16 MFMA and the group sum sum_k a on the
// same MFMA against a 0/1 operand; per group of 64
//   sum_k a w = s sum a (128 + q) + (b - 128 s) sum a,
// and 8-bit codes, exact in bf16 as they are,
//   sum_k a w = s sum a q + b sum a.
template <int FMT, int P>
__device__ __forceinline__ void tile_math(f32x4 (&acc)[P][2], const u32x4 (&a)[4],
                                          const typename Fm<FMT>::Codes (&c)[P],
                                          const typename Fm<FMT>::Scales (&s)[P]) {
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
    // b-bit widths: the group sums on the MFMA with the activations as the B
    // operand, against a 0/1 operand whose rows 0-3 take the tile's first
    // group (steps 0, 1) and rows 4-7 its second (steps 2, 3): lane (c, o)
    // then holds token c's sum over group o for o < 2 and 0 for o >= 2, the
    // A operand of an fp32 16x16x4 MFMA over the groups (k = o) that adds
    // the bias terms.  The 4-bit width, whose GEMM configurations run more
    // waves a SIMD, keeps them on FMAs (sums against ones, token-major).
    constexpr bool BM = FMT != kAffine;
    const int row = threadIdx.x & 15, og = (threadIdx.x >> 4) & 1;
    const unsigned g0 = !BM || row < 4 ? 0x3F803F80u : 0u, g1 = !BM || (row >= 4 && row < 8) ? 0x3F803F80u : 0u;
    const u32x4 sel0 = {g0, g0, g0, g0}, sel1 = {g1, g1, g1, g1};
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    unsigned mk = FMT == kAffine ? 0x000F000Fu : 0x00030003u, mg = 0x43004300u;
    asm("" : "+v"(mk), "+v"(mg));  // operand constants in registers (v_and_or_b32)
    f32x4 gs, as0, as1;
    if constexpr (BM) {
      gs = mfma_bf16(sel0, __builtin_bit_cast(bf16x8, a[0]), z);
      gs = mfma_bf16(sel0, __builtin_bit_cast(bf16x8, a[1]), gs);
      gs = mfma_bf16(sel1, __builtin_bit_cast(bf16x8, a[2]), gs);
      gs = mfma_bf16(sel1, __builtin_bit_cast(bf16x8, a[3]), gs);
    } else {
      const bf16x8 ones = __builtin_bit_cast(bf16x8, sel0);
      as0 = mfma_bf16(a[0], ones, z);
      as0 = mfma_bf16(a[1], ones, as0);
      as1 = mfma_bf16(a[2], ones, z);
      as1 = mfma_bf16(a[3], ones, as1);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      f32x4 q0, q1;
      const float off = FMT == kAffineBits + 8 ? 0.0f : -128.0f;  // the 128 under each code (none at 8 bits)
      if constexpr (FMT == kAffine) {
        q0 = mfma_bf16(a[0], affine_operand(c[p][0], mk, mg), z);
        q0 = mfma_bf16(a[1], affine_operand(c[p][1], mk, mg), q0);
        q1 = mfma_bf16(a[2], affine_operand(c[p][2], mk, mg), z);
        q1 = mfma_bf16(a[3], affine_operand(c[p][3], mk, mg), q1);
      } else {
        f32x4 q[2] = {z, z};
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i >> 1] = mfma_bf16(a[i], Fm<FMT>::operand(c[p], i, mk, mg), q[i >> 1]);
        q0 = q[0];
        q1 = q[1];
      }
      const float s0 = bf16_lo(s[p].x), s1 = bf16_lo(s[p].y);
      if constexpr (BM) {
        // sum_g (b_g + off s_g) (group sum) on the fp32 MFMA: lane (c, o)
        // gives column c's coefficient of group o & 1 (A's rows o >= 2 are 0)
        const unsigned sw = og ? s[p].y : s[p].x;
        acc[p][1] =
            __builtin_amdgcn_mfma_f32_16x16x4f32(gs[0], fmaf(off, bf16_lo(sw), bf16_hi(sw)), acc[p][1], 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[p][0][r] = fmaf(s1, q1[r], fmaf(s0, q0[r], acc[p][0][r]));
      } else {
        const float c0 = fmaf(off, s0, bf16_hi(s[p].x)), c1 = fmaf(off, s1, bf16_hi(s[p].y));
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
}

// Where a wave's activation operands come from.
//  * kAStaged: the workgroup staged its k-range of the activations in LDS
//    (stage_issue / stage_wait); ALds gives each lane its read address.
//  * kARing: the wave itself moves each tile's 16 activation rows into a
//    ring of D LDS slots with direct-to-LDS loads issued together with that
//    tile's weight loads (ARing), so the math of a tile waits only for that
//    tile's own loads.
//  * kAGlobal: lane (c, o) loads a[row c][k0 .. k0 + 8) straight into
//    registers from its row pointer.
//  * kAStagedRows: the workgroup staged whole rows of an activation matrix
//    in LDS (all its k-range, row stride stage_row_stride); each group names
//    the staged row every lane reads (GroupPtrs::alds), which is recorded with
//    the tile's loads, so the activations cost no memory instruction in the
//    stream.
enum AMode { kAStaged = 0, kARing = 1, kAGlobal = 2, kAStagedRows = 3 };

template <int FMT, int P, int AM>
struct StreamStage {
  typename Fm<FMT>::Codes c[P];
  typename Fm<FMT>::Scales s[P];
  u32x4 a[AM == kAGlobal ? 4 : 1];
  unsigned arow;  // kAStagedRows: LDS byte offset of this lane's staged row for this tile
};

// Ring slots of kARing: slot d holds one tile of 16 rows x 128 k (f16/bf16)
// as 16 rows of 256 bytes.  The loads that fill it move 4 rows x 256 bytes
// each (row group j = rows 4j .. 4j + 3; lane l: row 4j + (l >> 4), LDS
// position l & 15 of that row); the 16-byte chunk q (k = 8q .. 8q + 7) of
// row r is stored at position q ^ r, so that the 16 rows of one k-step
// (lane (c, o) reads row c, chunk 4i + o) fall in 16 different bank groups
// and the global side of every load still covers 4 whole 256-byte row
// segments.
constexpr int kRingSlot = 4096;
typedef __attribute__((address_space(3))) char lds_char;
__device__ __forceinline__ unsigned lds_offset(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<size_t>((const lds_char*)(p)));
}
struct ARing {
  unsigned base;   // LDS offset of this wave's D slots (wave-uniform)
  unsigned rd[4];  // this lane's read offset of k-step i in slot 0
};
__device__ __forceinline__ ARing aring_view(unsigned base) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, o = lane >> 4;
  ARing r;
  r.base = base;
#pragma unroll
  for (int i = 0; i < 4; ++i) r.rd[i] = base + 256u * c + 16u * static_cast<unsigned>((4 * i + o) ^ c);
  return r;
}
// Element offset, within a tile, of the chunk that lane l moves for row
// group j (row 4j + (l >> 4)); add it to that row's base pointer.
__device__ __forceinline__ int ring_chunk(int j) {
  const int lane = threadIdx.x & 63;
  return 8 * ((lane & 15) ^ (4 * j + (lane >> 4)));
}
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
// One direct-to-LDS load of 16 bytes per lane (lane l lands at lds_off +
// 16 l), issued as inline assembly so that the compiler does not count it
// among its outstanding loads: with such loads pending it would otherwise
// wait for every load before each use of a loaded register.  Its waits for
// the other loads then count fewer younger loads than are really in
// flight, which only makes them wait longer; the ring reads are ordered
// after these loads by a dependency on a load issued after them (loads
// complete in order).
__device__ __forceinline__ void dma16_to_lds(const void* src, unsigned lds_off) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_off) : "memory");
}

// Staged activations in LDS, row-major: row c (< M) of a workgroup's
// k-range of nt tiles is nt * 256 contiguous bytes at c * RS, with
// RS = nt * 256 + 16, so that the 16 rows of one 32-k step sit in 16
// different 16-byte bank groups (conflict-free ds_read_b128: lane (c, o)
// reads row c, k-octet o).  Lanes of rows c >= M read a zero row placed
// after the M rows.  For local tile t and step i, lane (c, o) reads
// base + t * 256 + i * 64 with base = c * RS + o * 16.
struct ALds {
  const char* base;  // this lane's address of step 0 of the wave's local tile 0
};
__host__ __device__ inline int stage_row_stride(int nt) { return nt * 256 + 16; }
__host__ __device__ inline int stage_bytes(int M, int nt) {
  return M * stage_row_stride(nt) + (M < 16 ? nt * 256 : 0);
}
__device__ __forceinline__ ALds alds_view(const char* stage, int nt_staged, int M, int t0) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15, o = lane >> 4;
  const int rs = stage_row_stride(nt_staged);
  ALds v;
  v.base = stage + (c < M ? c * rs : M * rs) + o * 16 + t0 * 256;
  return v;
}

// Staging of tiles [kt0, kt0 + nt) of rows 0..M-1 of a [M][K] into LDS
// (whole workgroup).  One direct-to-LDS load moves 64 consecutive 16-byte
// k-chunks of one row (1 KiB contiguous in both memories; lane l lands at
// the load's LDS base + 16 l); lanes past the range or at k >= K load
// nothing and the bytes they cover are never read as data (k >= K is
// written as zeros first).  Rows are dealt to the waves; each row's loads
// start at a workgroup-dependent block so that the CUs of an XCD do not all
// read the same lines at the same time.  stage_issue only
// issues the loads, so that they travel together with the first weight
// tiles; stage_wait (after those weight loads) waits for exactly the staging
// loads and synchronizes the workgroup.
struct StageGeom {
  const uint16_t* a;
  int M, K, kt0, nt, rs;
  int bpr;     // 1 KiB load blocks per row
};
__device__ __forceinline__ StageGeom stage_geom(const uint16_t* a, int M, int K, int kt0, int nt) {
  StageGeom g;
  g.a = a;
  g.M = M;
  g.K = K;
  g.kt0 = kt0;
  g.nt = nt;
  g.rs = stage_row_stride(nt);
  g.bpr = (nt * 16 + 63) / 64;
  return g;
}
__device__ __forceinline__ void stage_issue(const StageGeom& g, u32x4* lds) {
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nw = blockDim.x >> 6;
  char* const lb = reinterpret_cast<char*>(lds);
  const int kbase = g.kt0 * kTileK;
  const int nch = g.nt * 16;                                // 16-byte chunks per row
  const int kch = min(nch, max(0, (g.K - kbase + 7) / 8));  // chunks holding k < K
  // chunks at k >= K (the k-padding of the last tile) -> zeros; rows handled by waves
  if (kch < nch)
    for (int c = w; c < g.M; c += nw)
      for (int ch = kch + lane; ch < nch; ch += 64)
        *reinterpret_cast<u32x4*>(lb + c * g.rs + ch * 16) = u32x4{0u, 0u, 0u, 0u};
  if (g.M < 16)  // the zero row
    for (int ch = threadIdx.x; ch < nch; ch += blockDim.x)
      *reinterpret_cast<u32x4*>(lb + g.M * g.rs + ch * 16) = u32x4{0u, 0u, 0u, 0u};
  // rows are dealt to waves; within a row the 1 KiB blocks start at a
  // workgroup-dependent block (no integer division in the loop)
  int b0 = static_cast<int>(blockIdx.x) * 7;
  b0 -= (b0 / g.bpr) * g.bpr;
  for (int c = w; c < g.M; c += nw) {
    const uint16_t* row = g.a + static_cast<size_t>(c) * g.K + kbase;
    char* const lrow = lb + c * g.rs;
    int b = b0;
    for (int j = 0; j < g.bpr; ++j) {
      const int ch = b * 64 + lane;
      if (ch < kch) __builtin_amdgcn_global_load_lds(row + ch * 8, lrow + b * 1024, 16, 0, 0);
      if (++b == g.bpr) b = 0;
    }
  }
}
// NLATER = vector-memory instructions this wave issued after stage_issue.
// A plain barrier, not __syncthreads: the latter's fence would wait for every
// outstanding load (the weight tiles too), since direct-to-LDS loads count as
// vector-memory operations.
template <int NLATER>
__device__ __forceinline__ void stage_wait() {
  static_assert(NLATER >= 0 && NLATER < 64, "vmcnt range");
  // s_waitcnt vmcnt(NLATER) (bits 3:0 and 15:14) lgkmcnt(0), expcnt left at its maximum
  __builtin_amdgcn_s_waitcnt((NLATER & 15) | ((NLATER >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
}

// Where group g's data lives: the packed base of each of its P panels and,
// for the activations (valid rows for every lane: rows past the real ones
// only feed output rows that are never stored)
//  * kAGlobal: arsrc and aoff, this lane's row (c = lane & 15);
//  * kARing: ar[j], the row this lane moves for row group j plus
//    ring_chunk(j).
// kAGlobal: the activations are read through a buffer resource over the
// whole activation matrix; a lane whose row holds no token gets an offset
// past the resource's end, so its loads return zeros without touching
// memory, and every load stays one unconditional instruction (the
// compiler's wait counting stays exact).
constexpr unsigned kDeadLane = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t act_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 act_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}

template <int P>
struct GroupPtrs {
  const uint8_t* panel[P];
  const uint16_t* ar[4];
  __amdgpu_buffer_rsrc_t arsrc;  // kAGlobal: the activation matrix
  unsigned aoff;                 // kAGlobal: byte offset of this lane's row, or kDeadLane
  unsigned alds;                 // kAStagedRows: LDS byte offset of this lane's staged row
};

// Stream ng groups of P panels over the tiles [kt0, kt0 + KRg) of each group
// (global packed tile indices; if half_t falls in that range it must be the
// range's last tile, the 576-byte half tile), keeping D tiles of weight loads
// in flight across group boundaries.  group(g, ptrs) fills group g's
// pointers; it is called when the load cursor enters a group and must give
// in-bounds pointers for any g >= 0 (the prologue loads D tiles even when the
// wave has fewer).  After the last tile of group g, epi(g, acc) consumes the
// accumulators (it must not touch global memory: stores inside the loop
// would make the compiler's wait counting degenerate), which restart at zero;
// the half tile of every group is added afterwards through epi_add(g, acc).
// pre_issue() runs before the first weight loads and pre() after them (the
// workgroup stages its activations across the two, so both travel in the
// same round trip; every wave must reach pre()).  K is the activations' row
// length (kAGlobal and kARing: a multiple of 64).  All arguments except the
// lane-dependent pointers are wave-uniform.
template <int FMT, int P, int D, int AM, bool IH = false, class Group, class PreIssue, class Pre, class Epi,
          class EpiAdd>
__device__ __forceinline__ void stream_groups(int ng, int KRg, int kt0, int half_t, ALds al, ARing ring, int K,
                                              Group group, PreIssue pre_issue, Pre pre, Epi epi, EpiAdd epi_add) {
  constexpr bool ALDS = AM == kAStaged;
  constexpr bool STAGED = AM == kAStaged || AM == kAStagedRows;  // activations complete in LDS before the math
  // IH (NVFP4 with rows staged, whose k-padding is zero in LDS): the half
  // tile streams inline as each group's last tile (Fm::load_any), instead of
  // in a pass of its own after the stream
  constexpr bool INL = IH && AM == kAStagedRows && FMT == kNvfp4;
  const int lane = threadIdx.x & 63;
  const int o = lane >> 4;
  const int c = lane & 15;
  const bool has_half = half_t >= kt0 && half_t < kt0 + KRg;
  const int KRf = (has_half && !INL) ? KRg - 1 : KRg;  // tiles streamed per group
  const int F = ng * KRf;
  using St = StreamStage<FMT, P, AM>;

  // Global activations: a full tile lies entirely below K, so its loads are
  // unconditional (exact waits).  The half tile's k >= K half is read at k 0
  // and zeroed.
  // kARing: the tile's 4 row-group loads into slot d go first (the asm's
  // memory clobber keeps the weight loads after them), so that a wait for the
  // tile's first weight load also covers its activations.
  auto load_a = [&](St& st, const GroupPtrs<P>& gp, int tg, int d) {
    if constexpr (AM == kAGlobal) {
      const unsigned kb = static_cast<unsigned>(tg * kTileK + 8 * o) * 2u;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.a[i] = act_load16(gp.arsrc, gp.aoff + kb + 64u * i);
    } else if constexpr (AM == kAStagedRows) {
      st.arow = gp.alds;
    } else if constexpr (AM == kARing) {
      const int kb = tg * kTileK;
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_to_lds(gp.ar[j] + kb, ring.base + d * kRingSlot + j * 1024);
    }
  };
  // half tile: chunks at k >= K are zeros (the weights there are zero, but
  // the activations past the row end need not be finite)
  auto load_a_half = [&](St& st, const GroupPtrs<P>& gp, int d) {
    if constexpr (AM == kAGlobal) {
      const int kb = half_t * kTileK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k0 = kb + 32 * i + 8 * o;
        st.a[i] = act_load16(gp.arsrc, k0 < K ? gp.aoff + static_cast<unsigned>(k0) * 2u : kDeadLane);
      }
    } else if constexpr (AM == kAStagedRows) {
      st.arow = gp.alds;  // the staged k-padding is zero
    } else if constexpr (AM == kARing) {
      const int kb = half_t * kTileK;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const unsigned dst = ring.base + d * kRingSlot + j * 1024;
        if (ring_chunk(j) < kTileK / 2)
          dma16_to_lds(gp.ar[j] + kb, dst);
        else
          *(lds_u32x4*)(static_cast<size_t>(dst + 16u * static_cast<unsigned>(lane))) = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto load = [&](St& st, const GroupPtrs<P>& gp, int t, int d) {
    const int tg = kt0 + t;
    load_a(st, gp, tg, d);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      if constexpr (INL)
        Fm<FMT>::load_any(st.c[p], st.s[p], gp.panel[p] + static_cast<size_t>(tg) * Fm<FMT>::kTile, lane,
                          tg == half_t);
      else
        Fm<FMT>::load(st.c[p], st.s[p], gp.panel[p] + static_cast<size_t>(tg) * Fm<FMT>::kTile, lane);
    }
  };
  auto load_half_w = [&](St& st, const GroupPtrs<P>& gp) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      typename Fm<FMT>::HalfCodes hc;
      Fm<FMT>::load_half(hc, st.s[p], gp.panel[p] + static_cast<size_t>(half_t) * Fm<FMT>::kTile, lane);
      st.c[p] = Fm<FMT>::widen(hc);
    }
  };
  auto load_half = [&](St& st, const GroupPtrs<P>& gp, int d) {
    load_a_half(st, gp, d);
    load_half_w(st, gp);
  };

  f32x4 acc[P][2];
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  St st[D];
  int lg = 0, lt = 0;  // load cursor (group, tile)
  int cg = 0, ct = 0;  // compute cursor
  GroupPtrs<P> cur;    // the load cursor's group
  group(0, cur);
  // (>=: a range of only the half tile, KRf == 0, keeps t = 0, the half tile)
  auto load_next = [&](St& x, int d) {
    load(x, cur, lt, d);
    if (++lt >= KRf) {
      lt = 0;
      ++lg;
      group(lg, cur);
    }
  };
  // kARing: the read addresses pass through an empty asm that takes the
  // tile's first weight word, so the reads wait for that load and hence for
  // the activation loads issued before it.
  auto tile_a = [&](const St& x, int t, int d, u32x4 (&a)[4]) {
    if constexpr (ALDS) {
      const char* pa = al.base + t * 256;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4*>(pa + i * 64);
    } else if constexpr (AM == kAStagedRows) {
      const char* pa = al.base + x.arow + t * 256;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const u32x4*>(pa + i * 64);
    } else if constexpr (AM == kARing) {
      unsigned off = static_cast<unsigned>(d * kRingSlot);
      asm volatile("" : "+v"(off) : "v"(Fm<FMT>::first_word(x.c[0])));
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *(const lds_u32x4*)(static_cast<size_t>(ring.rd[i] + off));
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = x.a[i];
    }
  };
  auto compute_next = [&](const St& x, int d) {
    u32x4 a[4];
    tile_a(x, ct, d, a);
    tile_math<FMT, P>(acc, a, x.c, x.s);
    if (++ct == KRf) {
      epi(cg, acc);
#pragma unroll
      for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      ct = 0;
      ++cg;
    }
  };

  // Prologue: D tiles are loaded whatever F is (tiles past the wave's work
  // read in-bounds panels, or the half tile plus the zero guard behind the
  // last panel, and are never computed), so the code from here to
  // the steady loop is straight-line and every wait the compiler places in it
  // counts exactly the younger loads.  The steady loop issues exactly D loads
  // per D tiles of math with no condition around any load, so the wait before
  // each tile covers only that tile's loads; the drain computes the last
  // tiles with the remaining loads issued under conditions.
  // With kAGlobal or kARing and no full tile (a range of only the half tile,
  // or none), the prologue is skipped: its full-tile activation loads would
  // read past the end of rows shorter than a tile.  pre() must then not rely
  // on the prologue's loads (it does not in these modes).
  // The half tiles' weights of the first D groups are loaded before anything
  // else (not in the ring mode, whose half-tile activations move with its
  // own slots): the data is there when the half-tile math comes after the
  // stream, instead of one more memory round trip then.  Being older than
  // every load of the stream, these loads leave the stream's waits exact.
  const bool pre_half = has_half && AM != kARing && !INL;
  struct HalfW {
    typename Fm<FMT>::HalfCodes c[P];
    typename Fm<FMT>::Scales s[P];
  } hpre[D];
  if (pre_half) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      GroupPtrs<P> hp;
      group(d, hp);
#pragma unroll
      for (int p = 0; p < P; ++p)
        Fm<FMT>::load_half(hpre[d].c[p], hpre[d].s[p], hp.panel[p] + static_cast<size_t>(half_t) * Fm<FMT>::kTile,
                           lane);
    }
  }
  pre_issue();
  if (STAGED || KRf > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load_next(st[d], d);
      __builtin_amdgcn_sched_barrier(0);  // keep the steady loop's load order (see the waits below)
    }
    pre();
    int f = 0;
    for (; f + 2 * D <= F; f += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        compute_next(st[d], d);
        load_next(st[d], d);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (f + d < F) {
        compute_next(st[d], d);
        if (f + d + D < F) load_next(st[d], d);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d)
      if (f + D + d < F) compute_next(st[d], d);
  } else {
    pre();
  }
  if (KRf == 0) {  // a range of only the half tile: every group still owns a result
    for (int gg = 0; gg < ng; ++gg) epi(gg, acc);
  }

  // half tiles: loads of up to D groups in flight (the first D groups'
  // weights are already in hpre), then their math
  if (has_half && !INL) {
    for (int g0 = 0; g0 < ng; g0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (g0 + d < ng) {
          GroupPtrs<P> hp;
          group(g0 + d, hp);
          if (pre_half && g0 == 0) {
            load_a_half(st[d], hp, d);
#pragma unroll
            for (int p = 0; p < P; ++p) {
              st[d].c[p] = Fm<FMT>::widen(hpre[d].c[p]);
              st[d].s[p] = hpre[d].s[p];
            }
          } else {
            load_half(st[d], hp, d);
          }
        }
      }
#pragma unroll
      for (int d = 0; d < D; ++d) {
        if (g0 + d < ng) {
          f32x4 hacc[P][2];
#pragma unroll
          for (int p = 0; p < P; ++p) hacc[p][0] = hacc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
          u32x4 a[4];
          tile_a(st[d], KRg - 1, d, a);
          tile_math<FMT, P>(hacc, a, st[d].c, st[d].s);
          epi_add(g0 + d, hacc);
        }
      }
    }
  }
  // loads past the wave's work may still be writing the ring: they must land
  // before the workgroup can end and its LDS be handed to another
  if constexpr (AM == kARing) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Park a finished group's P panels in a row-major LDS result block
// res[m][col] (row stride rs floats; col0 = first column of the group):
// lane l holds rows 4 (l >> 4) + r of column l & 15.  Rows >= M are dropped.
template <int P, bool ADD>
__device__ __forceinline__ void stash_rows(float* res, int rs, int col0, int M, const f32x4 (&acc)[P][2]) {
  const int lane = threadIdx.x & 63;
  const int o = lane >> 4, c = lane & 15;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const f32x4 v = acc[p][0] + acc[p][1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * o + r;
      if (m < M) {
        float* q = res + m * rs + col0 + p * 16 + c;
        *q = ADD ? *q + v[r] : v[r];
      }
    }
  }
}

// Add a half tile's accumulators to a stashed group result.
template <int P>
__device__ __forceinline__ void stash_add(f32x4* wout, int g, const f32x4 (&acc)[P][2]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int p = 0; p < P; ++p) wout[(g * P + p) * 64 + lane] += acc[p][0] + acc[p][1];
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
