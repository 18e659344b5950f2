// W4A16 skinny GEMM kernels for gfx950 (MI355X): NVFP4 and MLX-style affine 4-bit.
//
// y[m][n] = sum_k a[m][k] w[n][k] for M <= 16 activation rows.  [gemma-cuda-hybrid
// README, "Everything it has": one tensor-core GEMM for every M <= 16 product,
// FP4 -> f16 dequant in registers from an offline-repacked layout, 16-byte
// loads that do not pollute the cache; TensorFold issue "Proposal: Gemma 4 on
// CUDA", "Why now": qlinear's affine 4-bit path with 64-value group sums.]
//
// Design (gfx950):
//  * A workgroup owns a block of PB panels (16 output columns each) and one
//    of KS ranges of 128-k tiles.  It stages that k-range of the activations
//    in LDS once, in MFMA operand order, then its W waves stream groups of P
//    panels (round-robin inside the block) through the k-range; the register
//    ring keeps D tiles of weight loads in flight across group boundaries.
//  * Per tile each lane issues one 16-byte non-temporal load of codes per
//    panel (1 KiB contiguous per wave) plus one small scale load; the four
//    activation operands come from LDS with conflict-free ds_read_b128.
//  * KS > 1: each workgroup writes fp32 partial sums to the workspace; the
//    last of the KS workgroups of a block (arrival counter) adds them in
//    ks order (deterministic) and applies the epilogue.
//  * NVFP4: v_cvt_scalef32_pk_f16_fp4 turns 2 codes into 2 f16 (scale operand
//    1.0: the hardware applies only its power-of-two part), then one
//    v_pk_mul_f16 by the E4M3 group scale (decoded by v_cvt_scalef32_pk_f16_fp8).
//    e2m1 * e4m3 is exact in f16, so B holds the exact weight / g; the fp32
//    accumulator is multiplied by the global scale once at the end.
//  * Affine: codes become bf16 (128 + q) by OR-ing them under the exponent of
//    128.0; an extra MFMA against a ones operand gives the 64-k group sums of
//    the activations in the accumulator layout, and per group
//      y += s * sum a (128 + q) + (b - 128 s) * sum a.
//  * v_mfma_f32_16x16x32_{f16,bf16}: A = activations (row m = lane & 15),
//    B = weights (column lane & 15), k-octet lane >> 4; D lane holds column
//    lane & 15, rows 4 (lane >> 4) + r.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "q4mi_tiles.h"

namespace q4mi {
namespace {
using namespace dev;

struct GemmParams {
  GemmArgs g;
  int npanels;
  int ntiles;      // packed tiles per panel, half tile included
  int half_t;      // packed index of the half tile, -1 if none
  int KS, KR;      // k-splits and tiles per split
  int KW;          // waves splitting a workgroup's k-range (one group per wave if > 1), a power of two
  int kw_shift;    // log2(KW)
  int PB;          // panels per workgroup block
  int nblocks;     // panel blocks
  int res_off;     // byte offset of the result area in dynamic LDS
  int rs;          // result row stride in floats (PB * 16 + 4)
  unsigned ks_magic;   // ceil(2^32 / KS): block of a workgroup without a division
  unsigned nc4_magic;  // ceil(2^32 / (PB * 4)): row of an epilogue item without a division
  unsigned nc4_magic_last;  // the same for the last block's (panels left) * 4
  float* partial;  // [KS][M][N] fp32 (KS > 1)
  unsigned* bcnt;  // [nblocks] arrival counters (KS > 1), left at zero
};

constexpr int kMaxKS = 8;  // partial sums summed per output by the last workgroup
constexpr size_t kGemmLdsMax = 160 * 1024 - 512;  // dynamic LDS per workgroup (static LDS is < 512 B)

// LDS bytes of one workgroup: staged activations (+ zero row), then KW row-major
// result blocks [M][PB * 16 + 4]
__host__ __device__ inline size_t gemm_res_offset(int M, int KR, bool ring, int W, int D) {
  return ring ? static_cast<size_t>(W) * D * kRingSlot : (static_cast<size_t>(stage_bytes(M, KR)) + 15) / 16 * 16;
}
__host__ __device__ inline size_t gemm_lds_bytes(int M, int KR, int KW, int PB, bool ring, int W, int D) {
  return gemm_res_offset(M, KR, ring, W, D) + static_cast<size_t>(KW) * M * (PB * 16 + 4) * 4;
}

// output element group (m, n .. n + 3) -> stored values (rounded to the output
// type).  Streaming stores: the outputs are not re-read by this kernel.
__device__ __forceinline__ f32x4 store_out4(void* out, int dtype, size_t off, f32x4 v) {
  if (dtype == Q4_F32) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(static_cast<float*>(out) + off));
    return v;
  } else if (dtype == Q4_F16) {
    const f16x2 h0 = {(f16)v[0], (f16)v[1]}, h1 = {(f16)v[2], (f16)v[3]};
    const u32x2 w = {__builtin_bit_cast(unsigned, h0), __builtin_bit_cast(unsigned, h1)};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(static_cast<f16*>(out) + off));
    return f32x4{(float)h0[0], (float)h0[1], (float)h1[0], (float)h1[1]};
  } else {
    const __bf16 b0 = (__bf16)v[0], b1 = (__bf16)v[1], b2 = (__bf16)v[2], b3 = (__bf16)v[3];
    const u32x2 w = {static_cast<unsigned>(__builtin_bit_cast(unsigned short, b0)) |
                         (static_cast<unsigned>(__builtin_bit_cast(unsigned short, b1)) << 16),
                     static_cast<unsigned>(__builtin_bit_cast(unsigned short, b2)) |
                         (static_cast<unsigned>(__builtin_bit_cast(unsigned short, b3)) << 16)};
    __builtin_nontemporal_store(w, reinterpret_cast<u32x2*>(static_cast<__bf16*>(out) + off));
    return f32x4{(float)b0, (float)b1, (float)b2, (float)b3};
  }
}

__device__ __forceinline__ unsigned long long max_key_64(unsigned long long k) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned lo = __shfl_xor(static_cast<unsigned>(k), off);
    const unsigned hi = __shfl_xor(static_cast<unsigned>(k >> 32), off);
    const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}

// ---- fused sampling ---------------------------------------------------------
// [TensorSharp docs, Gemma 4, 4.8 "Logit softcap"]: z = cap tanh(y / cap).
// [gemma-cuda-hybrid README, "Everything it has"]: temperature sampling by
// the Gumbel-max trick (temperature 0: greedy).  The noise generator is
// Philox4x32-10 (Salmon et al., SC 2011): key (seed lo, seed hi), counter
// (column n, row / 4, offset, 0), word row % 4; U = (2 (x >> 9) + 1) 2^-24 in
// (0, 1), exact in fp32; G = -ln(-ln U).  One call gives the four rows of a
// column that an MFMA accumulator lane holds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, unsigned k0, unsigned k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const unsigned hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const unsigned hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = u32x4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
  }
  return c;
}
__device__ __forceinline__ float uniform_of(unsigned x) {
  return static_cast<float>(((x >> 9) << 1) | 1u) * 0x1p-24f;  // exact: an odd integer < 2^24, times 2^-24
}
// -ln(-ln U) with the hardware base-2 log (1 ulp over the whole U grid,
// including next to 1, measured on MI355X): a few 1e-6 absolute
__device__ __forceinline__ float gumbel_of(float u) {
  constexpr float kLn2 = 0.69314718055994531f;
  const float t = -__builtin_amdgcn_logf(u) * kLn2;  // -ln U > 0
  return -__builtin_amdgcn_logf(t) * kLn2;
}
// cap tanh(y / cap) as cap (1 - 2 / (1 + e^(2y/cap))): exp2 and a reciprocal,
// a few 1e-7 absolute in tanh; saturates to +-cap
__device__ __forceinline__ float softcap_of(float y, float cap) {
  const float e = __builtin_amdgcn_exp2f(y * (2.8853900817779268f / cap));  // e^(2 y / cap)
  return cap * (1.0f - 2.0f * __builtin_amdgcn_rcpf(1.0f + e));
}
// the sampling key of row m, column n from the final logit y
__device__ __forceinline__ unsigned long long sample_key(const GemmArgs& g, float y, float noise, int n) {
  const float z = g.softcap > 0.f ? softcap_of(y, g.softcap) : y;
  const float sc = g.inv_temp > 0.f ? fmaf(z, g.inv_temp, noise) : z;
  return argmax_key(sc, n);
}
// noise of rows 4 q .. 4 q + 3 of column n (all 0 when greedy)
__device__ __forceinline__ f32x4 gumbel4(const GemmArgs& g, int n, int q) {
  if (!(g.inv_temp > 0.f)) return f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 x = philox4x32_10(u32x4{static_cast<unsigned>(n), static_cast<unsigned>(q), g.offset, 0u}, g.seed_lo,
                                g.seed_hi);
  return f32x4{gumbel_of(uniform_of(x.x)), gumbel_of(uniform_of(x.y)), gumbel_of(uniform_of(x.z)),
               gumbel_of(uniform_of(x.w))};
}

// RING: every wave moves its own tiles' activations into an LDS ring
// together with their weight loads (kARing) instead of the workgroup
// staging its k-range up front; chosen when each wave streams a single panel
// group, so that staging would save no re-reads and only hold back the first
// tile's math until the whole range has landed.
// SAMPLE: the fused-sampling variant (qgemm_nvfp4_sample); the plain GEMM
// kernels carry none of its code.
template <int FMT, int P, int W, int D, bool RING, bool SAMPLE>
__global__ __launch_bounds__(64 * W) void qgemm_kernel(GemmParams kp) {
  // dynamic LDS: staged activations (+ zero row), or with RING the W rings
  // of D slots; then KW row-major result blocks [M][rs]
  extern __shared__ u32x4 lds[];
  __shared__ unsigned long long sbest[16];
  __shared__ int s_last;
  const GemmArgs& g = kp.g;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (no integer division: KW and W are powers of two, KS by its magic)
  const int KS = kp.KS, KW = kp.KW, kws = kp.kw_shift;
  constexpr int kWShift = W == 8 ? 3 : (W == 4 ? 2 : (W == 2 ? 1 : 0));
  static_assert((1 << kWShift) == W, "W is a power of two");
  const int PWv = W >> kws;                                // wave columns (panel groups in parallel)
  const int kw = w & (KW - 1), pw = w >> kws;
  const int pb = KS == 1 ? static_cast<int>(blockIdx.x) : static_cast<int>(__umulhi(blockIdx.x, kp.ks_magic));
  const int ks = static_cast<int>(blockIdx.x) - pb * KS;
  const int kt0 = ks * kp.KR;
  const int KRg = min(kp.ntiles, kt0 + kp.KR) - kt0;       // this workgroup's tiles
  const int KRw = (KRg + KW - 1) >> kws;                   // per k-split wave
  const int wt0 = min(KRg, kw * KRw);
  const int wtn = min(KRg, wt0 + KRw) - wt0;
  const int p0 = pb * kp.PB;
  const int pend = min(kp.npanels, p0 + kp.PB);
  const int ngb = (pend - p0 + P - 1) / P;                 // panel groups in the block
  const int ng = ngb > pw ? (ngb - pw + PWv - 1) >> (kWShift - kws) : 0;  // this wave's: pw, pw + PWv, ...
  const int M = g.M, rs = kp.rs;
  float* const res = reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + kp.res_off);
  float* const wres = res + static_cast<size_t>(kw) * M * rs;  // this wave's k-slice block
  const float gs = g.gscale;

  if (threadIdx.x < 16) sbest[threadIdx.x] = 0ull;

  // RING: the row this lane moves for each row group (rows >= M repeat
  // row M - 1; their outputs are dropped), plus its swizzled chunk
  const uint16_t* ar[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    ar[j] = RING ? g.a + static_cast<size_t>(min(4 * j + static_cast<int>((threadIdx.x & 63) >> 4), M - 1)) * g.K +
                       ring_chunk(j)
                 : nullptr;
  auto group = [&](int gi, GroupPtrs<P>& gp) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      int panel = p0 + (pw + gi * PWv) * P + p;
      panel = panel < kp.npanels ? panel : kp.npanels - 1;  // in-bounds load, result dropped
      gp.panel[p] = g.w + static_cast<size_t>(panel) * static_cast<size_t>(g.panel_bytes);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) gp.ar[j] = ar[j];
  };
  const StageGeom sg = stage_geom(g.a, M, g.K, kt0, KRg);
  auto pre_issue = [&]() {
    if constexpr (!RING) stage_issue(sg, lds);
  };
  auto pre = [&]() {
    if constexpr (!RING) stage_wait<D * P * 2>();  // D tiles of P panels: codes + scales
  };
  auto col_of = [&](int gi) { return (pw + gi * PWv) * P * 16; };  // block-local first column
  // sampling with final per-group results (one k-range, one k-split wave, no
  // half tile added later): each lane ranks its 4 rows x P columns as soon as
  // the group is done, during the stream, with one generator call per column
  const bool keys_in_stream = SAMPLE && g.argmax && KS == 1 && KW == 1 && kp.half_t < 0;
  unsigned long long skey[4] = {0ull, 0ull, 0ull, 0ull};  // rows 4 (lane >> 4) + r
  auto epi = [&](int gi, f32x4 (&acc)[P][2]) {
    stash_rows<P, false>(wres, rs, col_of(gi), M, acc);
    if (SAMPLE && keys_in_stream) {
      const int lane = threadIdx.x & 63, o = lane >> 4, c = lane & 15;
      const int pan0 = p0 + (pw + gi * PWv) * P;
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const f32x4 v = acc[p][0] + acc[p][1];  // the value the epilogue reads back
        const int n = (pan0 + p) * 16 + c;
        const f32x4 gn = gumbel4(g, n, o);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if (pan0 + p < pend && 4 * o + r < M) {
            const unsigned long long kk = sample_key(g, gs * v[r], gn[r], n);
            skey[r] = kk > skey[r] ? kk : skey[r];
          }
        }
      }
    }
  };
  auto epi_add = [&](int gi, f32x4 (&acc)[P][2]) { stash_rows<P, true>(wres, rs, col_of(gi), M, acc); };
  const ALds al = alds_view(reinterpret_cast<const char*>(lds), KRg, M, wt0);
  const ARing rg = aring_view(lds_offset(lds) + static_cast<unsigned>(w * D * kRingSlot));
  // a wave without tiles streams an empty range placed at the last packed
  // tile, so that its prologue's loads (never computed) stay in the matrix
  const int wk0 = wtn > 0 ? kt0 + wt0 : kp.ntiles - 1;
  stream_groups<FMT, P, D, RING ? kARing : kAStaged>(ng, wtn, wk0, kp.half_t, al, rg, g.K, group, pre_issue, pre, epi,
                                                    epi_add);
  if (wtn == 0) {  // a k-split wave without tiles still owns zero partials
    f32x4 z[P][2];
#pragma unroll
    for (int p = 0; p < P; ++p) z[p][0] = z[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int gi = 0; gi < ng; ++gi) stash_rows<P, false>(wres, rs, col_of(gi), M, z);
  }
  __syncthreads();
  if (SAMPLE && keys_in_stream) {
    const int o = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (skey[r] != 0ull) atomicMax(&sbest[4 * o + r], skey[r]);
  }

  // Epilogue over the block's outputs, row-major in 4-column groups: every
  // thread sums the KW k-slices of its group, then stores 4 outputs (or 4
  // partials) in one vector store, so a wave writes 64 consecutive groups.
  const int nc4 = (pend - p0) * 4;  // 4-column groups per row
  // row of item q: q / nc4 by a multiply with ceil(2^32 / nc4) (exact while
  // q nc4 < 2^32, which the launch checks)
  const unsigned row_magic = pb == kp.nblocks - 1 ? kp.nc4_magic_last : kp.nc4_magic;
  auto item_row = [&](int q) { return static_cast<int>(__umulhi(static_cast<unsigned>(q), row_magic)); };
  // sampling: store the softcapped logits (if wanted) and, unless the keys
  // were taken in the stream, rank the 4 columns (one generator call each,
  // word m % 4)
  auto finish_sample = [&](int m, int n, size_t off, f32x4 y, bool with_keys, unsigned long long& key) {
    f32x4 z = y;
    if (g.softcap > 0.f) {
#pragma unroll
      for (int j = 0; j < 4; ++j) z[j] = softcap_of(y[j], g.softcap);
    }
    if (g.out) (void)store_out4(g.out, g.out_dtype, off, z);
    if (with_keys && g.argmax) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float noise = gumbel4(g, n + j, m >> 2)[m & 3];
        const unsigned long long kj = sample_key(g, y[j], noise, n + j);
        key = kj > key ? kj : key;
      }
    }
  };
  const int items = (SAMPLE && !g.out && keys_in_stream) ? 0 : M * nc4;
  const bool wave_rows = (nc4 & 63) == 0;  // each wave-wide batch of items lies in one row
  for (int q0 = 0; q0 < items; q0 += 64 * W) {
    const int q = q0 + static_cast<int>(threadIdx.x);
    unsigned long long key = 0ull;
    int m = 0;
    if (q < items) {
      m = item_row(q);
      const int c4 = q - m * nc4;
      const float* rp = res + m * rs + c4 * 4;
      f32x4 v = *reinterpret_cast<const f32x4*>(rp);
      for (int j = 1; j < KW; ++j) v += *reinterpret_cast<const f32x4*>(rp + static_cast<size_t>(j) * M * rs);
      const int n = p0 * 16 + c4 * 4;
      const size_t off = static_cast<size_t>(m) * g.N + n;
      if (KS == 1) {
        if constexpr (SAMPLE) {
          finish_sample(m, n, off, gs * v, !keys_in_stream, key);
        } else {
          const f32x4 y = store_out4(g.out, g.out_dtype, off, gs * v);
          if (g.argmax) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const unsigned long long kj = argmax_key(y[j], n + j);
              key = kj > key ? kj : key;
            }
          }
        }
      } else {
        store_coherent4(kp.partial + static_cast<size_t>(ks) * M * g.N + off, v);
      }
    }
    if (KS == 1 && g.argmax) {
      if (wave_rows) {  // uniform row per wave: one LDS atomic per wave
        key = max_key_64(key);
        if ((threadIdx.x & 63) == 0 && key != 0ull) atomicMax(&sbest[m], key);
      } else if (key != 0ull) {
        atomicMax(&sbest[m], key);
      }
    }
  }

  bool final_wg = true;  // does this workgroup hold final values of its block?
  if (KS > 1) {
    wait_stores();  // this wave's partials are at the coherence point
    __syncthreads();
    if (threadIdx.x == 0) s_last = count_arrival(kp.bcnt + pb) == static_cast<unsigned>(KS - 1);
    __syncthreads();
    final_wg = s_last != 0;
    if (final_wg) {
      // all KS partials of a 4-column group are loaded together, then summed in ks order
      for (int q = threadIdx.x; q < items; q += 64 * W) {
        const int m = item_row(q);
        const int n = p0 * 16 + (q - m * nc4) * 4;
        const size_t off = static_cast<size_t>(m) * g.N + n;
        f32x4 v[kMaxKS];
#pragma unroll
        for (int j = 0; j < kMaxKS; ++j)
          v[j] = j < KS ? load_coherent4(kp.partial + static_cast<size_t>(j) * M * g.N + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 sacc = v[0];
#pragma unroll
        for (int j = 1; j < kMaxKS; ++j) sacc += v[j];
        unsigned long long key = 0ull;
        if constexpr (SAMPLE) {
          finish_sample(m, n, off, gs * sacc, true, key);
        } else {
          const f32x4 y = store_out4(g.out, g.out_dtype, off, gs * sacc);
          if (g.argmax) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const unsigned long long kj = argmax_key(y[j], n + j);
              key = kj > key ? kj : key;
            }
          }
        }
        if (g.argmax && key) atomicMax(&sbest[m], key);
      }
      if (threadIdx.x == 0) atomicExch(kp.bcnt + pb, 0u);
    }
  }

  if (g.argmax && final_wg) {
    __syncthreads();
    if (threadIdx.x < 16 && static_cast<int>(threadIdx.x) < M && sbest[threadIdx.x] != 0ull)
      atomicMax(g.keys + threadIdx.x, sbest[threadIdx.x]);
    wait_stores();  // the key atomics have been performed
    __syncthreads();
    if (threadIdx.x == 0) s_last = count_arrival(g.counter) == static_cast<unsigned>(kp.nblocks - 1);
    __syncthreads();
    if (s_last) {
      // the last workgroup: one thread per row reads (and clears) its key
      // with an atomic, which acts at the coherence point; all rows at once
      if (static_cast<int>(threadIdx.x) < M) {
        const unsigned long long k = atomicExch(g.keys + threadIdx.x, 0ull);
        g.argmax[threadIdx.x] = k == 0ull ? -1 : static_cast<int>(0xFFFFFFFFu - static_cast<unsigned>(k & 0xFFFFFFFFull));
      }
      if (threadIdx.x == 0) atomicExch(g.counter, 0u);
    }
  }
}

// ---- test export: the sampling noise's uniforms -------------------------------
__global__ __launch_bounds__(256) void sample_uniforms_kernel(GemmArgs g, int M, int N, float* __restrict__ out) {
  const int n = blockIdx.x * 256 + threadIdx.x, q = blockIdx.y;  // rows 4 q .. 4 q + 3
  if (n >= N) return;
  const u32x4 x = philox4x32_10(u32x4{static_cast<unsigned>(n), static_cast<unsigned>(q), g.offset, 0u}, g.seed_lo,
                                g.seed_hi);
  const unsigned w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
  for (int r = 0; r < 4; ++r)
    if (4 * q + r < M) out[static_cast<size_t>(4 * q + r) * N + n] = uniform_of(w[r]);
}

// ---- test export: write out the dequantized weights -----------------------
template <int FMT>
__global__ __launch_bounds__(64) void dequant_kernel(const uint8_t* __restrict__ w, int64_t pb, int nfull, int half,
                                                     int K, int npanels, float gsc, float* __restrict__ out) {
  const int lane = threadIdx.x;
  const int o = lane >> 4, c = lane & 15;
  const int ntiles = nfull + half;
  const int p = blockIdx.x / ntiles, t = blockIdx.x % ntiles;
  if (p >= npanels) return;
  const bool is_half = t == nfull;
  const int steps = is_half ? 2 : 4;
  const uint8_t* tb = w + static_cast<size_t>(p) * pb + static_cast<size_t>(t) * kTileBytes;
  unsigned cw[4] = {0u, 0u, 0u, 0u};
  if (is_half) {
    const u32x2 cc = ld_nt8(tb + lane * 8);
    cw[0] = cc.x;
    cw[1] = cc.y;
  } else {
    const u32x4 cc = ld_nt16(tb + lane * 16);
    cw[0] = cc.x; cw[1] = cc.y; cw[2] = cc.z; cw[3] = cc.w;
  }
  const int n = p * 16 + c;
  const int kb = t * kTileK;
  if constexpr (FMT == kNvfp4) {
    const unsigned sw = is_half ? ld_nt2(tb + kHalfCodeBytes + (c * 2 + (lane >> 5)) * 2)
                                : ld_nt4(tb + kTileCodeBytes + (c * 2 + (lane >> 5)) * 4);
    const f16x2 s01 = e4m3_pair(sw, false), s23 = e4m3_pair(sw, true);
    for (int i = 0; i < steps; ++i) {
      const f16 s = i == 0 ? s01[0] : i == 1 ? s01[1] : i == 2 ? s23[0] : s23[1];
      const f16x8 v = nvfp4_operand(cw[i], s);
      for (int j = 0; j < 8; ++j) {
        const int k = kb + 32 * i + 8 * o + j;
        if (k < K) out[static_cast<size_t>(n) * K + k] = (float)v[j] * gsc;
      }
    }
  } else {
    const u32x2 sb = is_half ? u32x2{ld_nt4(tb + kHalfCodeBytes + c * 4), 0u} : ld_nt8(tb + kTileCodeBytes + c * 8);
    for (int i = 0; i < steps; ++i) {
      const unsigned wsb = (i < 2) ? sb.x : sb.y;
      const float s = bf16_lo(wsb), b = bf16_hi(wsb);
      const bf16x8 v = affine_operand(cw[i], 0x000F000Fu, 0x43004300u);
      for (int j = 0; j < 8; ++j) {
        const int k = kb + 32 * i + 8 * o + j;
        const float q = (float)v[j] - 128.0f;  // exact: 128 + q is exact in bf16
        if (k < K) out[static_cast<size_t>(n) * K + k] = fmaf(q, s, b);
      }
    }
  }
}


template <int FMT, int P, int W, int D, bool RING, bool SAMPLE>
int launch_cfg(const GemmParams& kp, hipStream_t s) {
  const size_t lds = gemm_lds_bytes(kp.g.M, kp.KR, kp.KW, kp.PB, RING, W, D);
  if (int e = ensure_dynamic_lds(reinterpret_cast<const void*>(&qgemm_kernel<FMT, P, W, D, RING, SAMPLE>), lds))
    return e;
  hipLaunchKernelGGL((qgemm_kernel<FMT, P, W, D, RING, SAMPLE>), dim3(kp.nblocks * kp.KS), dim3(64 * W), lds, s, kp);
  return static_cast<int>(hipGetLastError());
}

template <int FMT, bool SAMPLE>
int launch_fmt(const GemmParams& kp, const GemmCfg& cfg, hipStream_t s) {
#define Q4_CFG(P_, W_, D_) \
  if (cfg.P == P_ && cfg.W == W_ && cfg.D == D_)              \
    return cfg.RING ? launch_cfg<FMT, P_, W_, D_, true, SAMPLE>(kp, s) : launch_cfg<FMT, P_, W_, D_, false, SAMPLE>(kp, s);
  Q4_CFG(1, 4, 4)
  Q4_CFG(2, 4, 4)
  Q4_CFG(2, 8, 2)
  Q4_CFG(2, 8, 4)
  Q4_CFG(4, 4, 4)
  Q4_CFG(4, 8, 4)
  Q4_CFG(2, 4, 8)
  Q4_CFG(2, 8, 8)
  Q4_CFG(4, 4, 6)
#undef Q4_CFG
  return static_cast<int>(hipErrorInvalidConfiguration);
}

}  // namespace

GemmCfg choose_gemm_cfg(int fmt, int M, int64_t K, int64_t N) {
  (void)fmt;
  const int npanels = static_cast<int>(N / 16);
  const int ntiles = static_cast<int>(full_tiles(K) + (has_half_tile(K) ? 1 : 0));
  GemmCfg c{};
  const bool ring_ok = K % 64 == 0;  // full tiles lie below K: unconditional activation loads
  if (const char* e = std::getenv("Q4MI_GEMM_CFG")) {  // "P,W,D,KS,KW,PB[,RING]" for A/B measurements
    const int nf = std::sscanf(e, "%d,%d,%d,%d,%d,%d,%d", &c.P, &c.W, &c.D, &c.KS, &c.KW, &c.PB, &c.RING);
    if (nf >= 6) {
      c.KS = c.KS < 1 ? 1 : (c.KS > ntiles ? ntiles : (c.KS > kMaxKS ? kMaxKS : c.KS));
      c.KW = (c.KW >= 1 && c.W % c.KW == 0) ? c.KW : 1;
      c.RING = (nf == 7 && c.RING && ring_ok) ? 1 : 0;
      return c;
    }
  }
  // About one workgroup per CU: blocks * KS ~ 256.  Inside a workgroup, KW
  // waves split the k-range when a block has fewer panel groups than waves.
  // If all W waves then split the k-range of a single group, no two waves
  // share activations and, for M > 8 (the ring always moves 16 rows), each
  // wave moves its own (RING: no workgroup-wide stage, no k-split);
  // otherwise KS (k-ranges reduced across workgroups) grows only as far as
  // needed for the staged activations to fit in LDS.
  c.P = 2;
  c.W = 8;
  // tiles in flight per wave: more is not better here; measured on one
  // MI355X, 2 (37 KB per CU) beats 4 for the 44 MB affine matrices and 4
  // beats 8 for the 415 MB lm_head; the ring below uses 4
  c.D = npanels >= 4096 ? 4 : 2;
  // a small matrix (at most one panel per CU) with few rows: one panel per
  // workgroup of 4 waves, twice the workgroups of the 2-panel blocks
  // (measured at M = 1, K = N = 1024: 3.67 us against 4.01)
  if (npanels <= 256 && M <= 8) {
    c.P = 1;
    c.W = 4;
    c.D = 4;
  }
  auto shape = [&](int KS) {
    GemmCfg x = c;
    x.KS = KS;
    int PB = static_cast<int>((static_cast<int64_t>(npanels) * KS + 255) / 256);
    PB = (PB + x.P - 1) / x.P * x.P;
    if (PB >= x.P * x.W) {
      x.KW = 1;
      x.PB = PB;
    } else {
      x.KW = x.W;
      while (x.KW > 1 && x.P * (x.W / x.KW) < PB) x.KW /= 2;
      x.PB = x.P * (x.W / x.KW);
    }
    return x;
  };
  auto fits = [&](const GemmCfg& x) {
    const int KR = (ntiles + x.KS - 1) / x.KS;
    return gemm_lds_bytes(M, KR, x.KW, x.PB, false, x.W, x.D) <= kGemmLdsMax;
  };
  int KS = 1;
  c = shape(KS);
  c.RING = 0;
  if (ring_ok && M > 8 && c.KW == c.W && c.PB == c.P &&
      gemm_lds_bytes(M, ntiles, c.KW, c.PB, true, c.W, 4) <= kGemmLdsMax) {
    c.RING = 1;
    c.D = 4;
    return c;
  }
  while (!fits(c) && KS < kMaxKS && KS < ntiles) c = shape(++KS);
  if (c.KS > kMaxKS) c.KS = kMaxKS;
  if (c.KS > ntiles) c.KS = ntiles;
  if (c.KS > 1 && (npanels + c.PB - 1) / c.PB > kMaxSplitBlocks) c.KS = 1;
  return c;
}

// k-split actually launched: cfg.KS, less any k-range that would be empty
static int launch_ks(const GemmCfg& c, int ntiles) {
  const int KS = c.KS < 1 ? 1 : c.KS;
  const int KR = (ntiles + KS - 1) / KS;
  return (ntiles + KR - 1) / KR;
}

size_t gemm_workspace(int fmt, int M, int64_t K, int64_t N) {
  const GemmCfg c = choose_gemm_cfg(fmt, M, K, N);
  const int ntiles = static_cast<int>(full_tiles(K) + (has_half_tile(K) ? 1 : 0));
  const int KS = launch_ks(c, ntiles);
  size_t bytes = kWsCounterBytes;
  if (KS > 1) bytes += static_cast<size_t>(KS) * M * N * 4;
  return bytes;
}

int launch_gemm(int fmt, const GemmArgs& g, const GemmCfg& cfg, void* ws, void* stream) {
  GemmParams kp{};
  kp.g = g;
  kp.npanels = g.N / 16;
  kp.ntiles = g.nfull + g.half;
  kp.half_t = g.half ? g.nfull : -1;
  kp.KS = launch_ks(cfg, kp.ntiles);
  kp.KR = (kp.ntiles + kp.KS - 1) / kp.KS;
  kp.KW = cfg.KW;
  if (cfg.P < 1 || cfg.PB < 1) return static_cast<int>(hipErrorInvalidConfiguration);
  kp.PB = (cfg.PB + cfg.P - 1) / cfg.P * cfg.P;  // whole groups: every stashed column has a slot
  kp.nblocks = (kp.npanels + kp.PB - 1) / kp.PB;
  kp.rs = kp.PB * 16 + 4;
  kp.nc4_magic = static_cast<unsigned>(((1ull << 32) + kp.PB * 4 - 1) / (kp.PB * 4));
  const int last_nc4 = (kp.npanels - (kp.nblocks - 1) * kp.PB) * 4;
  kp.nc4_magic_last = static_cast<unsigned>(((1ull << 32) + last_nc4 - 1) / last_nc4);
  kp.ks_magic = static_cast<unsigned>(((1ull << 32) + kp.KS - 1) / kp.KS);
  kp.kw_shift = 0;
  while ((1 << kp.kw_shift) < cfg.KW) ++kp.kw_shift;
  if (cfg.RING && g.K % 64 != 0) return static_cast<int>(hipErrorInvalidConfiguration);
  kp.res_off = static_cast<int>(gemm_res_offset(g.M, kp.KR, cfg.RING != 0, cfg.W, cfg.D));
  if (kp.KS > kMaxKS) return static_cast<int>(hipErrorInvalidConfiguration);
  if (kp.KW < 1 || cfg.W % kp.KW != 0 || (1 << kp.kw_shift) != kp.KW || kp.PB < 1)
    return static_cast<int>(hipErrorInvalidConfiguration);
  // the magics give exact quotients while dividend * divisor < 2^32
  if (static_cast<int64_t>(g.M) * kp.PB * 4 * (kp.PB * 4) >= (1ll << 32) ||
      static_cast<int64_t>(kp.nblocks) * kp.KS * kp.KS >= (1ll << 32))
    return static_cast<int>(hipErrorInvalidConfiguration);
  if (kp.KS > 1) {
    if (kp.nblocks > kMaxSplitBlocks) return static_cast<int>(hipErrorInvalidConfiguration);
    kp.bcnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kWsBlockCounters);
    kp.partial = reinterpret_cast<float*>(static_cast<char*>(ws) + kWsCounterBytes);
  }
  if (gemm_lds_bytes(g.M, kp.KR, kp.KW, kp.PB, cfg.RING != 0, cfg.W, cfg.D) > kGemmLdsMax)
    return static_cast<int>(hipErrorInvalidConfiguration);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt != kNvfp4) return g.sample ? static_cast<int>(hipErrorInvalidConfiguration) : launch_fmt<kAffine, false>(kp, cfg, s);
  return g.sample ? launch_fmt<kNvfp4, true>(kp, cfg, s) : launch_fmt<kNvfp4, false>(kp, cfg, s);
}

int launch_sample_uniforms(unsigned seed_lo, unsigned seed_hi, unsigned offset, int M, int64_t N, float* out,
                           void* stream) {
  GemmArgs g{};
  g.seed_lo = seed_lo;
  g.seed_hi = seed_hi;
  g.offset = offset;
  hipLaunchKernelGGL(sample_uniforms_kernel, dim3(static_cast<unsigned>((N + 255) / 256), (M + 3) / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), g, M, static_cast<int>(N), out);
  return static_cast<int>(hipGetLastError());
}

int launch_dequant(int fmt, const uint8_t* w, int64_t pb, int64_t N, int64_t K, float gsc, float* out,
                   void* stream) {
  const int nfull = static_cast<int>(full_tiles(K));
  const int half = has_half_tile(K) ? 1 : 0;
  const int npanels = static_cast<int>(N / 16);
  const dim3 grid(static_cast<unsigned>(npanels * (nfull + half)));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (fmt == kNvfp4)
    hipLaunchKernelGGL(dequant_kernel<kNvfp4>, grid, dim3(64), 0, s, w, pb, nfull, half, static_cast<int>(K), npanels,
                       gsc, out);
  else
    hipLaunchKernelGGL(dequant_kernel<kAffine>, grid, dim3(64), 0, s, w, pb, nfull, half, static_cast<int>(K), npanels,
                       gsc, out);
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
