// W4A16 skinny GEMM kernels for gfx950 (MI355X): NVFP4 and MLX-style affine 4-bit.
//
// y[m][n] = sum_k a[m][k] w[n][k] for M <= 16 activation rows.  [gemma-cuda-hybrid
// README, "Everything it has": one tensor-core GEMM for every M <= 16 product,
// FP4 -> f16 dequant in registers from an offline-repacked layout, 16-byte
// loads that do not pollute the cache; TensorFold issue "Proposal: Gemma 4 on
// CUDA", "Why now": qlinear's affine 4-bit path with 64-value group sums.]
//
// Design (gfx950):
//  * One wave owns P panels of 16 output columns and a contiguous range of
//    128-k tiles; KW waves of a workgroup split K and reduce through LDS in a
//    fixed order; PW independent wave groups share a workgroup.
//  * Per tile each lane issues one 16-byte non-temporal load of codes per
//    panel (1 KiB contiguous per wave) plus one small scale load, and four
//    16-byte loads of activations (L2-resident, shared by the P panels).
//  * Loads run D tiles ahead of the math (register ring).
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

struct KParams {
  GemmArgs g;
  int nmain;      // full tiles needing no k bound check
  int tail;       // 0 none, 1 half tile, 2 full tile crossing K
  int npanels;
};

template <int FMT, int P, int KW, int PW, int D>
__global__ __launch_bounds__(64 * KW * PW) void qgemm_kernel(KParams kp) {
  const GemmArgs& g = kp.g;
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int kw = wid % KW;
  const int pw = wid / KW;
  const int o = lane >> 4;
  const int c = lane & 15;

  const int panel0 = (blockIdx.x * PW + pw) * P;
  const uint8_t* pbase[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    int pi = panel0 + p;
    pi = pi < kp.npanels ? pi : kp.npanels - 1;  // clamp: loads stay in bounds, stores are skipped
    pbase[p] = g.w + static_cast<size_t>(pi) * static_cast<size_t>(g.panel_bytes);
  }
  const bool arow_ok = c < g.M;
  const uint16_t* arow = g.a + static_cast<size_t>(arow_ok ? c : 0) * static_cast<size_t>(g.K);

  // this wave's tiles: [t0, t1) of the checked-free range
  const int per = (kp.nmain + KW - 1) / KW;
  const int t0 = kw * per;
  const int t1 = min(kp.nmain, t0 + per);
  const int nt = t1 > t0 ? t1 - t0 : 0;

  f32x4 acc[P][2];
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  dev::wave_accumulate<FMT, P, D>(acc, pbase, arow, arow_ok, g.K, t0, nt,
                                  kw == KW - 1 ? kp.tail : 0, kp.nmain);

  f32x4 res[P];
#pragma unroll
  for (int p = 0; p < P; ++p) res[p] = acc[p][0] + acc[p][1];

  const int M = g.M;
  const float gs = g.gscale;
  unsigned long long best[4] = {0ull, 0ull, 0ull, 0ull};  // argmax keys for rows 4o + r

  if constexpr (KW == 1) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int pi = panel0 + p;
      if (pi >= kp.npanels) continue;
      const int n = pi * 16 + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * o + r;
        if (m < M) {
          const float v = store_out(g.out, g.out_dtype, static_cast<size_t>(m) * g.N + n, gs * res[p][r]);
          const unsigned long long key = argmax_key(v, n);
          best[r] = key > best[r] ? key : best[r];
        }
      }
    }
  } else {
    __shared__ float red[KW][PW][P][4][64];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[kw][pw][p][r][lane] = res[p][r];
    __syncthreads();
    // the P x 4 (panel, accumulator row) items of the group are shared out
    // over its KW waves; each item is summed over the KW partials in order
#pragma unroll
    for (int pp = 0; pp < P; ++pp)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if ((pp * 4 + r) % KW != kw) continue;
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < KW; ++j) s += red[j][pw][pp][r][lane];
        const int pi = panel0 + pp;
        const int m = 4 * o + r;
        if (pi < kp.npanels && m < M) {
          const int n = pi * 16 + c;
          const float v = store_out(g.out, g.out_dtype, static_cast<size_t>(m) * g.N + n, gs * s);
          const unsigned long long key = argmax_key(v, n);
          best[r] = key > best[r] ? key : best[r];
        }
      }
  }

  if (g.argmax) {
    __shared__ unsigned long long sbest[16];
    if (threadIdx.x < 16) sbest[threadIdx.x] = 0ull;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const unsigned long long k = max_key_16(best[r]);
      if (c == 0 && k != 0ull) atomicMax(&sbest[4 * o + r], k);
    }
    __syncthreads();
    if (threadIdx.x < 16 && static_cast<int>(threadIdx.x) < M && sbest[threadIdx.x] != 0ull)
      atomicMax(g.keys + threadIdx.x, sbest[threadIdx.x]);
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const unsigned prev = atomicAdd(g.counter, 1u);
      if (prev == gridDim.x - 1) {
        __threadfence();
        for (int m = 0; m < M; ++m) {
          const unsigned long long k = atomicExch(g.keys + m, 0ull);
          g.argmax[m] = k == 0ull ? -1 : static_cast<int>(0xFFFFFFFFu - static_cast<unsigned>(k & 0xFFFFFFFFull));
        }
        atomicExch(g.counter, 0u);
      }
    }
  }
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
      const bf16x8 v = affine_operand(cw[i]);
      for (int j = 0; j < 8; ++j) {
        const int k = kb + 32 * i + 8 * o + j;
        const float q = (float)v[j] - 128.0f;  // exact: 128 + q is exact in bf16
        if (k < K) out[static_cast<size_t>(n) * K + k] = fmaf(q, s, b);
      }
    }
  }
}

template <int FMT, int P, int KW, int PW, int D>
int launch_cfg(const KParams& kp, hipStream_t s) {
  const int nwg = (kp.npanels + P * PW - 1) / (P * PW);
  hipLaunchKernelGGL((qgemm_kernel<FMT, P, KW, PW, D>), dim3(nwg), dim3(64 * KW * PW), 0, s, kp);
  return static_cast<int>(hipGetLastError());
}

template <int FMT>
int launch_fmt(const KParams& kp, const GemmCfg& cfg, hipStream_t s) {
#define Q4_CFG(P_, KW_, PW_, D_) \
  if (cfg.P == P_ && cfg.KW == KW_ && cfg.PW == PW_) return launch_cfg<FMT, P_, KW_, PW_, D_>(kp, s);
  Q4_CFG(1, 8, 1, 4)
  Q4_CFG(1, 4, 1, 4)
  Q4_CFG(2, 8, 1, 4)
  Q4_CFG(2, 4, 1, 4)
  Q4_CFG(2, 2, 1, 4)
  Q4_CFG(2, 1, 4, 4)
  Q4_CFG(4, 1, 4, 3)
  Q4_CFG(4, 2, 1, 3)
  Q4_CFG(4, 1, 2, 3)
#undef Q4_CFG
  return static_cast<int>(hipErrorInvalidConfiguration);
}

}  // namespace

GemmCfg choose_gemm_cfg(int fmt, int M, int64_t K, int64_t N) {
  (void)fmt;
  (void)M;
  if (const char* e = std::getenv("Q4MI_GEMM_CFG")) {  // "P,KW,PW" for A/B measurements
    GemmCfg c{};
    if (std::sscanf(e, "%d,%d,%d", &c.P, &c.KW, &c.PW) == 3) return c;
  }
  const int64_t npanels = N / 16;
  const int64_t ntiles = (K + kTileK - 1) / kTileK;
  if (npanels >= 8192) return {4, 1, 4};
  if (npanels >= 2048) return {2, 1, 4};
  if (npanels < 256 && ntiles >= 4) return {1, 8, 1};
  if (ntiles >= 16) return {2, 8, 1};
  if (ntiles >= 8) return {2, 4, 1};
  return {2, 2, 1};
}

int launch_gemm(int fmt, const GemmArgs& g, const GemmCfg& cfg, void* stream) {
  KParams kp{};
  kp.g = g;
  kp.npanels = g.N / 16;
  // tiles entirely inside K need no bound checks; the last one may not be
  const int full_in = g.K / kTileK;
  if (g.half) {
    kp.nmain = g.nfull;
    kp.tail = 1;
  } else if (full_in < g.nfull) {
    kp.nmain = full_in;
    kp.tail = 2;
  } else {
    kp.nmain = g.nfull;
    kp.tail = 0;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  return fmt == kNvfp4 ? launch_fmt<kNvfp4>(kp, cfg, s) : launch_fmt<kAffine>(kp, cfg, s);
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
