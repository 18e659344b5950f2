// NVFP4 W4A16 GEMM for more than 16 activation rows (prefill chunks and
// large verify blocks): y[M][N] = g * a[M][K] . W[N][K]^T.
//
// [README] "Everything it has" / "Why it's fast": the FP4 weight GEMM of the
// forward pass; with many rows the product is bound by the matrix cores, not
// by the weight stream, so this kernel reuses each dequantized weight
// fragment across 64 activation rows and each activation fragment across 64
// weight rows.
//
// A workgroup of 4 waves computes a 128 x 128 output block, the waves as
// 2 x 2: wave (wm, wn) owns rows 64 wm .. 64 wm + 63 and the 4 panels
// 4 wn .. 4 wn + 3 of the block (16 accumulators of 16 x 16).  Per 128-k
// tile the workgroup stages the block's 128 activation rows in LDS (double
// buffered, 16-byte chunks XOR-swizzled by row so the fragment reads are
// conflict-free) and every wave loads its 4 panels' packed tiles straight
// into registers (the next tile's loads in flight during this tile's math),
// dequantizes each 8-code step once and feeds it to 4 MFMAs.
#include <hip/hip_runtime.h>

#include "q4mi_tiles.h"

namespace q4mi {
using namespace dev;
namespace {

constexpr int kPfBM = 128, kPfBN = 128;  // rows x columns per workgroup
constexpr int kPfMT = 4, kPfNP = 4;       // 16-row m-tiles and panels per wave

// one panel's packed tile for one lane: 4 code dwords (full tile; 2 for a
// half tile) and the scale bytes of its groups
struct WTile {
  u32x4 c[kPfNP];
  unsigned s[kPfNP];
};

template <bool HALF>
__device__ __forceinline__ void load_wtile(WTile& t, const uint8_t* const (&pp)[kPfNP], const bool (&pv)[kPfNP],
                                           int64_t off, int lane) {
  const int c = lane & 15, h = (lane >> 5) & 1;
#pragma unroll
  for (int p = 0; p < kPfNP; ++p) {
    if (!pv[p]) {
      t.c[p] = u32x4{0u, 0u, 0u, 0u};
      t.s[p] = 0u;
      continue;
    }
    const uint8_t* b = pp[p] + off;
    if constexpr (HALF) {
      const u32x2 v = ld_nt8(b + lane * 8);
      t.c[p] = u32x4{v.x, v.y, 0u, 0u};
      t.s[p] = ld_nt2(b + kHalfCodeBytes + (c * 2 + h) * 2);
    } else {
      t.c[p] = ld_nt16(b + lane * 16);
      t.s[p] = ld_nt4(b + kTileCodeBytes + (c * 2 + h) * 4);
    }
  }
}

// activation block in LDS: row r (0..127) of 128 k as 16 chunks of 8 f16,
// chunk q stored at position q ^ (r & 15)
struct ABlock {
  u32x4 v[kPfBM][16];
};

// thread t moves chunks t + 256 j (row (t + 256 j) / 16, chunk t % 16)
__device__ __forceinline__ void fetch_a(u32x4 (&r)[8], const uint16_t* __restrict__ a, int M, int K, int m0, int k0) {
  const int q = threadIdx.x & 15;
  const int kk = k0 + 8 * q;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (threadIdx.x >> 4) + 16 * j;
    const int m = m0 + row;
    if (m < M && kk < K)  // K % 16 == 0: a chunk of 8 is all inside or all beyond
      r[j] = *reinterpret_cast<const u32x4*>(a + static_cast<int64_t>(m) * K + kk);
    else
      r[j] = u32x4{0u, 0u, 0u, 0u};
  }
}
__device__ __forceinline__ void put_a(ABlock& A, const u32x4 (&r)[8]) {
  const int q = threadIdx.x & 15;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int row = (threadIdx.x >> 4) + 16 * j;
    A.v[row][q ^ (row & 15)] = r[j];
  }
}

template <int STEPS>
__device__ __forceinline__ void tile_mma(f32x4 (&acc)[kPfMT][kPfNP], const ABlock& A, const WTile& w, int wm,
                                         int lane) {
  const int c = lane & 15, o = lane >> 4;
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    f16x8 b[kPfNP];
#pragma unroll
    for (int p = 0; p < kPfNP; ++p) b[p] = nvfp4_operand(w.c[p][i], e4m3_pair(w.s[p], i >= 2)[i & 1]);
#pragma unroll
    for (int mt = 0; mt < kPfMT; ++mt) {
      const int row = wm * 64 + mt * 16 + c;
      const u32x4 af = A.v[row][(4 * i + o) ^ c];
#pragma unroll
      for (int p = 0; p < kPfNP; ++p) acc[mt][p] = mfma_f16(af, b[p], acc[mt][p]);
    }
  }
}

// Workgroups are dealt so that the 8 XCDs (blockIdx.x % 8) each take a
// contiguous range of column blocks, row blocks fastest: the workgroups that
// share a column block's weights run on one XCD and read them through its L2.
__global__ __launch_bounds__(256) void qgemm_prefill_kernel(const uint8_t* __restrict__ w, int64_t pb, float gscale,
                                                            const uint16_t* __restrict__ a, int M, int K, int N,
                                                            void* __restrict__ out, int out_dtype, int nfull, int half,
                                                            int mblocks, int nblocks) {
  __shared__ ABlock As[2];
  const int nwg = mblocks * nblocks;
  const int b = blockIdx.x;
  // XCD-major order: the grid is padded to a multiple of 8, idle slots return
  const int per_xcd = (nwg + 7) / 8;
  const int item = (b & 7) * per_xcd + (b >> 3);
  if (item >= nwg) return;
  const int mb = item % mblocks, nb = item / mblocks;
  const int m0 = mb * kPfBM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int npanels = N / 16;
  const uint8_t* pp[kPfNP];
  bool pv[kPfNP];
#pragma unroll
  for (int p = 0; p < kPfNP; ++p) {
    const int pn = nb * (kPfBN / 16) + wn * kPfNP + p;
    pv[p] = pn < npanels;
    pp[p] = w + static_cast<int64_t>(pv[p] ? pn : 0) * pb;
  }
  f32x4 acc[kPfMT][kPfNP];
#pragma unroll
  for (int mt = 0; mt < kPfMT; ++mt)
#pragma unroll
    for (int p = 0; p < kPfNP; ++p) acc[mt][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = nfull + half;
  u32x4 ra[8];
  WTile wc, wnx;
  fetch_a(ra, a, M, K, m0, 0);
  if (nfull > 0)
    load_wtile<false>(wc, pp, pv, 0, lane);
  else
    load_wtile<true>(wc, pp, pv, 0, lane);
  put_a(As[0], ra);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1;
    const bool more = t + 1 < ntiles;
    if (more) {  // the next tile's activations and weights, in flight during this tile's math
      fetch_a(ra, a, M, K, m0, (t + 1) * kTileK);
      if (t + 1 < nfull)
        load_wtile<false>(wnx, pp, pv, static_cast<int64_t>(t + 1) * kTileBytes, lane);
      else
        load_wtile<true>(wnx, pp, pv, static_cast<int64_t>(t + 1) * kTileBytes, lane);
    }
    if (t < nfull)
      tile_mma<4>(acc, As[cur], wc, wm, lane);
    else
      tile_mma<2>(acc, As[cur], wc, wm, lane);
    if (more) put_a(As[cur ^ 1], ra);  // that buffer's last readers passed the previous barrier
    __syncthreads();
    wc = wnx;
  }

  // lane (c, o) holds rows 4 o + r of column c of each 16 x 16 accumulator
  const int c = lane & 15, o = lane >> 4;
#pragma unroll
  for (int p = 0; p < kPfNP; ++p) {
    if (!pv[p]) continue;
    const int n = (nb * (kPfBN / 16) + wn * kPfNP + p) * 16 + c;
#pragma unroll
    for (int mt = 0; mt < kPfMT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * 64 + mt * 16 + 4 * o + r;
        if (m < M) store_out(out, out_dtype, static_cast<size_t>(m) * N + n, gscale * acc[mt][p][r]);
      }
  }
}

}  // namespace

int launch_prefill(const GemmArgs& g, void* stream) {
  const int mblocks = (g.M + kPfBM - 1) / kPfBM;
  const int nblocks = (g.N / 16 + kPfBN / 16 - 1) / (kPfBN / 16);
  const int64_t nwg = static_cast<int64_t>(mblocks) * nblocks;
  const int64_t grid = (nwg + 7) / 8 * 8;
  hipLaunchKernelGGL(qgemm_prefill_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), g.w, g.panel_bytes, g.gscale, g.a, g.M, g.K, g.N, g.out,
                     g.out_dtype, g.nfull, g.half, mblocks, nblocks);
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
