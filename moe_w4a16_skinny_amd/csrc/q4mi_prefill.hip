// NVFP4 W4A16 GEMM for more than 16 activation rows (prefill chunks and
// large verify blocks): y[M][N] = g * a[M][K] . W[N][K]^T.
//
// [README, repository layout]: the engine runs a prefill beside decode;
// [DOC 3.3 "Decode vs prefill"]: a prefill pushes many tokens through each
// layer at once.  With many rows the product is bound by the matrix cores,
// not by the weight stream, so each dequantized weight fragment feeds several
// activation m-tiles and each activation fragment several weight panels.
//
// A workgroup of 4 waves computes a block of (16 WM MT) rows x (16 WN NP)
// columns, its waves as a WM x WN grid, each wave MT m-tiles x NP panels of
// 16 x 16 accumulators (by default 1 x 4 waves of 4 x 2: 64 x 128 blocks).
// Per 128-k tile the workgroup stages the block's activation rows in LDS
// (double buffered, 16-byte chunks XOR-swizzled by row so the fragment
// reads are conflict-free); every wave loads its panels' packed tiles
// straight into registers through a ring D tiles deep, dequantizes each
// 8-code step once and feeds it to MT MFMAs.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

#include "q4mi_tiles.h"

namespace q4mi {
using namespace dev;
namespace {

// The workgroup's 4 waves form a WM x WN grid; each wave owns MT 16-row
// m-tiles and NP 16-row weight panels, so a block is (16 WM MT) x (16 WN NP).

// NP panels' packed tiles for one lane: 4 code dwords (full tile; 2 for a
// half tile) and the scale bytes of its groups
template <int NP>
struct WTile {
  u32x4 c[NP];
  unsigned s[NP];
};

template <bool HALF, int NP>
__device__ __forceinline__ void load_wtile(WTile<NP>& t, const uint8_t* const (&pp)[NP], int64_t off, int lane) {
  const int c = lane & 15, h = (lane >> 5) & 1;
#pragma unroll
  for (int p = 0; p < NP; ++p) {  // a panel past N reads panel 0; its results are never stored
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

// activation block in LDS: row r (0..BM-1) of 128 k as 16 chunks of 8 f16,
// chunk q stored at position q ^ (r & 15)
template <int BM>
struct ABlock {
  u32x4 v[BM][16];
};

// thread t moves chunks t + 256 j (row (t + 256 j) / 16, chunk t % 16).
// Rows at or past M read row M - 1 instead (they only feed output rows that
// are never stored); chunks at k >= K (the last tile's padding) read a valid
// chunk and are replaced by zeros.  No load is predicated.
template <int BM>
struct ARows {
  const uint16_t* p[BM / 16];  // this thread's row pointers, chunk offset included
};
template <int BM>
__device__ __forceinline__ ARows<BM> a_rows(const uint16_t* __restrict__ a, int M, int K, int m0) {
  ARows<BM> r;
  const int q = threadIdx.x & 15;
#pragma unroll
  for (int j = 0; j < BM / 16; ++j) {
    const int m = min(m0 + (static_cast<int>(threadIdx.x) >> 4) + 16 * j, M - 1);
    r.p[j] = a + static_cast<int64_t>(m) * K + 8 * q;
  }
  return r;
}
// chunk inside k < K?  (K % 16 == 0: a chunk of 8 is all inside or all beyond)
__device__ __forceinline__ bool a_inside(int K, int k0) { return k0 + 8 * static_cast<int>(threadIdx.x & 15) < K; }
template <int BM>
__device__ __forceinline__ void fetch_a(u32x4 (&r)[BM / 16], const ARows<BM>& rows, int K, int k0) {
  // outside: the row's first chunk (replaced by zeros when it moves to LDS)
  const int off = a_inside(K, k0) ? k0 : -8 * static_cast<int>(threadIdx.x & 15);
#pragma unroll
  for (int j = 0; j < BM / 16; ++j) r[j] = *reinterpret_cast<const u32x4*>(rows.p[j] + off);
}
template <int BM>
__device__ __forceinline__ void put_a(ABlock<BM>& A, const u32x4 (&r)[BM / 16], int K, int k0) {
  const int q = threadIdx.x & 15;
  const bool inside = a_inside(K, k0);
#pragma unroll
  for (int j = 0; j < BM / 16; ++j) {
    const int row = (threadIdx.x >> 4) + 16 * j;
    A.v[row][q ^ (row & 15)] = inside ? r[j] : u32x4{0u, 0u, 0u, 0u};
  }
}

template <int STEPS, int MT, int NP, int BM>
__device__ __forceinline__ void tile_mma(f32x4 (&acc)[MT][NP], const ABlock<BM>& A, const WTile<NP>& w, int wm,
                                         int lane) {
  const int c = lane & 15, o = lane >> 4;
#pragma unroll
  for (int i = 0; i < STEPS; ++i) {
    f16x8 b[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) b[p] = nvfp4_operand(w.c[p][i], e4m3_pair(w.s[p], i >= 2)[i & 1]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = (wm * MT + mt) * 16 + c;
      const u32x4 af = A.v[row][(4 * i + o) ^ c];
#pragma unroll
      for (int p = 0; p < NP; ++p) acc[mt][p] = mfma_f16(af, b[p], acc[mt][p]);
    }
  }
}

// Workgroups are dealt in bands of up to SR row blocks: within a band the
// column blocks go in order, the band's row blocks fastest, and the 8 XCDs
// (blockIdx.x % 8) each take a contiguous range of that order.  The
// workgroups running together on one XCD then share a few column blocks'
// weights and the band's activation rows through its L2 (with the row
// blocks of all M fastest, every column block re-read all the activations).
template <int WM, int WN, int MT, int NP, int D>
__global__ __launch_bounds__(256) void qgemm_prefill_kernel(const uint8_t* __restrict__ w, int64_t pb, float gscale,
                                                            const uint16_t* __restrict__ a, int M, int K, int N,
                                                            void* __restrict__ out, int out_dtype, int nfull, int half,
                                                            int mblocks, int nblocks, int SR) {
  static_assert(WM * WN == 4, "4 waves");
  static_assert(D % 2 == 0, "the LDS buffer of tile t0 + d is d & 1");
  constexpr int BM = 16 * WM * MT, BN = 16 * WN * NP;
  static_assert(BM % 16 == 0 && BM <= 256, "block rows");
  __shared__ ABlock<BM> As[2];
  const int nwg = mblocks * nblocks;
  const int b = blockIdx.x;
  // XCD-major order: the grid is padded to a multiple of 8, idle slots return
  const int per_xcd = (nwg + 7) / 8;
  const int item = (b & 7) * per_xcd + (b >> 3);
  if (item >= nwg) return;
  const int band = item / (SR * nblocks);  // every band before the last is full
  const int rem = item - band * SR * nblocks;
  const int h = min(SR, mblocks - band * SR);  // row blocks in this band
  const int nb = rem / h;
  const int mb = band * SR + (rem - nb * h);
  const int m0 = mb * BM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WM, wn = wave / WM;
  const int npanels = N / 16;
  const uint8_t* pp[NP];
  bool pv[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int pn = nb * (BN / 16) + wn * NP + p;
    pv[p] = pn < npanels;
    pp[p] = w + static_cast<int64_t>(pv[p] ? pn : 0) * pb;
  }
  f32x4 acc[MT][NP];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int p = 0; p < NP; ++p) acc[mt][p] = f32x4{0.f, 0.f, 0.f, 0.f};

  // D-deep register ring over the full tiles: slot t % D holds tile t's
  // activation chunks (until they move to LDS) and weight tiles (until its
  // math); the loads of tile t + D are issued right after tile t's math, so
  // D - 1 tiles of math cover their latency.  The loop is unrolled by D so
  // every slot index is a compile-time constant, and the loads are issued
  // unconditionally (past the last tile they re-read it and are never used)
  // so that every path through the loop has the same loads in flight and the
  // waits for one slot's data do not wait for the younger slots.  A final
  // half tile (K ending inside a 128-k tile) is loaded and multiplied after
  // the ring.
  u32x4 ra[D][BM / 16];
  WTile<NP> wq[D];
  const ARows<BM> arows = a_rows<BM>(a, M, K, m0);
  auto issue = [&](int t, u32x4 (&r)[BM / 16], WTile<NP>& wt) {
    fetch_a<BM>(r, arows, K, t * kTileK);
    load_wtile<false>(wt, pp, static_cast<int64_t>(t) * kTileBytes, lane);
  };
  if (nfull > 0) {
#pragma unroll
    for (int d = 0; d < D; ++d) issue(min(d, nfull - 1), ra[d], wq[d]);
    put_a<BM>(As[0], ra[0], K, 0);
    __syncthreads();
    for (int t0 = 0; t0 < nfull; t0 += D) {
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const int t = t0 + d;
        if (t < nfull) tile_mma<4>(acc, As[d & 1], wq[d], wm, lane);
        if (t + 1 < nfull)  // that buffer's last readers passed the previous barrier
          put_a<BM>(As[(d + 1) & 1], ra[(d + 1) % D], K, (t + 1) * kTileK);
        issue(min(t + D, nfull - 1), ra[d], wq[d]);
        __syncthreads();
      }
    }
  }
  if (half) {  // tile nfull, in the buffer last read two tiles ago
    u32x4 rh[BM / 16];
    WTile<NP> wh;
    fetch_a<BM>(rh, arows, K, nfull * kTileK);
    load_wtile<true>(wh, pp, static_cast<int64_t>(nfull) * kTileBytes, lane);
    put_a<BM>(As[nfull & 1], rh, K, nfull * kTileK);
    __syncthreads();
    tile_mma<2>(acc, As[nfull & 1], wh, wm, lane);
  }

  // lane (c, o) holds rows 4 o + r of column c of each 16 x 16 accumulator
  const int c = lane & 15, o = lane >> 4;
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    if (!pv[p]) continue;
    const int n = (nb * (BN / 16) + wn * NP + p) * 16 + c;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + (wm * MT + mt) * 16 + 4 * o + r;
        if (m < M) store_out(out, out_dtype, static_cast<size_t>(m) * N + n, gscale * acc[mt][p][r]);
      }
  }
}

template <int WM, int WN, int MT, int NP, int D>
int launch_prefill_cfg(const GemmArgs& g, int sr, void* stream) {
  constexpr int BM = 16 * WM * MT, BN = 16 * WN * NP;
  const int mblocks = (g.M + BM - 1) / BM;
  const int nblocks = (g.N / 16 + BN / 16 - 1) / (BN / 16);
  const int64_t nwg = static_cast<int64_t>(mblocks) * nblocks;
  const int64_t grid = (nwg + 7) / 8 * 8;
  hipLaunchKernelGGL((qgemm_prefill_kernel<WM, WN, MT, NP, D>), dim3(static_cast<unsigned>(grid)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), g.w, g.panel_bytes, g.gscale, g.a, g.M, g.K, g.N, g.out,
                     g.out_dtype, g.nfull, g.half, mblocks, nblocks, sr);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

// Block shapes (waves WM x WN, per wave MT m-tiles x NP panels, D tiles of
// loads in flight); the choice can be overridden for measurements with
// Q4MI_PREFILL_CFG="WM,WN,MT,NP,D[,SR]".
int launch_prefill(const GemmArgs& g, void* stream) {
  int cfg[6] = {1, 4, 4, 2, 2, 8};  // ..., and SR: row blocks per band of the workgroup order
  if (const char* e = getenv("Q4MI_PREFILL_CFG"))
    sscanf(e, "%d,%d,%d,%d,%d,%d", &cfg[0], &cfg[1], &cfg[2], &cfg[3], &cfg[4], &cfg[5]);
  const int sr = cfg[5] < 1 ? 1 : cfg[5];
  const int key = cfg[0] * 10000 + cfg[1] * 1000 + cfg[2] * 100 + cfg[3] * 10 + cfg[4];
  switch (key) {
    case 14422: return launch_prefill_cfg<1, 4, 4, 2, 2>(g, sr, stream);
    case 14424: return launch_prefill_cfg<1, 4, 4, 2, 4>(g, sr, stream);
    case 14426: return launch_prefill_cfg<1, 4, 4, 2, 6>(g, sr, stream);
    case 14244: return launch_prefill_cfg<1, 4, 2, 4, 4>(g, sr, stream);
    case 22244: return launch_prefill_cfg<2, 2, 2, 4, 4>(g, sr, stream);
    case 22444: return launch_prefill_cfg<2, 2, 4, 4, 4>(g, sr, stream);
    case 22424: return launch_prefill_cfg<2, 2, 4, 2, 4>(g, sr, stream);
    case 14442: return launch_prefill_cfg<1, 4, 4, 4, 2>(g, sr, stream);
    case 14444: return launch_prefill_cfg<1, 4, 4, 4, 4>(g, sr, stream);
    case 22442: return launch_prefill_cfg<2, 2, 4, 4, 2>(g, sr, stream);
    case 14242: return launch_prefill_cfg<1, 4, 2, 4, 2>(g, sr, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace q4mi
