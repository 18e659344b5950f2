// MLX-style affine W{2,3,5,6,8}A16 skinny GEMM (M <= 16):
//   y[m][n] = sum_k a[m][k] * (q[n][k] * s[n][k / 64] + b[n][k / 64])
//
// [ISSUE "Why now"; "Steps" 3 and 9]: MLX's affine weights come at 2, 3, 4,
// 5, 6 and 8 bits in groups of 64 (the 4-bit width has its own layout and
// kernel).  Packed layout (q4_affine_bits_repack): per 16-row
// panel, 128-k tiles of 256 * BITS code bytes and 128 scale/bias bytes
// (the Fm<kAffineBits + BITS> trait of q4mi_tiles.h gives the lane
// geometry and the MFMA math); K is padded to 128 with zero codes and zero
// scale/bias.
//
// The kernel streams the tiles with the same register ring as the 4-bit
// GEMMs (stream_groups): a workgroup of W waves computes P panels, its waves
// splitting the tiles into W consecutive ranges, each wave keeping D tiles
// of weight loads in flight and moving each tile's 16 activation rows into
// its own LDS ring slot with direct-to-LDS loads issued beside them (rows
// past M repeat row M - 1; their outputs are dropped).  The waves' partial
// sums are added in LDS (in the rings' memory) in wave order
// (deterministic).
#include <hip/hip_runtime.h>

#include "q4mi_tiles.h"

namespace q4mi {
using namespace dev;
namespace {

template <int BITS, int P, int W, int D>
__global__ __launch_bounds__(64 * W) void qgemm_affineb_kernel(const uint8_t* __restrict__ w, int64_t pb, int ntiles,
                                                               int half_t, const uint16_t* __restrict__ a, int M,
                                                               int K, int N, void* __restrict__ out, int out_dtype) {
  constexpr int FMT = kAffineBits + BITS;
  // W rings of D slots; after the stream, the waves' partial sums [W][P][64]
  // in the same memory
  extern __shared__ u32x4 ring_lds[];
  f32x4(*const part)[P][64] = reinterpret_cast<f32x4(*)[P][64]>(ring_lds);
  static_assert(W * P * 64 * 16 <= W * D * kRingSlot, "the partial sums fit in the rings");
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, o = lane >> 4;
  const int npanels = N / 16;
  const int p0 = blockIdx.x * P;
  const int kt0 = (wv * ntiles) / W;  // this wave's tiles [kt0, kt0 + krg)
  const int krg = ((wv + 1) * ntiles) / W - kt0;
  const uint16_t* ar[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ar[j] = a + static_cast<size_t>(min(4 * j + o, M - 1)) * K + ring_chunk(j);
  auto group = [&](int, GroupPtrs<P>& gp) {  // one group: the workgroup's panels (past N: the last, never stored)
#pragma unroll
    for (int p = 0; p < P; ++p)
      gp.panel[p] = w + static_cast<size_t>(min(p0 + p, npanels - 1)) * static_cast<size_t>(pb);
#pragma unroll
    for (int j = 0; j < 4; ++j) gp.ar[j] = ar[j];
  };
  // the wave's sums stay in registers until every wave is out of its ring
  f32x4 sum[P];
#pragma unroll
  for (int p = 0; p < P; ++p) sum[p] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto park = [&](int, f32x4 (&acc)[P][2]) {
#pragma unroll
    for (int p = 0; p < P; ++p) sum[p] = acc[p][0] + acc[p][1];
  };
  auto park_add = [&](int, f32x4 (&acc)[P][2]) {
#pragma unroll
    for (int p = 0; p < P; ++p) sum[p] += acc[p][0] + acc[p][1];
  };
  auto none = [] {};
  const ARing rg = aring_view(lds_offset(ring_lds) + static_cast<unsigned>(wv * D * kRingSlot));
  if (krg > 0)  // (fewer tiles than waves: this wave's share stays zero)
    stream_groups<FMT, P, D, kARing>(1, krg, kt0, half_t, ALds{}, rg, K, group, none, none, park, park_add);
  __syncthreads();  // every ring is drained (the stream waits for its own loads at its end)
#pragma unroll
  for (int p = 0; p < P; ++p) part[wv][p][lane] = sum[p];
  __syncthreads();
  // wave p sums panel p over the waves in order and stores its 16 columns
  for (int p = wv; p < P; p += W) {
    f32x4 v = part[0][p][lane];
#pragma unroll
    for (int u = 1; u < W; ++u) v += part[u][p][lane];
    const int pn = p0 + p;
    if (pn < npanels) {
      const int n = pn * 16 + c;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 4 * o + r;
        if (m < M) store_out(out, out_dtype, static_cast<size_t>(m) * N + n, v[r]);
      }
    }
  }
}

template <int BITS, int P, int W, int D>
int launch_bits(const uint8_t* w, int64_t N, int64_t K, const uint16_t* a, int M, void* out, int out_dtype,
                void* stream) {
  const int ntiles = static_cast<int>((K + kTileK - 1) / kTileK);
  const int64_t pb = static_cast<int64_t>(ntiles) * Fm<kAffineBits + BITS>::kTile;
  // a last tile half past K streams as a half tile: its activations past K
  // are zeroed (its codes and scale/bias there are zero, but the activations
  // past the row's end need not be finite, or in the buffer)
  const int half_t = K % kTileK ? ntiles - 1 : -1;
  const int64_t blocks = (N / 16 + P - 1) / P;
  const size_t lds = static_cast<size_t>(W) * D * kRingSlot;
  const void* fn = reinterpret_cast<const void*>(&qgemm_affineb_kernel<BITS, P, W, D>);
  if (int e = ensure_dynamic_lds(fn, lds)) return e;
  hipLaunchKernelGGL((qgemm_affineb_kernel<BITS, P, W, D>), dim3(static_cast<unsigned>(blocks)), dim3(64 * W), lds,
                     static_cast<hipStream_t>(stream), w, pb, ntiles, half_t, a, M, static_cast<int>(K),
                     static_cast<int>(N), out, out_dtype);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

// Per width: P panels per workgroup, W waves, D tiles in flight per wave.
// Measured at M = 16, K = 5120, N = 15360 (same-process sweeps): 4 panels
// beat 2, 1 and 8; 2 tiles in flight beat 3, 4, 6 and 8 (smaller rings:
// more workgroups per CU); 8 waves suit the narrow codes (2-bit: 11.9 us
// against 13.8 with 4 waves, 12.9 with 16), 4 the wide ones (8-bit: 24.3
// against 24.6 with 8 and 57.6 with 16).
int launch_affine_bits(int bits, const uint8_t* w, int64_t N, int64_t K, const uint16_t* a, int M, void* out,
                       int out_dtype, void* stream) {
  switch (bits) {
    case 2: return launch_bits<2, 4, 8, 2>(w, N, K, a, M, out, out_dtype, stream);
    case 3: return launch_bits<3, 4, 8, 2>(w, N, K, a, M, out, out_dtype, stream);
    case 5: return launch_bits<5, 4, 4, 2>(w, N, K, a, M, out, out_dtype, stream);
    case 6: return launch_bits<6, 4, 4, 2>(w, N, K, a, M, out, out_dtype, stream);
    case 8: return launch_bits<8, 4, 4, 2>(w, N, K, a, M, out, out_dtype, stream);
    default: return static_cast<int>(hipErrorInvalidValue);
  }
}

}  // namespace q4mi
