// Router and grouped top-k MoE kernels for gfx950.
//
// [TensorSharp docs, Gemma 4, 3.2 "Per-layer (MoE)" and 4.6 "MoE"]: router
// matmul -> softmax -> top-k; each chosen expert runs its gated FFN and the
// outputs are summed with the routing weights.  [gemma-cuda-hybrid README,
// "Everything it has"]: 128 experts, top-8 plus one shared expert, a grouped
// MoE that reads each expert's weights once per step and uses no atomics.
// [TensorSharp docs, 14 "Completed": expert-batched GEGLU, a bounded number
// of launches per layer whatever the expert count.]
//
// Launch sequence of moe_grouped_qgemm (one stream, no host synchronization):
//   1. gate_up: grid (F/16 panel pairs / PW, experts).  Every workgroup
//      derives its expert's (token, slot) list from topk_idx with wave
//      ballots (stable in token, slot order), exits if the expert has no
//      tokens, and streams gate panel j and up panel j together so that
//      h = gelu_tanh(g_gate acc_g) * (g_up acc_u) is formed in registers and
//      written as f16 to the expert-sorted scratch h[pair][F].
//   2. down: grid (D/16 panels / (P PW), experts); rows are the expert's
//      contiguous h rows; o[pair][D] = w_pair * g_down * acc in fp32.
//   3. combine: y[t] = sum over slots in order + shared row (fixed order).
//
// moe_route_topk: one kernel; workgroups split D and write partial logits,
// the last workgroup to finish (completion counter) sums them in a fixed
// order, then computes the softmax and the top-k per token (ties to the lower
// expert index) and resets the counter.
#include <hip/hip_runtime.h>

#include "q4mi_tiles.h"

namespace q4mi {
namespace {
using namespace dev;

// ------------------------------------------------------------------ router

constexpr int kRouteThreads = 256;
constexpr int kRouteTG = 8;         // tokens per thread item
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs r) {
  extern __shared__ float rsm[];  // [rows][E] of W_r, then [T][rows] of x
  const int T = r.T, D = r.D, E = r.E;
  const int tid = threadIdx.x;
  const int rows = route_rows(T, D, E);
  const int d0 = blockIdx.x * rows;
  const int cn = min(D, d0 + rows) - d0;
  float* wrs = rsm;
  float* xs = rsm + static_cast<size_t>(rows) * E;
  const int ntg = (T + kRouteTG - 1) / kRouteTG;
  const int nitems = E * ntg;

  // stage the block: loads issued 8 at a time per thread, coalesced along E and D
  {
    const int nw = cn * E;
    for (int q0 = tid; q0 < nw; q0 += kRouteThreads * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * kRouteThreads;
        v[u] = q < nw ? r.wr[static_cast<size_t>(d0) * E + q] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * kRouteThreads;
        if (q < nw) wrs[q] = v[u];
      }
    }
    const int nx = T * cn;
    for (int q0 = tid; q0 < nx; q0 += kRouteThreads * 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * kRouteThreads;
        const int t = q / max(cn, 1), dd = q - t * cn;
        v[u] = q < nx ? (float)reinterpret_cast<const _Float16*>(r.x)[static_cast<size_t>(t) * D + d0 + dd] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * kRouteThreads;
        if (q < nx) xs[q] = v[u];
      }
    }
  }
  __syncthreads();
  for (int item = tid; item < nitems; item += kRouteThreads) {
    const int e = item % E, tg = item / E;
    float acc[kRouteTG];
#pragma unroll
    for (int t = 0; t < kRouteTG; ++t) acc[t] = 0.f;
    for (int dd = 0; dd < cn; ++dd) {
      const float w = wrs[dd * E + e];
#pragma unroll
      for (int t = 0; t < kRouteTG; ++t) {
        const int tt = tg * kRouteTG + t;
        if (tt < T) acc[t] = fmaf(xs[tt * cn + dd], w, acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < kRouteTG; ++t) {
      const int tt = tg * kRouteTG + t;
      if (tt < T) store_coherent(r.partial + (static_cast<size_t>(blockIdx.x) * T + tt) * E + e, acc[t]);
    }
  }
  wait_stores();  // this wave's partials are at the coherence point
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) s_last = count_arrival(r.counter) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // last workgroup: every block's partial of an item is loaded at once, then
  // summed in block order; then softmax and top-k per token
  float* lg = rsm;  // reuse: [T][E]
  const int nb = gridDim.x;
  for (int q = tid; q < T * E; q += kRouteThreads) {
    float v[kRouteMaxBlocks];
#pragma unroll
    for (int b = 0; b < kRouteMaxBlocks; ++b)
      v[b] = b < nb ? load_coherent(r.partial + static_cast<size_t>(b) * T * E + q) : 0.f;
    float s = 0.f;
#pragma unroll
    for (int b = 0; b < kRouteMaxBlocks; ++b) s += v[b];
    lg[q] = s;
    if (r.logits) r.logits[q] = s;
  }
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  for (int t = wv; t < T; t += kRouteThreads / 64) {
    const float* l = lg + static_cast<size_t>(t) * E;
    float v[4];
    bool taken[4];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      v[j] = e < E ? l[e] : -INFINITY;
      taken[j] = e >= E;
      mx = fmaxf(mx, v[j]);
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    float se = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) se += (lane + 64 * j < E) ? expf(v[j] - mx) : 0.f;
    for (int off = 32; off > 0; off >>= 1) se += __shfl_xor(se, off);
    float wsel[16];
    int isel[16];
    float wsum = 0.f;
    for (int s = 0; s < r.k; ++s) {
      // best (largest value, then lowest index) among the not-yet-chosen
      float bv = -INFINITY;
      int bi = 0x7FFFFFFF;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = lane + 64 * j;
        if (!taken[j] && (v[j] > bv || (v[j] == bv && e < bi))) {
          bv = v[j];
          bi = e;
        }
      }
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (lane + 64 * j == bi) taken[j] = true;
      const float p = expf(bv - mx) / se;
      if (s < 16) {
        wsel[s] = p;
        isel[s] = bi;
      }
      wsum += p;
    }
    if (lane == 0) {
      for (int s = 0; s < r.k && s < 16; ++s) {
        r.idx[t * r.k + s] = isel[s];
        r.w[t * r.k + s] = r.renormalize ? wsel[s] / wsum : wsel[s];
      }
    }
  }
  if (tid == 0) atomicExch(r.counter, 0u);
}

// ------------------------------------------------------------------ grouping

// (token, slot) pairs routed to expert e, in token-major order, plus the
// number of valid pairs routed to lower experts (the expert's first row in
// the expert-sorted scratch).  Run by wave 0; results in LDS.  Indices
// outside 0..E-1 are dropped; pairs past the 16th of one expert (possible
// only when a token names the same expert twice) are dropped too.
__device__ void group_expert(const int32_t* idx, int T, int k, int E, int e, int* s_tok, int* s_slot,
                             int* s_meta) {
  const int lane = threadIdx.x & 63;
  if (e >= E) {  // the shared expert: every token, after all routed pairs
    if (lane < T) {
      s_tok[lane] = lane;
      s_slot[lane] = -1;
    }
    if (lane == 0) {
      s_meta[0] = T;
      s_meta[1] = T * k;
    }
    return;
  }
  int cnt = 0, below = 0;
  const int n = T * k;  // <= 16 * 64: at most 16 indices per lane, all loaded at once
  int v[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int j = u * 64 + lane;
    v[u] = j < n ? idx[j] : -1;
  }
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    if (u * 64 >= n) break;
    const int j = u * 64 + lane;
    const bool valid = v[u] >= 0 && v[u] < E;
    const unsigned long long eq = __ballot(valid && v[u] == e);
    const unsigned long long lt = __ballot(valid && v[u] < e);
    if (valid && v[u] == e) {
      const int rk = cnt + __popcll(eq & ((1ull << lane) - 1ull));
      if (rk < 16) {
        s_tok[rk] = j / k;
        s_slot[rk] = j % k;
      }
    }
    cnt += __popcll(eq);
    below += __popcll(lt);
  }
  if (lane == 0) {
    s_meta[0] = min(cnt, 16);
    s_meta[1] = below;
  }
}

__device__ __forceinline__ float gelu_tanh(float u) {
  const float z = 0.7978845608028654f * fmaf(0.044715f * u * u, u, u);
  return 0.5f * u * (1.0f + tanhf(z));
}

// ------------------------------------------------------------------ gate/up

// Grid (panel-pair blocks, experts).  A workgroup owns PPB consecutive panel
// pairs of its expert; wave w streams pairs w, w + W, ... (gate panel j and
// up panel j together, P = 2) over all of K = D with D tiles in flight.
template <int W, int DP>
__global__ __launch_bounds__(64 * W) void moe_gate_up_kernel(MoeArgs m, int PPB) {
  const int e = blockIdx.y;
  __shared__ int s_tok[16], s_slot[16], s_meta[2];
  if (threadIdx.x < 64) group_expert(m.idx, m.T, m.k, m.E, e, s_tok, s_slot, s_meta);
  __syncthreads();
  const int me = s_meta[0];
  if (me == 0) return;
  const int base = s_meta[1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o = lane >> 4, c = lane & 15;
  const int npp = m.F / 16;                        // panel pairs of the expert
  const int j0 = blockIdx.x * PPB;
  const int jend = min(npp, j0 + PPB);
  const int ngb = jend - j0;
  const int ng = ngb > w ? (ngb - w + W - 1) / W : 0;
  const uint8_t* gate_e = m.gate + static_cast<size_t>(e) * m.gate_stride;
  const uint8_t* up_e = m.up + static_cast<size_t>(e) * m.gate_stride;
  const bool arow_ok = c < me;
  const uint16_t* arow = m.x + static_cast<size_t>(arow_ok ? s_tok[c] : 0) * m.D;
  const int nfull = static_cast<int>(full_tiles(m.D));
  const bool half = has_half_tile(m.D);
  const float gg = m.g_gate[e], gu = m.g_up[e];

  auto gbase = [&](int gi, int p) -> const uint8_t* {
    int jp = j0 + w + gi * W;
    jp = jp < npp ? jp : npp - 1;
    return (p == 0 ? gate_e : up_e) + static_cast<size_t>(jp) * m.gate_panel_bytes;
  };
  extern __shared__ f32x4 gu_out[];  // [W][NGW][2 panels][64 lanes]
  const int NGW = (PPB + W - 1) / W;
  f32x4* wout = gu_out + static_cast<size_t>(w) * NGW * 2 * 64;
  auto pre = [] {};
  auto epi = [&](int gi, f32x4 (&acc)[2][2]) { stash<2>(wout, gi, acc); };
  auto epi_add = [&](int gi, f32x4 (&acc)[2][2]) { stash_add<2>(wout, gi, acc); };
  stream_groups<kNvfp4, 2, DP, false>(ng, nfull + (half ? 1 : 0), 0, half ? nfull : -1, ALds{}, arow, arow_ok,
                                      m.D, gbase, pre, pre, epi, epi_add);
  for (int gi = 0; gi < ng; ++gi) {
    const int jp = j0 + w + gi * W;
    if (jp >= jend) continue;
    const f32x4 rg = wout[(gi * 2 + 0) * 64 + lane], ru = wout[(gi * 2 + 1) * 64 + lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * o + r;
      if (row < me) {
        const float h = gelu_tanh(gg * rg[r]) * (gu * ru[r]);
        reinterpret_cast<_Float16*>(m.h)[static_cast<size_t>(base + row) * m.F + jp * 16 + c] = (_Float16)h;
      }
    }
  }
}

// ------------------------------------------------------------------ down

// Grid (panel blocks, experts): PB panels of W_down (N = D) per workgroup,
// groups of P panels per wave, K = F; the activation rows are the expert's
// contiguous h rows.  o[pair][n] = w_pair * g_down * acc.
template <int P, int W, int DP>
__global__ __launch_bounds__(64 * W) void moe_down_kernel(MoeArgs m, int PB) {
  const int e = blockIdx.y;
  __shared__ int s_tok[16], s_slot[16], s_meta[2];
  if (threadIdx.x < 64) group_expert(m.idx, m.T, m.k, m.E, e, s_tok, s_slot, s_meta);
  __syncthreads();
  const int me = s_meta[0];
  if (me == 0) return;
  const int base = s_meta[1];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o = lane >> 4, c = lane & 15;
  const int npan = m.D / 16;
  const int p0 = blockIdx.x * PB;
  const int pend = min(npan, p0 + PB);
  const int ngb = (pend - p0 + P - 1) / P;
  const int ng = ngb > w ? (ngb - w + W - 1) / W : 0;
  const uint8_t* down_e = m.down + static_cast<size_t>(e) * m.down_stride;
  const bool arow_ok = c < me;
  const uint16_t* arow = m.h + static_cast<size_t>(base + (arow_ok ? c : 0)) * m.F;
  const int nfull = static_cast<int>(full_tiles(m.F));
  const bool half = has_half_tile(m.F);
  const float gd = m.g_down[e];
  float wrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * o + r;
    wrow[r] = 0.f;
    if (row < me) wrow[r] = s_slot[row] < 0 ? 1.0f : m.tw[s_tok[row] * m.k + s_slot[row]];
  }

  auto gbase = [&](int gi, int p) -> const uint8_t* {
    int pi = p0 + (w + gi * W) * P + p;
    pi = pi < npan ? pi : npan - 1;
    return down_e + static_cast<size_t>(pi) * m.down_panel_bytes;
  };
  extern __shared__ f32x4 dn_out[];  // [W][NGW][P][64]
  const int NGW = ((PB + P - 1) / P + W - 1) / W;
  f32x4* wout = dn_out + static_cast<size_t>(w) * NGW * P * 64;
  auto pre = [] {};
  auto epi = [&](int gi, f32x4 (&acc)[P][2]) { stash<P>(wout, gi, acc); };
  auto epi_add = [&](int gi, f32x4 (&acc)[P][2]) { stash_add<P>(wout, gi, acc); };
  stream_groups<kNvfp4, P, DP, false>(ng, nfull + (half ? 1 : 0), 0, half ? nfull : -1, ALds{}, arow, arow_ok,
                                      m.F, gbase, pre, pre, epi, epi_add);
  for (int gi = 0; gi < ng; ++gi) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int pi = p0 + (w + gi * W) * P + p;
      if (pi >= pend) continue;
      const f32x4 v = wout[(gi * P + p) * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * o + r;
        if (row < me) m.o[static_cast<size_t>(base + row) * m.D + pi * 16 + c] = wrow[r] * (gd * v[r]);
      }
    }
  }
}

// ------------------------------------------------------------------ combine

// y[t][n] = sum_{s<k} o[pos(t, s)][n] (+ o[T k + t][n] for the shared expert),
// slots in order.  pos(t, s) = (valid pairs routed to lower experts) + (rank of
// the pair among its expert's pairs), the row gate_up/down used for it.
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs m) {
  const int t = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  __shared__ int s_idx[16 * 64];
  __shared__ int s_pos[64];
  const int nall = m.T * m.k;
  for (int j = threadIdx.x; j < nall; j += 256) s_idx[j] = m.idx[j];
  __syncthreads();
  for (int s = threadIdx.x; s < m.k; s += 256) {
    const int e = s_idx[t * m.k + s];
    int pos = -1;
    if (e >= 0 && e < m.E) {
      int below = 0, rank = 0;
      for (int j = 0; j < nall; ++j) {
        const int v = s_idx[j];
        if (v >= 0 && v < m.E) {
          below += v < e;
          rank += (v == e) && (j < t * m.k + s);
        }
      }
      pos = rank < 16 ? below + rank : -1;
    }
    s_pos[s] = pos;
  }
  __syncthreads();
  if (n >= m.D) return;
  float acc = 0.f;
  for (int s0 = 0; s0 < m.k; s0 += 16) {  // 16 slots' rows in flight, summed in slot order
    float v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int s = s0 + u;
      const int pos = s < m.k ? s_pos[s] : -1;
      v[u] = pos >= 0 ? m.o[static_cast<size_t>(pos) * m.D + n] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += v[u];
  }
  if (m.has_shared) acc += m.o[static_cast<size_t>(nall + t) * m.D + n];
  if (m.out_dtype == Q4_F32)
    static_cast<float*>(m.y)[static_cast<size_t>(t) * m.D + n] = acc;
  else
    static_cast<_Float16*>(m.y)[static_cast<size_t>(t) * m.D + n] = (_Float16)acc;
}

}  // namespace

int launch_route(const RouteArgs& r, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = route_lds_bytes(r.T, r.D, r.E);
  static size_t lds_allowed = 48 * 1024;
  if (need > lds_allowed) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&route_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(need));
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return static_cast<int>(e);
    }
    lds_allowed = need;
  }
  hipLaunchKernelGGL(route_kernel, dim3(r.nblk), dim3(kRouteThreads), need, s, r);
  return static_cast<int>(hipGetLastError());
}

int launch_moe(const MoeArgs& m, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nexp = m.E + m.has_shared;
  constexpr int GU_W = 4, DN_P = 2, DN_W = 4;
  const int npp = m.F / 16;
  const int ppb = 2 * GU_W;  // panel pairs per gate/up workgroup: 2 per wave
  const size_t gu_lds = static_cast<size_t>(GU_W) * ((ppb + GU_W - 1) / GU_W) * 2 * 64 * 16;
  hipLaunchKernelGGL((moe_gate_up_kernel<GU_W, 4>), dim3((npp + ppb - 1) / ppb, nexp), dim3(64 * GU_W), gu_lds, s,
                     m, ppb);
  if (hipError_t e = hipGetLastError()) return static_cast<int>(e);
  const int npan = m.D / 16;
  const int pb = 2 * DN_P * DN_W;  // panels per down workgroup: 2 groups per wave
  const size_t dn_lds = static_cast<size_t>(DN_W) * (((pb + DN_P - 1) / DN_P + DN_W - 1) / DN_W) * DN_P * 64 * 16;
  hipLaunchKernelGGL((moe_down_kernel<DN_P, DN_W, 4>), dim3((npan + pb - 1) / pb, nexp), dim3(64 * DN_W), dn_lds, s,
                     m, pb);
  if (hipError_t e = hipGetLastError()) return static_cast<int>(e);
  hipLaunchKernelGGL(moe_combine_kernel, dim3(m.T, (m.D + 255) / 256), dim3(256), 0, s, m);
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
