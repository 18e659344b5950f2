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

// Ordered key of (logit, expert), kRouteKeyBits wide: larger logit first,
// then lower expert index (9 bits, E <= 256); distinct and non-zero for every
// expert (a NaN logit ranks below -inf); 0 marks "no expert".
constexpr int kRouteKeyBits = 41;
__device__ __forceinline__ unsigned long long route_key(float v, int e) {
  unsigned ord = 0u;
  if (v == v) {
    if (v == 0.0f) v = 0.0f;  // -0 and +0 compare equal
    const unsigned b = __float_as_uint(v);
    ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  }
  return (static_cast<unsigned long long>(ord) << 9) | (511u - static_cast<unsigned>(e)) + 0ull;
}
// logit of a key (inverse of the order map; NaN keys never reach this)
__device__ __forceinline__ float route_key_value(unsigned long long key) {
  const unsigned ord = static_cast<unsigned>(key >> 9);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Wave-wide reductions with DPP: row_shr 1, 2, 4, 8 leave each row's total in
// its lane 15, row_bcast 15 and 31 fold the rows into lane 63, which is then
// read into a scalar register (a fixed combination order).  Lanes shifted in
// from outside a row read 0, the identity of both reductions used here.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned x) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ unsigned long long dpp_max_key(unsigned long long k) {
  const unsigned lo = dpp_u32<CTRL>(static_cast<unsigned>(k));
  const unsigned hi = dpp_u32<CTRL>(static_cast<unsigned>(k >> 32));
  const unsigned long long o = (static_cast<unsigned long long>(hi) << 32) | lo;
  return o > k ? o : k;
}
__device__ __forceinline__ unsigned long long wave_max_key(unsigned long long k) {
  k = dpp_max_key<0x111>(k);  // row_shr:1
  k = dpp_max_key<0x112>(k);  // row_shr:2
  k = dpp_max_key<0x114>(k);  // row_shr:4
  k = dpp_max_key<0x118>(k);  // row_shr:8
  k = dpp_max_key<0x142>(k);  // row_bcast:15
  k = dpp_max_key<0x143>(k);  // row_bcast:31
  const unsigned lo = __builtin_amdgcn_readlane(static_cast<unsigned>(k), 63);
  const unsigned hi = __builtin_amdgcn_readlane(static_cast<unsigned>(k >> 32), 63);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(x)));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = dpp_add<0x111>(x);
  x = dpp_add<0x112>(x);
  x = dpp_add<0x114>(x);
  x = dpp_add<0x118>(x);
  x = dpp_add<0x142>(x);
  x = dpp_add<0x143>(x);
  return __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(x), 63));
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs r) {
  extern __shared__ float rsm[];  // [rows][16] staged x (fp32), then [slices][16][E] sums / [T][E] logits
  const int T = r.T, D = r.D, E = r.E;
  const int tid = threadIdx.x;
  const int R = r.rows;  // a multiple of 16 * (row slices)
  const int d0 = blockIdx.x * R;
  float* xs = rsm;
  float* red = rsm + (R * 16 > 4096 ? R * 16 : 4096);  // after the staged-x area (>= 16 KiB)
  const _Float16* x = reinterpret_cast<const _Float16*>(r.x);

  // Tokens in groups of 16: stage x (zeros past T and past D) as [row][16],
  // then v_mfma_f32_16x16x4_f32 jobs of 16 experts x a slice of the rows:
  // lane (c, q) = (lane & 15, lane >> 4) supplies A = x[token c][row 4i + q]
  // and B = W_r[row 4i + q][expert e0 + c]; its accumulator holds expert
  // e0 + c of tokens 4q + r.  Slices are summed in LDS in slice order.
  const int lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, kq = lane >> 4;
  const int cb = (E + 15) / 16;              // 16-expert column blocks
  const int ns = cb >= 8 ? 1 : 8 / cb;       // row slices per column block
  const int rps = R / ns;                    // rows per slice (a multiple of 16)
  for (int t0 = 0; t0 < T; t0 += 16) {
    const int tn = min(16, T - t0);
    for (int q0 = 0; q0 < R * 16; q0 += 8 * kRouteThreads) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * kRouteThreads + tid;
        const int dd = q >> 4, t = q & 15;
        const bool ok = q < R * 16 && t < tn && d0 + dd < D;
        const float xv = static_cast<float>(x[ok ? static_cast<size_t>(t0 + t) * D + d0 + dd : 0]);
        v[u] = ok ? xv : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u * kRouteThreads + tid;
        if (q < R * 16) xs[q] = v[u];
      }
    }
    __syncthreads();
    for (int job = wv; job < cb * ns; job += kRouteThreads / 64) {
      const int cbk = job % cb, sl = job / cb;
      const int e0 = cbk * 16;
      const float* wcol = r.wr + min(e0 + c, E - 1);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int i0 = sl * rps; i0 < (sl + 1) * rps; i0 += 16) {
        float av[4], bv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int dd = i0 + 4 * j + kq;
          av[j] = xs[dd * 16 + c];
          bv[j] = wcol[static_cast<size_t>(min(d0 + dd, D - 1)) * E];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[j], bv[j], acc, 0, 0, 0);
      }
      if (e0 + c < E) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) red[(sl * 16 + 4 * kq + rr) * E + e0 + c] = acc[rr];
      }
    }
    __syncthreads();
    for (int q = tid; q < tn * E; q += kRouteThreads) {
      const int t = q / E, ee = q - t * E;
      float sum = 0.f;
      for (int j = 0; j < ns; ++j) sum += red[(j * 16 + t) * E + ee];
      store_coherent(r.partial + (static_cast<size_t>(blockIdx.x) * T + t0 + t) * E + ee, sum);
    }
    __syncthreads();  // xs and red are reused
  }
  wait_stores();  // this wave's partials are at the coherence point
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) s_last = count_arrival(r.counter) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // last workgroup: the blocks' partials of 4 items per thread are loaded at
  // once, then summed in block order
  float* lg = red;  // reuse: [T][E]
  const int nb = gridDim.x;
  for (int q0 = 0; q0 < T * E; q0 += 4 * kRouteThreads) {
    float v[4][kRouteMaxBlocks];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kRouteThreads + tid;
#pragma unroll
      for (int b = 0; b < kRouteMaxBlocks; ++b)
        v[u][b] = (b < nb && q < T * E) ? load_coherent(r.partial + static_cast<size_t>(b) * T * E + q) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * kRouteThreads + tid;
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < kRouteMaxBlocks; ++b) sum += v[u][b];
      if (q < T * E) {
        lg[q] = sum;
        if (r.logits) r.logits[q] = sum;
      }
    }
  }
  __syncthreads();

  // Per token (one wave; lane l holds experts l + 64 j): k rounds of a
  // wave-wide maximum of the not-yet-chosen keys (keys are distinct, so each
  // round picks exactly one expert, in decreasing order, ties to the lower
  // index); softmax over all E with the first choice as the maximum.
  for (int t = wv; t < T; t += kRouteThreads / 64) {
    const float* l = lg + static_cast<size_t>(t) * E;
    float v[4];
    unsigned long long key[4];
    int slot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ee = lane + 64 * j;
      v[j] = ee < E ? l[ee] : -INFINITY;
      key[j] = ee < E ? route_key(v[j], ee) : 0ull;
      slot[j] = -1;
    }
    unsigned long long first = 0ull;
    for (int s = 0; s < r.k; ++s) {
      unsigned long long mine = 0ull;
#pragma unroll
      for (int j = 0; j < 4; ++j) mine = (slot[j] < 0 && key[j] > mine) ? key[j] : mine;
      const unsigned long long best = wave_max_key(mine);
#pragma unroll
      for (int j = 0; j < 4; ++j) slot[j] = key[j] == best ? s : slot[j];
      if (s == 0) first = best;
    }
    const float mx = route_key_value(first);
    float se = 0.f, ws = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float p = lane + 64 * j < E ? expf(v[j] - mx) : 0.f;
      se += p;
      ws += slot[j] >= 0 ? p : 0.f;
    }
    se = wave_sum(se);
    ws = wave_sum(ws);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (slot[j] >= 0) {
        const float p = expf(v[j] - mx) / se;
        r.idx[t * r.k + slot[j]] = lane + 64 * j;
        r.w[t * r.k + slot[j]] = r.renormalize ? p / (ws / se) : p;
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
  const size_t need = route_lds_bytes(r.D, r.E);
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
