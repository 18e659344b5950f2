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
//   1. gate_up: a fixed grid of 256 workgroups of 8 waves (one per CU).
//      Every workgroup stages x in LDS and builds the expert grouping (the
//      (token, slot) pairs sorted by expert, stable in token order) in LDS
//      from topk_idx; workgroup 0 also writes it to the workspace.  Work
//      items (active expert, gate panel j + up panel j) are dealt over the
//      waves; h = gelu_tanh(g_gate acc_g) * (g_up acc_u) is formed from the
//      parked results and written as f16 to the expert-sorted scratch
//      h[row][F].
//   2. down: the same grid; reads the grouping back, each workgroup a
//      contiguous range of items (active expert, group of P panels of
//      W_down) over the experts' h rows, staged in LDS;
//      o[t][slot][D] = w_pair * g_down * acc in fp32 (token-major).
//   3. combine: y[t] = sum over slots in order + the shared expert's slot.
// The MoE block runs its experts and its dense branch as two layers of one
// gate_up and one down launch (no combine: the block's own combine reads o).
//
// moe_route_topk: one kernel; workgroups split D and write partial logits,
// the last workgroup to finish (completion counter) sums them in a fixed
// order, then computes the softmax and the top-k per token (ties to the lower
// expert index) and resets the counter.  For the MoE block the same tail
// first turns the logits into the block's scores.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "q4mi_tiles.h"

namespace q4mi {
namespace {
using namespace dev;

// ------------------------------------------------------------------ router

// Order-preserving 32-bit code of a logit: a larger logit gets a larger
// code, -0 and +0 the same one; NaN gets 1, below every number; 0 marks "no
// expert" (taken, or past E).  Equal codes are told apart by expert index
// (the lower wins).
__device__ __forceinline__ unsigned route_ord(float v) {
  if (v != v) return 1u;
  if (v == 0.0f) v = 0.0f;
  const unsigned b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
// logit of a code (inverse of the order map; 1 gives a NaN)
__device__ __forceinline__ float route_ord_value(unsigned o) {
  return o == 1u ? __uint_as_float(0x7FC00000u) : __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

// DPP lane move (bound_ctrl: a lane whose source is outside the row reads 0)
template <int CTRL>
__device__ __forceinline__ unsigned dpp_u32(unsigned x) {
  return static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ __forceinline__ unsigned dpp_max_u32(unsigned x) {
  const unsigned o = dpp_u32<CTRL>(x);
  return o > x ? o : x;
}
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __uint_as_float(dpp_u32<CTRL>(__float_as_uint(x)));
}

// Reductions over the 16 lanes of a row, result in every lane: quad_perm
// [1,0,3,2] and [2,3,0,1] combine the lanes of a quad, row_half_mirror (lane
// i with 7 - i) and row_mirror (i with 15 - i) join quads and halves; every
// lane combines the same values in the same pairing order.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_min_u32(unsigned x) {
  const unsigned o = dpp_u32<CTRL>(x);
  return o < x ? o : x;
}
__device__ __forceinline__ unsigned row_max_u32(unsigned x) {
  x = dpp_max_u32<0xB1>(x);
  x = dpp_max_u32<0x4E>(x);
  x = dpp_max_u32<0x141>(x);
  return dpp_max_u32<0x140>(x);
}
__device__ __forceinline__ unsigned row_min_u32(unsigned x) {
  x = dpp_min_u32<0xB1>(x);
  x = dpp_min_u32<0x4E>(x);
  x = dpp_min_u32<0x141>(x);
  return dpp_min_u32<0x140>(x);
}
__device__ __forceinline__ float row_sum(float x) {
  x = dpp_add<0xB1>(x);
  x = dpp_add<0x4E>(x);
  x = dpp_add<0x141>(x);
  return dpp_add<0x140>(x);
}

// Top-k of the scores lg[T][E] (LDS) and their softmax, a token per 16-lane
// row (four per wave); lane p of the row holds experts p + 16 j, j < J (E <=
// 16 J).  Each of the k rounds takes the row-wide maximum of the codes still
// in play, then the row-wide minimum expert index holding it, and retires
// that expert; lane s keeps the round-s choice.  Softmax over all E with the
// first choice as the maximum.  Pair (t, s) goes to gidx (when non-NULL)
// and, with its weight (times ds[e] when ds is non-NULL; renormalized over
// the k when renorm), to oidx / ow (when oidx is non-NULL).  Used by the
// router's tail and by the routed gate/up prologue.
template <int J>
__device__ void route_topk_rows(int T, int E, int k, int renorm, const float* lg, const float* ds, int* gidx,
                                int32_t* oidx, float* ow) {
  const int lane = threadIdx.x & 63, p = lane & 15;
  for (int t0 = (threadIdx.x >> 6) * 4; t0 < T; t0 += (blockDim.x >> 6) * 4) {
    const int t = t0 + (lane >> 4);
    const bool ok = t < T;
    const float* l = lg + static_cast<size_t>(ok ? t : t0) * E;
    float v[J];
    unsigned ord[J];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const int ee = p + 16 * j;
      v[j] = ee < E ? l[ee] : 0.f;
      ord[j] = (ok && ee < E) ? route_ord(v[j]) : 0u;
    }
    unsigned first = 0u, my_ord = 0u, my_e = 0u;
    for (int s = 0; s < k; ++s) {
      unsigned lm = 0u;
#pragma unroll
      for (int j = 0; j < J; ++j) lm = max(lm, ord[j]);
      const unsigned m = row_max_u32(lm);
      unsigned ci = 0xFFFFu;
#pragma unroll
      for (int j = 0; j < J; ++j) ci = min(ci, ord[j] == m ? static_cast<unsigned>(p + 16 * j) : 0xFFFFu);
      const unsigned ce = row_min_u32(ci);
#pragma unroll
      for (int j = 0; j < J; ++j) ord[j] = static_cast<unsigned>(p + 16 * j) == ce ? 0u : ord[j];
      if (s == 0) first = m;
      if (p == s) {
        my_e = ce;
        my_ord = m;
      }
    }
    const float mx = route_ord_value(first);
    float se = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) se += p + 16 * j < E ? expf(v[j] - mx) : 0.f;
    se = row_sum(se);
    const float pm = p < k ? expf(route_ord_value(my_ord) - mx) : 0.f;
    const float ws = row_sum(pm);
    if (ok && p < k) {
      const int q = t * k + p;
      if (gidx) gidx[q] = static_cast<int>(my_e);
      if (oidx) {
        const float pr = pm / se;
        const float wv = renorm ? pr / (ws / se) : pr;
        oidx[q] = static_cast<int>(my_e);
        ow[q] = ds ? wv * ds[my_e] : wv;
      }
    }
  }
}

// The MoE block's router scores, in place over the [T][E] logits in LDS:
// z = RMSNorm(row; unit weights, eps) * zs (the scales, in LDS), a wave per
// token (sum of squares over lanes e = lane + 64 j, butterfly-reduced).
// Both routing paths (the router's tail, the routed gate/up) use it.
__device__ void route_block_scores(int T, int E, float eps, float* lg, const float* zs) {
  const int lane = threadIdx.x & 63;
  const int nw = blockDim.x >> 6;
  for (int t = threadIdx.x >> 6; t < T; t += nw) {
    float* row = lg + static_cast<size_t>(t) * E;
    float ss = 0.f;
    for (int e = lane; e < E; e += 64) ss = fmaf(row[e], row[e], ss);
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
    const float inv = 1.0f / sqrtf(ss / static_cast<float>(E) + eps);
    for (int e = lane; e < E; e += 64) row[e] = row[e] * inv * zs[e];
  }
}

constexpr int kRouteBatch = 12;  // 16-row steps of router weights loaded before their MFMAs

// Logits of 16 experts (column block eb) for every token over one split of
// D (rows [r0, r0 + R)), then, in the last workgroup, their sum over the
// splits and the top-k.  Tokens go in groups of 16: x is staged as
// [row][16] fp32 (zeros past T and past D); wave w takes rows r0 + w R/4 ..
// with v_mfma_f32_16x16x4_f32: lane (c, q) = (lane & 15, lane >> 4) supplies
// A = x[token c][row 4i + q] and B = W_r[row 4i + q][expert e0 + c], and its
// accumulator holds expert e0 + c of tokens 4q + r.  The router weights of up
// to kRouteBatch 16-row steps are loaded at once, the first batch right
// behind the x loads, and the staging barrier waits only for the x stores,
// so a wave waits for one round trip per batch.  Four independent
// accumulator chains are added in a fixed order; the waves' partial sums
// are added in LDS in wave order.
__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs r) {
  extern __shared__ float rsm[];  // [R][16] staged x (fp32; the last workgroup's [T][E] logits), then [4][256] sums
  const int T = r.T, D = r.D, E = r.E, R = r.rows;
  const int tid = threadIdx.x;
  const int neb = (E + 15) / 16;
  const int eb = blockIdx.x % neb, ds = blockIdx.x / neb;
  const int e0 = eb * 16, r0 = ds * R;
  const int xs_floats = R * 16 > 16384 ? R * 16 : 16384;
  float* xs = rsm;
  float* red = rsm + xs_floats;
  const _Float16* x = reinterpret_cast<const _Float16*>(r.x);
  const int lane = tid & 63, wv = tid >> 6;
  const int c = lane & 15, kq = lane >> 4;
  const int rw = R / (kRouteThreads / 64);  // rows per wave (a multiple of 16)
  const int i0w = wv * rw, i1w = i0w + rw;  // this wave's rows, relative to r0
  const float* wcol = r.wr + min(e0 + c, E - 1);

  float bv[kRouteBatch][4];
  auto load_batch = [&](int i0) {
#pragma unroll
    for (int b = 0; b < kRouteBatch; ++b)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int dd = min(i0 + 16 * b + 4 * j + kq, i1w - 1);  // past the wave's rows: a valid row, unused
        bv[b][j] = wcol[static_cast<size_t>(min(r0 + dd, D - 1)) * E];
      }
  };
  // x staging: item q = (chunk q >> 4 of 8 rows, token q & 15), one 16-byte
  // load of 8 consecutive f16 of the token's row (D % 8 == 0, so a chunk is
  // wholly inside or outside D), written as xs[row][token]
  const int nq = R * 2;  // R / 8 chunks x 16 tokens
  for (int t0 = 0; t0 < T; t0 += 16) {
    const int tn = min(16, T - t0);
    for (int q0 = 0; q0 < nq; q0 += 4 * kRouteThreads) {
      u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * kRouteThreads + tid;
        const int dd = (q >> 4) * 8, t = q & 15;
        const bool ok = q < nq && t < tn && r0 + dd < D;
        v[u] = ok ? *reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t0 + t) * D + r0 + dd)
                  : u32x4{0u, 0u, 0u, 0u};
      }
      if (q0 == 0) load_batch(i0w);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + u * kRouteThreads + tid;
        if (q < nq) {
          const int dd = (q >> 4) * 8, t = q & 15;
          const f16x8 h = __builtin_bit_cast(f16x8, v[u]);
#pragma unroll
          for (int i = 0; i < 8; ++i) xs[(dd + i) * 16 + t] = static_cast<float>(h[i]);
        }
      }
    }
    // LDS stores done (s_waitcnt lgkmcnt(0), vmcnt and expcnt left at their
    // maximum: the weight batch stays in flight), then the barrier
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    f32x4 acc4[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc4[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i0 = i0w; i0 < i1w; i0 += 16 * kRouteBatch) {
      if (i0 != i0w) load_batch(i0);
#pragma unroll
      for (int b = 0; b < kRouteBatch; ++b) {
        if (i0 + 16 * b < i1w) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc4[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(xs[(i0 + 16 * b + 4 * j + kq) * 16 + c], bv[b][j], acc4[j],
                                                           0, 0, 0);
        }
      }
    }
    const f32x4 acc = (acc4[0] + acc4[1]) + (acc4[2] + acc4[3]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) red[wv * 256 + (4 * kq + rr) * 16 + c] = acc[rr];
    __syncthreads();
    {
      const int t = tid >> 4, cc = tid & 15;  // 256 threads: token t, expert e0 + cc
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < kRouteThreads / 64; ++w) sum += red[w * 256 + tid];
      if (t < tn && e0 + cc < E) store_coherent(r.partial + (static_cast<size_t>(ds) * T + t0 + t) * E + e0 + cc, sum);
    }
    __syncthreads();  // xs and red are reused
  }
  if (r.partials_only) return;  // the gate/up launch sums them (the kernel boundary orders the two)
  wait_stores();  // this wave's partials are at the coherence point
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) s_last = count_arrival(r.counter) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;

  // last workgroup: every thread loads the splits' partials of 2 x 4 logits
  // at once with 16-byte loads (when T E is a multiple of 4, so that they
  // stay aligned; one logit per thread otherwise), then sums them in split
  // order.  The loads are unconditional (indexes past the end are clamped,
  // their values dropped), so that they all issue before the first wait.
  float* lg = xs;  // reuse: [T][E]
  const int ns = r.nsplit;
  const int TE = T * E;
  // the block's scales of expert tid (E <= 256 = the workgroup's threads),
  // loaded with the partials and parked in LDS after them
  __shared__ float s_zs[kRouteThreads], s_ds[kRouteThreads];
  float zs = 0.f, dsc = 1.0f;
  if (r.zscale && tid < E) {
    zs = r.zscale[tid];
    if (r.down_scale) dsc = r.down_scale[tid];
  }
  auto put = [&](int q, float v) {
    lg[q] = v;
    if (r.logits) r.logits[q] = v;
  };
  if ((TE & 3) == 0) {
    constexpr int kQ = 4 * kRouteThreads;  // logits per pass of the workgroup
    for (int q0 = 4 * tid; q0 < TE; q0 += 2 * kQ) {
      f32x4 v[2][kRouteMaxSplits];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int qc = min(q0 + h * kQ, TE - 4);
#pragma unroll
        for (int b = 0; b < kRouteMaxSplits; ++b)
          v[h][b] = load_coherent4(r.partial + static_cast<size_t>(min(b, ns - 1)) * TE + qc);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int q = q0 + h * kQ;
        f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < kRouteMaxSplits; ++b)
          if (b < ns) sum += v[h][b];
        if (q < TE) {
#pragma unroll
          for (int u = 0; u < 4; ++u) put(q + u, sum[u]);
        }
      }
    }
  } else {
    for (int q = tid; q < TE; q += kRouteThreads) {
      float v[kRouteMaxSplits];
#pragma unroll
      for (int b = 0; b < kRouteMaxSplits; ++b)
        v[b] = load_coherent(r.partial + static_cast<size_t>(min(b, ns - 1)) * TE + q);
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < kRouteMaxSplits; ++b)
        if (b < ns) sum += v[b];
      put(q, sum);
    }
  }
  if (r.zscale) {
    s_zs[tid] = zs;
    s_ds[tid] = dsc;
  }
  __syncthreads();
  if (r.zscale) {
    route_block_scores(r.T, r.E, r.eps, lg, s_zs);
    __syncthreads();
  }
  // (the down scale only for the block's scores: s_ds is 1 without one)
  const float* dsv = r.zscale ? s_ds : nullptr;
  if (E <= 128)
    route_topk_rows<8>(T, E, r.k, r.renormalize, lg, dsv, nullptr, r.idx, r.w);
  else
    route_topk_rows<16>(T, E, r.k, r.renormalize, lg, dsv, nullptr, r.idx, r.w);
  if (r.didx)  // the dense branch's one-expert routing
    for (int t = tid; t < T; t += blockDim.x) {
      r.didx[t] = 0;
      r.dw[t] = 1.0f;
    }
  if (tid == 0) atomicExch(r.counter, 0u);
}

// ------------------------------------------------------------------ grouping

// The expert-sorted scratch: routed (token, slot) pairs with a valid expert
// index, by expert, then token-major (t k + s) order inside an expert; then,
// with a shared expert, one row per token at T k + t.  At most 16 rows of an
// expert are computed (more only when a token names one expert twice); the
// rest are dropped, here and in the combine.  Every GEMM workgroup builds
// the table in LDS from topk_idx on its own (a few microseconds, no launch
// and no handoff between workgroups).
constexpr int kMoeMaxE = 1024;
constexpr int kMoeMaxPairs = 16 * 64;
struct MoeGroups {
  int cnt[kMoeMaxE + 1];       // valid pairs per expert (shared expert: T)
  int base[kMoeMaxE + 1];      // first scratch row of each expert
  unsigned tmask[kMoeMaxE];    // tokens (bit t) routed to each expert
  int act[kMoeMaxE + 1];       // experts with pairs, increasing
  int nact;
  int dup;                     // some token names one expert twice
  int idx[kMoeMaxPairs];
  int rowof[kMoeMaxPairs];     // pair t k + s -> scratch row (-1: invalid index or dropped)
  short tok[kMoeMaxPairs + 16];   // scratch row -> token
  short slot[kMoeMaxPairs + 16];  // scratch row -> slot (-1: shared expert)
  float gs0[kMoeMaxE + 1];        // g_gate and g_up of every expert, loaded with the
  float gs1[kMoeMaxE + 1];        // table so that the epilogue waits on no global load
};
// What down keeps of the grouping (read from the workspace), plus g_down of
// every expert and the routing weights [T k], loaded with it.  Smaller than
// MoeGroups, so that two down workgroups still fit in a CU's LDS.
struct MoeDownTable {
  int cnt[kMoeMaxE + 1];
  int base[kMoeMaxE + 1];
  int act[kMoeMaxE + 1];
  int nact;
  short tok[kMoeMaxPairs + 16];
  short slot[kMoeMaxPairs + 16];
  float gs0[kMoeMaxE + 1];
  float twl[kMoeMaxPairs];
  float fac[kMoeMaxPairs + 16];  // row -> its routing weight (1 for the shared expert)
};

// The routed gate/up prologue (m.rpart): the router's partial logits summed
// in split order (as the router's own tail sums them, so the logits are the
// same bits), the block's scores when m.zscale, then the router's top-k
// (route_topk_rows) into G.idx; also loads the gate/up global scales into
// gs0 / gs1.  rbuf: LDS for the
// logits and the two scale vectors (moe_route_lds bytes).  Ends after a
// barrier.
__device__ void route_pairs(const MoeArgs& m, MoeGroups& G, float* rbuf, bool publish) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int E = m.E, TE = m.T * E, ns = m.rsplit;
  const int ne = E + m.has_shared;
  float* lg = rbuf;
  float* zs = rbuf + TE;
  float* dsl = zs + E;
  // one batch of loads (ne <= E + 1 <= 257 < the workgroup's threads)
  float ga = 0.f, gb = 0.f, zv = 0.f, dv = 1.0f;
  if (tid < ne) {
    ga = m.g_gate[tid];
    gb = m.g_up[tid];
  }
  if (tid < E && m.zscale) zv = m.zscale[tid];
  if (tid < E && m.down_scale && publish) dv = m.down_scale[tid];
  for (int q0 = 4 * tid; q0 < TE; q0 += 4 * nt) {
    f32x4 v[kRouteMaxSplits];
#pragma unroll
    for (int b = 0; b < kRouteMaxSplits; ++b)
      v[b] = *reinterpret_cast<const f32x4*>(m.rpart + static_cast<size_t>(min(b, ns - 1)) * TE + q0);
    f32x4 sum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < kRouteMaxSplits; ++b)
      if (b < ns) sum += v[b];
    *reinterpret_cast<f32x4*>(lg + q0) = sum;
    if (publish && m.rlogits) *reinterpret_cast<f32x4*>(m.rlogits + q0) = sum;
  }
  if (tid < ne) {
    G.gs0[tid] = ga;
    G.gs1[tid] = gb;
  }
  if (tid < E) {
    zs[tid] = zv;
    dsl[tid] = dv;
  }
  __syncthreads();
  if (m.zscale) {
    route_block_scores(m.T, E, m.eps, lg, zs);
    __syncthreads();
  }
  const float* ds = m.down_scale ? dsl : nullptr;
  if (E <= 128)
    route_topk_rows<8>(m.T, E, m.k, m.renorm, lg, ds, G.idx, publish ? m.ridx : nullptr, m.rtw);
  else
    route_topk_rows<16>(m.T, E, m.k, m.renorm, lg, ds, G.idx, publish ? m.ridx : nullptr, m.rtw);
  __syncthreads();
}

// (also loads the gate/up global scales of every expert into gs0 / gs1)
// Routing: from topk_idx; from the router's partials (m.rpart; rbuf, the
// LDS that route_pairs borrows); or the constant one-expert routing
// (m.rconst).  publish: this workgroup writes the routing (ridx, rtw,
// rlogits) for the caller and for down.
__device__ void build_groups(const MoeArgs& m, MoeGroups& G, float* rbuf = nullptr, bool publish = false) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int E = m.E, k = m.k, n = m.T * k;
  const int ne = E + m.has_shared;
  for (int e = tid; e <= E; e += nt) {
    G.cnt[e] = 0;
    if (e < E) G.tmask[e] = 0u;
  }
  if (tid == 0) G.dup = 0;
  if (m.rpart) {
    route_pairs(m, G, rbuf, publish);
  } else {
    for (int q = tid; q < max(n, ne); q += nt) {  // one batch of loads
      const int e = q < n ? (m.rconst ? 0 : m.idx[q]) : -1;
      const float ga = q < ne ? m.g_gate[q] : 0.f, gb = q < ne ? m.g_up[q] : 0.f;
      if (q < n) G.idx[q] = (e >= 0 && e < E) ? e : -1;
      if (q < ne) {
        G.gs0[q] = ga;
        G.gs1[q] = gb;
      }
      if (q < n && m.rconst && publish) {
        m.ridx[q] = 0;
        m.rtw[q] = 1.0f;
      }
    }
    __syncthreads();
  }
  for (int q = tid; q < n; q += nt) {
    const int e = G.idx[q];
    if (e < 0) continue;
    const int t = q / k;
    atomicAdd(&G.cnt[e], 1);
    // of two slots of one token naming the same expert, the later OR sees the bit set
    if (atomicOr(&G.tmask[e], 1u << t) & (1u << t)) G.dup = 1;
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    // exclusive scans of the counts (row bases) and of the active flags, lane l
    // owning experts [l per, (l + 1) per)
    const int per = (E + 63) / 64;
    const int e0 = lane * per;
    int sc = 0, sa = 0;
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) {
        sc += G.cnt[e];
        sa += G.cnt[e] > 0 ? 1 : 0;
      }
    }
    // both scans in one word (each sum is at most T k + E < 2^16)
    int x = (sc << 16) | sa;
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    int xc = (x >> 16) - sc;
    int xa = (x & 0xFFFF) - sa;
    for (int j = 0; j < per; ++j) {
      const int e = e0 + j;
      if (e < E) {
        G.base[e] = xc;
        xc += G.cnt[e];
        if (G.cnt[e] > 0) G.act[xa++] = e;
      }
    }
    if (lane == 63) {
      int na = xa;
      if (m.has_shared) {
        G.cnt[E] = m.T;
        G.base[E] = n;
        G.act[na++] = E;
      }
      G.nact = na;
    }
  }
  __syncthreads();
  // Row of pair (t, s) = base[e] + rank, the rank counting the expert's
  // pairs of lower tokens (token-major order): the popcount of its token
  // mask below bit t.  Tokens that name one expert twice break that count;
  // then wave 0 ranks the pairs 64 at a time instead (earlier lanes with the
  // same expert, broadcast through scalar registers, plus earlier chunks).
  if (!G.dup) {
    for (int q = tid; q < n; q += nt) {
      const int e = G.idx[q];
      int row = -1;
      if (e >= 0) {
        const int t = q / k;
        const int rank = __popc(G.tmask[e] & ((1u << t) - 1u));
        if (rank < 16) {
          row = G.base[e] + rank;
          G.tok[row] = static_cast<short>(t);
          G.slot[row] = static_cast<short>(q - t * k);
        }
      }
      G.rowof[q] = row;
    }
  } else if (tid < 64) {
    const int lane = tid;
    for (int q0 = 0; q0 < n; q0 += 64) {
      const int q = q0 + lane;
      const int e = q < n ? G.idx[q] : -1;
      int below = 0;
      for (int l = 0; l < 64; ++l) {
        const int el = __builtin_amdgcn_readlane(e, l);
        below += (el == e && l < lane) ? 1 : 0;
      }
      int earlier = 0;  // same-expert pairs in earlier chunks
      for (int j = 0; j < q0; ++j) earlier += (G.idx[j] == e) ? 1 : 0;
      int row = -1;
      if (e >= 0) {
        const int rank = earlier + below;
        if (rank < 16) {
          row = G.base[e] + rank;
          G.tok[row] = static_cast<short>(q / k);
          G.slot[row] = static_cast<short>(q - (q / k) * k);
        }
      }
      if (q < n) G.rowof[q] = row;
    }
  }
  if (m.has_shared)
    for (int t = tid; t < m.T; t += nt) {
      G.tok[n + t] = static_cast<short>(t);
      G.slot[n + t] = -1;
    }
  __syncthreads();
}

// Issue priority of a wave by the number of its items not yet entered (0..3):
// on a CU shared by waves with different amounts of work left, the ones with
// more left go first, so that the CU's waves finish closer together.
__device__ __forceinline__ void prio_by_items_left(int left) {
  if (left >= 3)
    __builtin_amdgcn_s_setprio(3);
  else if (left == 2)
    __builtin_amdgcn_s_setprio(2);
  else if (left == 1)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// The grouping as the down kernel needs it (counts, row bases, active
// experts, row -> token and slot), passed from gate/up through the
// workspace: gate/up's workgroup 0 writes it after building it, and every
// down workgroup reads it into LDS instead of building it again (the kernel
// boundary orders the two).
__device__ void publish_groups(const MoeArgs& m, const MoeGroups& G) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int E1 = m.E + 1, nrow = m.T * m.k + m.T;
  int32_t* g = m.grp;
  if (tid == 0) g[0] = G.nact;
  for (int e = tid; e < E1; e += nt) {
    g[4 + e] = G.act[e];
    g[4 + E1 + e] = G.cnt[e];
    g[4 + 2 * E1 + e] = G.base[e];
  }
  short* ts = reinterpret_cast<short*>(g + 4 + 3 * E1);
  for (int q = tid; q < nrow; q += nt) {
    ts[q] = G.tok[q];
    ts[nrow + q] = G.slot[q];
  }
}
// (also loads g_down of every expert into gs0 and the routing weights into twl)
__device__ void fetch_groups(const MoeArgs& m, MoeDownTable& G) {
  const int tid = threadIdx.x, nt = blockDim.x;
  const int E1 = m.E + 1, nrow = m.T * m.k + m.T, npair = m.T * m.k;
  const int ne = m.E + m.has_shared;
  const int32_t* g = m.grp;
  const short* ts = reinterpret_cast<const short*>(g + 4 + 3 * E1);
  if (tid == 0) G.nact = g[0];
  for (int i = tid; i < max(E1, nrow); i += nt) {  // one batch of loads
    int a = 0, c = 0, b = 0;
    short tk = 0, sl = 0;
    float gd = 0.f, tw = 0.f;
    if (i < E1) {
      a = g[4 + i];
      c = g[4 + E1 + i];
      b = g[4 + 2 * E1 + i];
    }
    if (i < ne) gd = m.g_down[i];
    if (i < nrow) {
      tk = ts[i];
      sl = ts[nrow + i];
    }
    if (i < npair) tw = m.tw[i];
    if (i < E1) {
      G.act[i] = a;
      G.cnt[i] = c;
      G.base[i] = b;
    }
    if (i < ne) G.gs0[i] = gd;
    if (i < nrow) {
      G.tok[i] = tk;
      G.slot[i] = sl;
    }
    if (i < npair) G.twl[i] = tw;
  }
  __syncthreads();
  for (int i = tid; i < nrow; i += nt) {
    const int sl = G.slot[i];
    G.fac[i] = sl < 0 ? 1.0f : G.twl[G.tok[i] * m.k + sl];
  }
  __syncthreads();
}

// GELU, tanh form: 0.5 u (1 + tanh z), z = sqrt(2/pi) (u + 0.044715 u^3).
// Since 1 + tanh z = 2 / (1 + e^(-2z)), this is u / (1 + e^(-2z)): one
// hardware exp2 and one reciprocal (a few ulp; e^(-2z) = inf gives 0, and
// 0 gives u, so both tails saturate exactly).
__device__ __forceinline__ float gelu_tanh(float u) {
  const float z = 0.7978845608028654f * fmaf(0.044715f * u * u, u, u);
  const float e = __builtin_amdgcn_exp2f(-2.8853900817779268f * z);  // e^(-2z) = 2^(-2z log2 e)
  return u * __builtin_amdgcn_rcpf(1.0f + e);
}

// it / d for the item indexes (it d < 2^32): multiply-high by ceil(2^32 / d)
struct DivBy {
  unsigned d, mag;
  __device__ explicit DivBy(unsigned dd) : d(dd), mag(dd > 1 ? 0xFFFFFFFFu / dd + 1u : 0u) {}
  __device__ int operator()(int it) const {
    return d > 1 ? static_cast<int>(__umulhi(static_cast<unsigned>(it), mag)) : it;
  }
};

// Work items are dealt round-robin over the workgroups first, then over the
// waves of a workgroup: wave w of workgroup b is wave gw = b + w gridDim of
// NW and takes items gw, gw + NW, ...; its g-th item is gw + g NW.  Every
// workgroup (and so every CU) then gets the same number of items up to one,
// and consecutive items, such as the shared expert's, land on different
// workgroups.
__device__ __forceinline__ int items_of_wave(int nitems, int gw, int NW) {
  return gw < nitems ? (nitems - gw + NW - 1) / NW : 0;
}

// Two layers in one launch: the workgroups of the first layer, in proportion
// to the tile-items of each (the first layer's from its active experts, u0
// per expert; w1 for the second), at least one each.  Every workgroup
// computes the same value from the same grouping.
__device__ __forceinline__ int layer_split(int nact0, int u0, int w1) {
  const long long w0 = static_cast<long long>(nact0) * u0;
  const long long n = gridDim.x;
  const long long sp = (n * w0 + (w0 + w1) / 2) / (w0 + w1 > 0 ? w0 + w1 : 1);
  return static_cast<int>(sp < 1 ? 1 : (sp > n - 1 ? n - 1 : sp));
}

// ------------------------------------------------------------------ gate/up

// Item (active expert a, panel pair j): gate panel j and up panel j of the
// expert streamed together over K = D (P = 2), h = gelu_tanh(g_gate acc_g) *
// (g_up acc_u) for the expert's rows, written as f16 to the scratch row.
// AM = kAStagedRows: the workgroup first stages all of x [T][D] in LDS
// (with its first weight loads in flight), and each item's tokens are read
// from there, so the stream issues only weight loads; AM = kAGlobal (when x
// does not fit beside the stash): lanes load their token's activations.
// KS: a layer with few items (one expert: the block's dense branch) gives
// each item to a whole workgroup, its W waves streaming W consecutive
// ranges of the K tiles; the waves' partial sums meet in LDS and are added
// in wave order before the epilogue.  Otherwise an item is one wave's.
// TWO: two layers share the launch (the MoE block's experts and its dense
// branch): workgroups below `split` run layer L.l[0], the others L.l[1],
// each set dealing its own layer's items among its own workgroups (bid of
// nwg).
template <int W, int DP, int AM, bool KS, bool TWO>
__global__ __launch_bounds__(64 * W) void moe_gate_up_kernel(MoeLayers L, int u0, int w1, int ngw0, int ngw1) {
  __shared__ MoeGroups G;
  extern __shared__ f32x4 gu_dyn[];
  auto stage_x = [&](const MoeArgs& mm) {
    if constexpr (AM == kAStagedRows) {
      const int ntx = static_cast<int>(full_tiles(mm.D) + (has_half_tile(mm.D) ? 1 : 0));
      stage_issue(stage_geom(mm.x, mm.T, mm.D, 0, ntx), reinterpret_cast<u32x4*>(gu_dyn));
    }
  };
  // the routed prologue's LDS: the start of the stash (past the staged x;
  // the two layers of a launch have the same T and D)
  float* const rbuf = reinterpret_cast<float*>(
      reinterpret_cast<char*>(gu_dyn) +
      (AM == kAStagedRows
           ? (static_cast<size_t>(stage_bytes(L.l[0].T, static_cast<int>(full_tiles(L.l[0].D) +
                                                                            (has_half_tile(L.l[0].D) ? 1 : 0)))) +
              15) / 16 * 16
           : 0));
  int r = 0, split = static_cast<int>(gridDim.x);
  if constexpr (TWO) {
    // the split follows the first layer's active experts; the second
    // layer's workgroups then build their own grouping and stage their x,
    // which has landed at the barrier below (staging the first layer's x
    // before the grouping, for the many workgroups that run it, measured
    // no faster: the second layer's then stage twice)
    build_groups(L.l[0], G, rbuf, blockIdx.x == 0);
    split = layer_split(G.nact, u0, w1);
    r = static_cast<int>(blockIdx.x) >= split ? 1 : 0;
    if (r) {
      __syncthreads();
      build_groups(L.l[1], G, rbuf, static_cast<int>(blockIdx.x) == split);
    }
    stage_x(L.l[r]);
    __syncthreads();
  } else {
    // x is staged first, its loads in flight while the grouping's own loads
    // (topk_idx or the router's partials, the global scales) make their
    // round trip; the grouping's first barrier waits for both
    stage_x(L.l[0]);
    build_groups(L.l[0], G, rbuf, blockIdx.x == 0);
  }
  const MoeArgs& m = L.l[r];  // (a uniform index into the kernel arguments: one load per field)
  const int bid = static_cast<int>(blockIdx.x) - (r ? split : 0);
  const int nwg = r ? static_cast<int>(gridDim.x) - split : split;
  const int NGW = r ? ngw1 : ngw0;
  if (bid == 0) {  // the pair -> row map, for the combine; the grouping, for down
    for (int q = threadIdx.x; q < m.T * m.k; q += blockDim.x) m.rowof[q] = G.rowof[q];
    publish_groups(m, G);
  }
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o = lane >> 4, c = lane & 15;
  const int npp = m.F / 16;
  const int nitems = G.nact * npp;
  // the item dealer: a wave (gw of NW), or with KS the whole workgroup
  const int gw = KS ? bid : bid + nwg * w;
  const int NW = KS ? nwg : nwg * W;
  // a wave's items go in chunks of at most NGW (its stash slots)
  const int ntot = items_of_wave(nitems, gw, NW);
  if (KS && ntot == 0) return;  // the whole workgroup idle
  int c0 = 0, ng = 0;  // current chunk: items c0 .. c0 + ng
  const int nfull = static_cast<int>(full_tiles(m.D));
  const bool half = has_half_tile(m.D);
  const int ntx0 = nfull + (half ? 1 : 0);
  const int kt0 = KS ? (w * ntx0) / W : 0;  // this wave's K tiles [kt0, kt0 + krg)
  const int krg = KS ? ((w + 1) * ntx0) / W - kt0 : ntx0;

  const DivBy by_npp(static_cast<unsigned>(npp));
  const __amdgpu_buffer_rsrc_t xr = act_rsrc(m.x, static_cast<unsigned>(m.T) * static_cast<unsigned>(m.D) * 2u);
  const int ntx = nfull + (half ? 1 : 0);
  const unsigned xrs = static_cast<unsigned>(stage_row_stride(ntx));  // staged row stride (bytes)
  auto item = [&](int gi, int& e, int& jp) {
    int it = gw + (c0 + gi) * NW;
    it = it < nitems ? it : nitems - 1;  // past the wave's items: in-bounds, never computed
    const int a = by_npp(it);
    jp = it - a * npp;
    e = G.act[a];
  };
  auto group = [&](int gi, GroupPtrs<2>& gp) {
    prio_by_items_left(ntot - c0 - gi);
    int e, jp;
    item(gi, e, jp);
    gp.panel[0] = m.gate + static_cast<size_t>(e) * m.gate_stride + static_cast<size_t>(jp) * m.gate_panel_bytes;
    gp.panel[1] = m.up + static_cast<size_t>(e) * m.gate_stride + static_cast<size_t>(jp) * m.gate_panel_bytes;
    const int me = min(G.cnt[e], 16);
    if constexpr (AM == kAStagedRows) {
      gp.alds = static_cast<unsigned>(G.tok[G.base[e] + min(c, me - 1)]) * xrs + static_cast<unsigned>(kt0) * 256u;
    } else {
      gp.arsrc = xr;
      gp.aoff = c < me ? static_cast<unsigned>(G.tok[G.base[e] + c]) * static_cast<unsigned>(m.D) * 2u : kDeadLane;
    }
  };
  // dynamic LDS: [staged x (kAStagedRows)] then the stash [W][NGW][2 panels][64 lanes]
  char* const dyn = reinterpret_cast<char*>(gu_dyn);
  const size_t xbytes = AM == kAStagedRows ? (static_cast<size_t>(stage_bytes(m.T, ntx)) + 15) / 16 * 16 : 0;
  f32x4* wout = reinterpret_cast<f32x4*>(dyn + xbytes) + static_cast<size_t>(w) * NGW * 2 * 64;
  const ALds al{dyn + 16 * o};
  auto none = [] {};
  auto epi = [&](int gi, f32x4 (&acc)[2][2]) { stash<2>(wout, gi, acc); };
  auto epi_add = [&](int gi, f32x4 (&acc)[2][2]) { stash_add<2>(wout, gi, acc); };
  f32x4* const stash0 = reinterpret_cast<f32x4*>(dyn + xbytes);
  auto finish = [&]() {
    if constexpr (KS) __syncthreads();  // every wave's partial sums parked
    for (int gi = KS ? w : 0; gi < ng; gi += KS ? W : 1) {
      int e, jp;
      item(gi, e, jp);
      const int me = min(G.cnt[e], 16), base = G.base[e];
      const float gg = G.gs0[e], gu = G.gs1[e];
      f32x4 rg = wout[(gi * 2 + 0) * 64 + lane], ru = wout[(gi * 2 + 1) * 64 + lane];
      if constexpr (KS) {
        rg = ru = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int v = 0; v < W; ++v) {  // the waves' K ranges, in order
          const f32x4* sv = stash0 + static_cast<size_t>(v) * NGW * 2 * 64;
          rg += sv[(gi * 2 + 0) * 64 + lane];
          ru += sv[(gi * 2 + 1) * 64 + lane];
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * o + r;
        if (row < me) {
          const float h = gelu_tanh(gg * rg[r]) * (gu * ru[r]);
          reinterpret_cast<_Float16*>(m.h)[static_cast<size_t>(base + row) * m.F + jp * 16 + c] = (_Float16)h;
        }
      }
    }
    if constexpr (KS) __syncthreads();  // the stash is free for the next chunk
    c0 += NGW;
  };
  while (c0 < ntot) {
    ng = min(NGW, ntot - c0);
    stream_groups<kNvfp4, 2, DP, AM>(ng, krg, kt0, half ? nfull : -1, al, ARing{}, m.D, group, none, none, epi,
                                     epi_add);
    finish();
  }
}

// ------------------------------------------------------------------ down

// Item (active expert a, group q of P panels of W_down, N = D): K = F, the
// activation rows are the expert's contiguous h rows; o[row][n] = w_pair *
// g_down * acc in fp32.  KS: every item of the workgroup's range is streamed
// by all W waves, each over its own range of the K tiles, as in gate/up.
// TWO as in gate/up; lds is the launch's dynamic LDS size.
// DPG: tiles in flight when a workgroup's rows do not fit in LDS (read
// through a buffer resource instead); a shallower ring there keeps that
// rarely taken path from setting the register budget of the staged one.
template <int P, int W, int DP, bool KS, bool TWO, int DPG = DP>
__global__ __launch_bounds__(64 * W) void moe_down_kernel(MoeLayers L, int u0, int w1, int ngw0, int ngw1,
                                                          int lds) {
  __shared__ MoeDownTable G;
  fetch_groups(L.l[0], G);
  int r = 0, split = static_cast<int>(gridDim.x);
  if constexpr (TWO) {  // the split as in gate/up, then the second layer's table
    split = layer_split(G.nact, u0, w1);
    r = static_cast<int>(blockIdx.x) >= split ? 1 : 0;
    if (r) {
      __syncthreads();
      fetch_groups(L.l[1], G);
    }
  }
  const MoeArgs& m = L.l[r];
  const int bid = static_cast<int>(blockIdx.x) - (r ? split : 0);
  const int nwg = r ? static_cast<int>(gridDim.x) - split : split;
  const int NGW = r ? ngw1 : ngw0;
  // the rest of the dynamic LDS past the stash holds the staged h rows
  const int stage_room = lds - W * NGW * P * 64 * 16;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o = lane >> 4, c = lane & 15;
  const int npan = m.D / 16;
  const int ngp = (npan + P - 1) / P;  // panel groups per expert
  const int nitems = G.nact * ngp;
  // the workgroup's items: a contiguous range (one or two experts' panel
  // groups), dealt round-robin to its waves
  const int i0 = static_cast<int>((static_cast<long long>(bid) * nitems) / nwg);
  const int i1 = static_cast<int>((static_cast<long long>(bid + 1) * nitems) / nwg);
  if (i1 <= i0) return;  // no item for this workgroup (uniform)
  // items of this wave (all of the range with KS), in chunks of at most NGW, as in gate/up
  const int ntot = KS ? i1 - i0 : (i1 - i0 > w ? (i1 - i0 - w + W - 1) / W : 0);
  int c0 = 0, ng = 0;
  const int nfull = static_cast<int>(full_tiles(m.F));
  const bool half = has_half_tile(m.F);
  const int ntf = nfull + (half ? 1 : 0);
  const int kt0 = KS ? (w * ntf) / W : 0;  // this wave's K tiles [kt0, kt0 + krg)
  const int krg = KS ? ((w + 1) * ntf) / W - kt0 : ntf;

  const DivBy by_ngp(static_cast<unsigned>(ngp));
  const unsigned nrows_h = static_cast<unsigned>(m.T * m.k + (m.has_shared ? m.T : 0));
  const __amdgpu_buffer_rsrc_t hr = act_rsrc(m.h, nrows_h * static_cast<unsigned>(m.F) * 2u);
  auto item = [&](int gi, int& e, int& q) {
    int it = KS ? i0 + c0 + gi : i0 + w + (c0 + gi) * W;
    it = it < i1 ? it : i1 - 1;  // past the wave's items: in-bounds, never computed
    const int a = by_ngp(it);
    q = it - a * ngp;
    e = G.act[a];
  };
  // the h rows of the experts the range spans are contiguous: stage them in
  // LDS if they fit, so the stream issues only weight loads
  const int e_lo = G.act[by_ngp(i0)], e_hi = G.act[by_ngp(i1 - 1)];
  const int rlo = G.base[e_lo], rhi = G.base[e_hi] + G.cnt[e_hi];
  const unsigned hrs = static_cast<unsigned>(stage_row_stride(ntf));
  const bool staged = static_cast<long long>(stage_bytes(rhi - rlo, ntf)) <= stage_room;
  extern __shared__ f32x4 dn_dyn[];  // [W][NGW][P][64] stash, then the staged rows
  f32x4* wout = dn_dyn + static_cast<size_t>(w) * NGW * P * 64;
  char* const stage = reinterpret_cast<char*>(dn_dyn + static_cast<size_t>(W) * NGW * P * 64);
  const ALds al{stage + 16 * o};
  const StageGeom sg = stage_geom(m.h + static_cast<size_t>(rlo) * m.F, rhi - rlo, m.F, 0, ntf);
  auto epi = [&](int gi, f32x4 (&acc)[P][2]) { stash<P>(wout, gi, acc); };
  auto epi_add = [&](int gi, f32x4 (&acc)[P][2]) { stash_add<P>(wout, gi, acc); };
  const int nrow = m.T * m.k + m.T;
  auto finish = [&]() {
    if constexpr (KS) __syncthreads();  // every wave's partial sums parked
    for (int gi = KS ? w : 0; gi < ng; gi += KS ? W : 1) {
      int e, q;
      item(gi, e, q);
      const int me = min(G.cnt[e], 16), base = G.base[e];
      const float gd = G.gs0[e];
      float wp[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wp[r] = G.fac[min(base + 4 * o + r, nrow - 1)];
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int pi = q * P + p;
        f32x4 v = wout[(gi * P + p) * 64 + lane];
        if constexpr (KS) {
          v = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int u = 0; u < W; ++u) v += dn_dyn[(static_cast<size_t>(u) * NGW + gi) * P * 64 + p * 64 + lane];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 4 * o + r;
          if (pi < npan && row < me) {
            const int sl = G.slot[base + row];  // the row's (token, slot); -1: the shared expert, slot k
            const size_t orow = static_cast<size_t>(G.tok[base + row]) * (m.k + 1) + (sl < 0 ? m.k : sl);
            m.o[orow * m.D + pi * 16 + c] = wp[r] * (gd * v[r]);
          }
        }
      }
    }
    if constexpr (KS) __syncthreads();  // the stash is free for the next chunk
    c0 += NGW;
  };
  // the two ways of reaching the activations; the first chunk's stream
  // (entered by every wave, possibly with no item, so that all reach the
  // staging barrier) stages the rows; it is a separate instance so that the
  // staging and its wait are unconditional and the later streams' waits know
  // the staging has landed
  auto run = [&](auto mode) {
    constexpr int AM = decltype(mode)::value;
    constexpr int DD = AM == kAStagedRows ? DP : DPG;
    auto group = [&](int gi, GroupPtrs<P>& gp) {
      prio_by_items_left(ntot - c0 - gi);
      int e, q;
      item(gi, e, q);
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int pi = min(q * P + p, npan - 1);
        gp.panel[p] = m.down + static_cast<size_t>(e) * m.down_stride + static_cast<size_t>(pi) * m.down_panel_bytes;
      }
      const int me = min(G.cnt[e], 16);
      if constexpr (AM == kAStagedRows) {
        gp.alds = static_cast<unsigned>(G.base[e] + min(c, me - 1) - rlo) * hrs + static_cast<unsigned>(kt0) * 256u;
      } else {
        gp.arsrc = hr;
        gp.aoff = c < me ? static_cast<unsigned>(G.base[e] + c) * static_cast<unsigned>(m.F) * 2u : kDeadLane;
      }
    };
    auto stage_pre_issue = [&] {
      if constexpr (AM == kAStagedRows) stage_issue(sg, reinterpret_cast<u32x4*>(stage));
    };
    auto stage_pre = [&] {
      if constexpr (AM == kAStagedRows) stage_wait<DD * P * 2>();  // the prologue's D tiles of P panels
    };
    auto none = [] {};
    ng = min(NGW, ntot);
    stream_groups<kNvfp4, P, DD, AM, true>(ng, krg, kt0, half ? nfull : -1, al, ARing{}, m.F, group,
                                           stage_pre_issue, stage_pre, epi, epi_add);
    finish();
    while (c0 < ntot) {
      ng = min(NGW, ntot - c0);
      stream_groups<kNvfp4, P, DD, AM, true>(ng, krg, kt0, half ? nfull : -1, al, ARing{}, m.F, group, none, none,
                                             epi, epi_add);
      finish();
    }
  };
  if (staged)
    run(std::integral_constant<int, kAStagedRows>{});
  else
    run(std::integral_constant<int, kAGlobal>{});
}

// ------------------------------------------------------------------ combine

// y[t][n] = sum_{s<k} o[t][s][n] (+ o[t][k][n] for the shared expert), slots
// in order; a slot whose pair has no row (an index outside 0..E-1, or past an
// expert's 16th) adds nothing.  Four columns per thread; the row map and the
// outputs are loaded together (the output rows are at fixed places).
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs m) {
  const int t = blockIdx.x;
  const int n = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (n >= m.D) return;
  const float* ot = m.o + static_cast<size_t>(t) * (m.k + 1) * m.D + n;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < m.k; s0 += 8) {  // 8 slots' rows in flight, summed in slot order
    f32x4 v[8];
    int pos[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sl = min(s0 + u, m.k - 1);
      pos[u] = s0 + u < m.k ? m.rowof[t * m.k + sl] : -1;
      v[u] = *reinterpret_cast<const f32x4*>(ot + static_cast<size_t>(sl) * m.D);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (pos[u] >= 0) acc += v[u];
  }
  if (m.has_shared) acc += *reinterpret_cast<const f32x4*>(ot + static_cast<size_t>(m.k) * m.D);
  if (m.out_dtype == Q4_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(m.y) + static_cast<size_t>(t) * m.D + n) = acc;
  } else {
    const f16x2 h0 = {(f16)acc[0], (f16)acc[1]}, h1 = {(f16)acc[2], (f16)acc[3]};
    *reinterpret_cast<u32x2*>(static_cast<f16*>(m.y) + static_cast<size_t>(t) * m.D + n) =
        u32x2{__builtin_bit_cast(unsigned, h0), __builtin_bit_cast(unsigned, h1)};
  }
}

// Scratch of moe_grouped_qgemm_noalloc: one array per device, in the code
// object, so that the entry point needs no allocation.  Host code never uses
// its name as an address (on the host it is only a stand-in): the device
// address comes from hipGetSymbolAddress, once per device.
constexpr size_t kMoeScratchBytes = size_t(8) << 20;
__device__ __align__(256) unsigned char scratch[kMoeScratchBytes];

}  // namespace

int moe_noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices) return static_cast<int>(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) {
      (void)hipGetLastError();
      return static_cast<int>(e);
    }
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kMoeScratchBytes;
  return 0;
}

int launch_route(const RouteArgs& r, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const size_t need = route_lds_bytes(r.D);
  if (int e = ensure_dynamic_lds(reinterpret_cast<const void*>(&route_kernel), need)) return e;
  hipLaunchKernelGGL(route_kernel, dim3(route_eblocks(r.E) * r.nsplit), dim3(kRouteThreads), need, s, r);
  return static_cast<int>(hipGetLastError());
}

namespace {
constexpr int GU_W = 8, DN_P = 2, DN_W = 8, kWG = 256;  // one 8-wave workgroup per CU
// down for a lone layer (item per wave): 16 waves per workgroup, its
// unstaged path 1 tile deep (measured 24.8 us against 25.8 for the 128 + 1
// expert layer)
constexpr int DN_W1 = 16;

// Shapes of one layer's two launches.
struct MoeShape {
  int nact_max;  // experts that can be active: one per routed pair at most, plus the shared one
  int npp, ngp;  // gate/up items (panel pairs) and down items (groups of DN_P panels) per expert
  int ntx, ntf;  // K tiles of gate/up (K = D) and of down (K = F)
};
MoeShape moe_shape(const MoeArgs& m) {
  MoeShape h;
  h.nact_max = std::min(m.E, m.T * m.k) + m.has_shared;
  h.npp = m.F / 16;
  h.ngp = (m.D / 16 + DN_P - 1) / DN_P;
  h.ntx = static_cast<int>(full_tiles(m.D) + (has_half_tile(m.D) ? 1 : 0));
  h.ntf = static_cast<int>(full_tiles(m.F) + (has_half_tile(m.F) ? 1 : 0));
  return h;
}
// workgroups of kWG for the first of two layers, in proportion to their
// tile-items (at least one each), with every expert of the first active
int split_of(int64_t w0, int64_t w1) {
  const int64_t s = (kWG * w0 + (w0 + w1) / 2) / (w0 + w1);
  return static_cast<int>(std::min<int64_t>(kWG - 1, std::max<int64_t>(1, s)));
}

template <int AM, bool KS, bool TWO>
int launch_gu(const MoeLayers& L, int u0, int w1, int ngw0, int ngw1, size_t lds, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&moe_gate_up_kernel<GU_W, 4, AM, KS, TWO>);
  if (int e = ensure_dynamic_lds(fn, lds)) return e;
  hipLaunchKernelGGL((moe_gate_up_kernel<GU_W, 4, AM, KS, TWO>), dim3(kWG), dim3(64 * GU_W), lds, s, L, u0, w1, ngw0,
                     ngw1);
  return static_cast<int>(hipGetLastError());
}
template <int W, bool KS, bool TWO, int DPG>
int launch_dn(const MoeLayers& L, int u0, int w1, int ngw0, int ngw1, size_t lds, hipStream_t s) {
  const void* fn = reinterpret_cast<const void*>(&moe_down_kernel<DN_P, W, 4, KS, TWO, DPG>);
  if (int e = ensure_dynamic_lds(fn, lds)) return e;
  hipLaunchKernelGGL((moe_down_kernel<DN_P, W, 4, KS, TWO, DPG>), dim3(kWG), dim3(64 * W), lds, s, L, u0, w1, ngw0,
                     ngw1, static_cast<int>(lds));
  return static_cast<int>(hipGetLastError());
}
}  // namespace

// Whether the routed gate/up prologue's LDS (moe_route_lds) fits beside the
// staged x and the grouping table, as launch_moe lays them out.
bool moe_gu_route_fits(int T, int D, int E) {
  const size_t lds_total = 160 * 1024;
  const int ntx = static_cast<int>(full_tiles(D) + (has_half_tile(D) ? 1 : 0));
  const size_t xbytes = (static_cast<size_t>(stage_bytes(T, ntx)) + 15) / 16 * 16;
  const size_t slot = static_cast<size_t>(GU_W) * 2 * 64 * 16;
  const size_t fixed = sizeof(MoeGroups) + xbytes;
  const bool staged = lds_total > fixed && lds_total - fixed >= slot;
  const size_t need = sizeof(MoeGroups) + (staged ? xbytes : 0) + std::max(slot, moe_route_lds(T, E));
  return E % 4 == 0 && E <= 256 && need <= lds_total;
}

// One layer (m1 NULL), or two layers sharing each launch (m1: the MoE
// block's dense branch, which has the experts' T and D); no combine launch
// with two.
int launch_moe(const MoeArgs& m0, const MoeArgs* m1, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool two = m1 != nullptr;
  const MoeArgs& mb = two ? *m1 : m0;
  const MoeShape h0 = moe_shape(m0), h1 = moe_shape(mb);
  // workgroups per layer: all of them for one layer
  const int gu_split = two ? split_of(int64_t(h0.nact_max) * h0.npp * h0.ntx, int64_t(h1.nact_max) * h1.npp * h1.ntx)
                           : kWG;
  const int dn_split = two ? split_of(int64_t(h0.nact_max) * h0.ngp * h0.ntf, int64_t(h1.nact_max) * h1.ngp * h1.ntf)
                           : kWG;
  // K split over a workgroup's waves when a lone layer has too few items to
  // give every CU's waves one each (at least one K tile per wave)
  const bool gu_ks = !two && h0.nact_max * h0.npp <= 2 * kWG && h0.ntx >= GU_W;
  const bool dn_ks = !two && h0.nact_max * h0.ngp <= 2 * kWG && h0.ntf >= DN_W;
  // stash slots per wave (items parked until the wave's stream ends): as many
  // as a wave has items at most, up to what 96 KiB of LDS holds; a wave with
  // more items streams them in chunks of that many
  constexpr size_t kStashLds = 96 * 1024;
  auto need = [](int items, int units) { return (items + units - 1) / units; };
  const int gu_cap = static_cast<int>(kStashLds / (size_t(GU_W) * 2 * 64 * 16));
  int gu_need0, gu_need1 = 1;
  if (gu_ks) {
    gu_need0 = need(h0.nact_max * h0.npp, kWG);
  } else {
    // (with two layers the device gives the first layer about kWG w0 / (w0 +
    // w1) workgroups for its w0 actual tile-items, so that a wave of it has
    // at most about (w0 + w1) / (kWG W) tile-items, w0 at its largest; the
    // second layer has the fewest workgroups when all experts are active)
    gu_need0 = two ? need((h0.nact_max * h0.npp * h0.ntx + h1.nact_max * h1.npp * h1.ntx) / h0.ntx, kWG * GU_W) + 1
                   : need(h0.nact_max * h0.npp, gu_split * GU_W);
    if (two) gu_need1 = need(h1.nact_max * h1.npp, (kWG - gu_split) * GU_W) + 1;
  }
  int gu_ngw0 = std::min(gu_need0, gu_cap), gu_ngw1 = std::min(gu_need1, gu_cap);
  size_t gu_lds = static_cast<size_t>(GU_W) * std::max(gu_ngw0, gu_ngw1) * 2 * 64 * 16;
  // gate/up stages x in LDS when it fits beside the grouping table and a
  // stash of at least one item per wave (a wave with more items than slots
  // streams them in chunks); with the K split each wave reads only its range
  // of x, from global memory
  const size_t xbytes = (static_cast<size_t>(stage_bytes(std::max(m0.T, mb.T), std::max(h0.ntx, h1.ntx))) + 15) /
                        16 * 16;
  const size_t lds_total = 160 * 1024;
  const size_t slot = static_cast<size_t>(GU_W) * 2 * 64 * 16;
  const size_t room = lds_total > sizeof(MoeGroups) + xbytes ? lds_total - sizeof(MoeGroups) - xbytes : 0;
  const bool gu_staged = !gu_ks && room >= slot;
  if (gu_staged) {
    gu_ngw0 = std::min(gu_need0, static_cast<int>(room / slot));
    gu_ngw1 = std::min(gu_need1, static_cast<int>(room / slot));
    gu_lds = xbytes + static_cast<size_t>(std::max(gu_ngw0, gu_ngw1)) * slot;
  }
  // the routed prologue borrows the start of the stash for the logits and
  // the scale vectors
  if (m0.rpart) {
    const size_t need_r = (gu_staged ? xbytes : 0) + moe_route_lds(m0.T, m0.E);
    if (need_r > gu_lds) gu_lds = need_r;
    if (sizeof(MoeGroups) + gu_lds > lds_total) return static_cast<int>(hipErrorInvalidConfiguration);
  }
  // waves per down workgroup; the 16-wave lone-layer kernel parks at most 2
  // items per wave (64 KiB), leaving room to stage the rows of two experts
  const int dn_w = (two || dn_ks) ? DN_W : DN_W1;
  const size_t dn_stash_max = (two || dn_ks) ? kStashLds : 64 * 1024;
  const int dn_cap = static_cast<int>(dn_stash_max / (size_t(dn_w) * DN_P * 64 * 16));
  int dn_need0, dn_need1 = 1;
  if (dn_ks) {
    dn_need0 = need(h0.nact_max * h0.ngp, kWG);
  } else {
    dn_need0 = two ? need((h0.nact_max * h0.ngp * h0.ntf + h1.nact_max * h1.ngp * h1.ntf) / h0.ntf, kWG * dn_w) + 1
                   : need(h0.nact_max * h0.ngp, dn_split * dn_w);
    if (two) dn_need1 = need(h1.nact_max * h1.ngp, (kWG - dn_split) * dn_w) + 1;
  }
  const int dn_ngw0 = std::min(dn_need0, dn_cap), dn_ngw1 = std::min(dn_need1, dn_cap);
  // the CU's LDS past the table: each role's stash, then its workgroup's
  // staged h rows (a workgroup whose rows do not fit reads them from global
  // memory)
  const size_t dn_fixed = sizeof(MoeDownTable) + 512;  // the table and the kernel's other static LDS
  const size_t dn_lds = 160 * 1024 - dn_fixed;
  if (gu_ngw0 < 1 || gu_ngw1 < 1 || dn_ngw0 < 1 || dn_ngw1 < 1) return static_cast<int>(hipErrorInvalidConfiguration);
  MoeLayers L;
  L.l[0] = m0;
  L.l[1] = mb;
  // the two-layer split is taken on the device from the first layer's
  // active experts: tile-items per active expert, and the second layer's
  const int gu_u0 = h0.npp * h0.ntx, gu_w1 = h1.nact_max * h1.npp * h1.ntx;
  const int dn_u0 = h0.ngp * h0.ntf, dn_w1 = h1.nact_max * h1.ngp * h1.ntf;
  int e;
  if (gu_ks)
    e = launch_gu<kAGlobal, true, false>(L, gu_u0, gu_w1, gu_ngw0, gu_ngw1, gu_lds, s);
  else if (two)
    e = gu_staged ? launch_gu<kAStagedRows, false, true>(L, gu_u0, gu_w1, gu_ngw0, gu_ngw1, gu_lds, s)
                  : launch_gu<kAGlobal, false, true>(L, gu_u0, gu_w1, gu_ngw0, gu_ngw1, gu_lds, s);
  else
    e = gu_staged ? launch_gu<kAStagedRows, false, false>(L, gu_u0, gu_w1, gu_ngw0, gu_ngw1, gu_lds, s)
                  : launch_gu<kAGlobal, false, false>(L, gu_u0, gu_w1, gu_ngw0, gu_ngw1, gu_lds, s);
  if (e) return e;
  if (dn_ks)
    e = launch_dn<DN_W, true, false, 4>(L, dn_u0, dn_w1, dn_ngw0, dn_ngw1, dn_lds, s);
  else if (two)
    e = launch_dn<DN_W, false, true, 4>(L, dn_u0, dn_w1, dn_ngw0, dn_ngw1, dn_lds, s);
  else
    e = launch_dn<DN_W1, false, false, 1>(L, dn_u0, dn_w1, dn_ngw0, dn_ngw1, dn_lds, s);
  if (e) return e;
  if (two || !m0.combine) return 0;
  hipLaunchKernelGGL(moe_combine_kernel, dim3(m0.T, (m0.D / 4 + 255) / 256), dim3(256), 0, s, m0);
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
