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
constexpr int kRouteChunk = 64;   // rows of W_r staged per pass
constexpr int kRouteTG = 8;       // tokens per thread item

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs r) {
  const int T = r.T, D = r.D, E = r.E;
  const int tid = threadIdx.x;
  const int rows = (D + r.nblk - 1) / r.nblk;
  const int d0 = blockIdx.x * rows;
  const int d1 = min(D, d0 + rows);
  const int ntg = (T + kRouteTG - 1) / kRouteTG;
  const int nitems = E * ntg;

  __shared__ float xs[64][kRouteChunk];  // [token][row in chunk]
  float acc[2][kRouteTG];                // 2 items per thread: host limits roundup(T, 8) * E to 4096
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < kRouteTG; ++t) acc[i][t] = 0.f;

  for (int c0 = d0; c0 < d1; c0 += kRouteChunk) {
    const int cn = min(kRouteChunk, d1 - c0);
    __syncthreads();
    for (int q = tid; q < T * kRouteChunk; q += kRouteThreads) {
      const int t = q / kRouteChunk, dd = q % kRouteChunk;
      xs[t][dd] = dd < cn ? (float)reinterpret_cast<const _Float16*>(r.x)[static_cast<size_t>(t) * D + c0 + dd] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int item = tid + i * kRouteThreads;
      if (item < nitems) {
        const int e = item % E, tg = item / E;
        for (int dd = 0; dd < cn; ++dd) {
          const float w = r.wr[static_cast<size_t>(c0 + dd) * E + e];
#pragma unroll
          for (int t = 0; t < kRouteTG; ++t) {
            const int tt = tg * kRouteTG + t;
            if (tt < T) acc[i][t] = fmaf(xs[tt][dd], w, acc[i][t]);
          }
        }
      }
    }
  }
  // partial logits of this row block
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int item = tid + i * kRouteThreads;
    if (item < nitems) {
      const int e = item % E, tg = item / E;
#pragma unroll
      for (int t = 0; t < kRouteTG; ++t) {
        const int tt = tg * kRouteTG + t;
        if (tt < T) r.partial[(static_cast<size_t>(blockIdx.x) * T + tt) * E + e] = acc[i][t];
      }
    }
  }
  __threadfence();
  __syncthreads();
  __shared__ int s_last;
  if (tid == 0) s_last = atomicAdd(r.counter, 1u) == gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();

  // last workgroup: fixed-order sum of the partials, softmax, top-k
  __shared__ float lg[4096];
  for (int q = tid; q < T * E; q += kRouteThreads) {
    float s = 0.f;
    for (int b = 0; b < static_cast<int>(gridDim.x); ++b)
      s += __builtin_nontemporal_load(r.partial + static_cast<size_t>(b) * T * E + q);
    lg[q] = s;
    if (r.logits) r.logits[q] = s;
  }
  __syncthreads();
  const int lane = tid & 63, wv = tid >> 6;
  for (int t = wv; t < T; t += kRouteThreads / 64) {
    const float* l = lg + t * E;
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
  const int n = T * k;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    const int v = j < n ? idx[j] : -1;
    const bool valid = v >= 0 && v < E;
    const unsigned long long eq = __ballot(valid && v == e);
    const unsigned long long lt = __ballot(valid && v < e);
    if (valid && v == e) {
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

template <int KW, int PW, int DP>
__global__ __launch_bounds__(64 * KW * PW) void moe_gate_up_kernel(MoeArgs m) {
  const int e = blockIdx.y;
  __shared__ int s_tok[16], s_slot[16], s_meta[2];
  if (threadIdx.x < 64) group_expert(m.idx, m.T, m.k, m.E, e, s_tok, s_slot, s_meta);
  __syncthreads();
  const int me = s_meta[0];
  if (me == 0) return;
  const int base = s_meta[1];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = wid % KW, pw = wid / KW;
  const int o = lane >> 4, c = lane & 15;
  const int npp = m.F / 16;                       // panel pairs
  const int jp = blockIdx.x * PW + pw;            // this wave's panel pair
  const int jc = jp < npp ? jp : npp - 1;         // clamped for loads
  const uint8_t* pbase[2] = {
      m.gate + static_cast<size_t>(e) * m.gate_stride + static_cast<size_t>(jc) * m.gate_panel_bytes,
      m.up + static_cast<size_t>(e) * m.gate_stride + static_cast<size_t>(jc) * m.gate_panel_bytes};
  const bool arow_ok = c < me;
  const uint16_t* arow = m.x + static_cast<size_t>(arow_ok ? s_tok[c] : 0) * m.D;

  const KSplit ks = ksplit(m.D);
  const int per = (ks.nmain + KW - 1) / KW;
  const int t0 = kw * per;
  const int nt = max(0, min(ks.nmain, t0 + per) - t0);
  f32x4 acc[2][2];
  acc[0][0] = acc[0][1] = acc[1][0] = acc[1][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  wave_accumulate<kNvfp4, 2, DP>(acc, pbase, arow, arow_ok, m.D, t0, nt, kw == KW - 1 ? ks.tail : 0, ks.nmain);
  f32x4 rg = acc[0][0] + acc[0][1], ru = acc[1][0] + acc[1][1];
  if constexpr (KW > 1) {
    __shared__ float red[KW][PW][2][4][64];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      red[kw][pw][0][r][lane] = rg[r];
      red[kw][pw][1][r][lane] = ru[r];
    }
    __syncthreads();
    if (kw != 0) return;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sg = 0.f, su = 0.f;
#pragma unroll
      for (int j = 0; j < KW; ++j) {
        sg += red[j][pw][0][r][lane];
        su += red[j][pw][1][r][lane];
      }
      rg[r] = sg;
      ru[r] = su;
    }
  }
  if (jp >= npp) return;
  const float gg = m.g_gate[e], gu = m.g_up[e];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * o + r;
    if (row < me) {
      const float h = gelu_tanh(gg * rg[r]) * (gu * ru[r]);
      reinterpret_cast<_Float16*>(m.h)[static_cast<size_t>(base + row) * m.F + jp * 16 + c] = (_Float16)h;
    }
  }
}

// ------------------------------------------------------------------ down

template <int P, int PW, int DP>
__global__ __launch_bounds__(64 * PW) void moe_down_kernel(MoeArgs m) {
  const int e = blockIdx.y;
  __shared__ int s_tok[16], s_slot[16], s_meta[2];
  if (threadIdx.x < 64) group_expert(m.idx, m.T, m.k, m.E, e, s_tok, s_slot, s_meta);
  __syncthreads();
  const int me = s_meta[0];
  if (me == 0) return;
  const int base = s_meta[1];

  const int lane = threadIdx.x & 63;
  const int pw = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int o = lane >> 4, c = lane & 15;
  const int npan = m.D / 16;
  const int panel0 = (blockIdx.x * PW + pw) * P;
  const uint8_t* pbase[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int pi = min(panel0 + p, npan - 1);
    pbase[p] = m.down + static_cast<size_t>(e) * m.down_stride + static_cast<size_t>(pi) * m.down_panel_bytes;
  }
  const bool arow_ok = c < me;
  const uint16_t* arow = m.h + static_cast<size_t>(base + (arow_ok ? c : 0)) * m.F;
  const KSplit ks = ksplit(m.F);
  f32x4 acc[P][2];
#pragma unroll
  for (int p = 0; p < P; ++p) acc[p][0] = acc[p][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  wave_accumulate<kNvfp4, P, DP>(acc, pbase, arow, arow_ok, m.F, 0, ks.nmain, ks.tail, ks.nmain);

  const float gd = m.g_down[e];
  float wrow[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = 4 * o + r;
    wrow[r] = 0.f;
    if (row < me) wrow[r] = s_slot[row] < 0 ? 1.0f : m.tw[s_tok[row] * m.k + s_slot[row]];
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int pi = panel0 + p;
    if (pi >= npan) continue;
    const f32x4 v = acc[p][0] + acc[p][1];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * o + r;
      if (row < me) m.o[static_cast<size_t>(base + row) * m.D + pi * 16 + c] = wrow[r] * (gd * v[r]);
    }
  }
}

// ------------------------------------------------------------------ combine

__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs m) {
  const int t = blockIdx.x;
  const int n = blockIdx.y * 256 + threadIdx.x;
  extern __shared__ int s_pos[];  // [k]
  const int nall = m.T * m.k;
  for (int s = threadIdx.x; s < m.k; s += 256) {
    const int e = m.idx[t * m.k + s];
    int pos = -1;
    if (e >= 0 && e < m.E) {
      int below = 0, rank = 0;
      for (int j = 0; j < nall; ++j) {
        const int v = m.idx[j];
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
  for (int s = 0; s < m.k; ++s) {
    const int pos = s_pos[s];
    if (pos >= 0) acc += m.o[static_cast<size_t>(pos) * m.D + n];
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
  hipLaunchKernelGGL(route_kernel, dim3(r.nblk), dim3(kRouteThreads), 0, s, r);
  return static_cast<int>(hipGetLastError());
}

int launch_moe(const MoeArgs& m, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int nexp = m.E + m.has_shared;
  constexpr int GU_KW = 2, GU_PW = 2, DN_P = 2, DN_PW = 4;
  const int npp = m.F / 16;
  hipLaunchKernelGGL((moe_gate_up_kernel<GU_KW, GU_PW, 4>), dim3((npp + GU_PW - 1) / GU_PW, nexp),
                     dim3(64 * GU_KW * GU_PW), 0, s, m);
  if (hipError_t e = hipGetLastError()) return static_cast<int>(e);
  const int npan = m.D / 16;
  hipLaunchKernelGGL((moe_down_kernel<DN_P, DN_PW, 4>), dim3((npan + DN_P * DN_PW - 1) / (DN_P * DN_PW), nexp),
                     dim3(64 * DN_PW), 0, s, m);
  if (hipError_t e = hipGetLastError()) return static_cast<int>(e);
  hipLaunchKernelGGL(moe_combine_kernel, dim3(m.T, (m.D + 255) / 256), dim3(256), m.k * sizeof(int), s, m);
  return static_cast<int>(hipGetLastError());
}

}  // namespace q4mi
