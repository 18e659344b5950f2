// Private declarations shared by the host code and the HIP kernels of libq4mi.
//
// Packed weight geometry (both formats).  A "panel" is 16 consecutive output
// rows n; it is stored as a run of tiles along K:
//   full tile (128 k): 1024 B of codes, 64 lanes x 16 B, then 128 B of scales
//   half tile  (64 k):  512 B of codes, 64 lanes x  8 B, then  64 B of scales
// Lane l of a wave owns column c = l & 15 and k-octet o = l >> 4; its code
// dword i holds the 8 codes at k = kb + 32 i + 8 o + (0..7), which is the
// B-operand slice of MFMA step i of v_mfma_f32_16x16x32_{f16,bf16} (lane l:
// column l & 15, k = 8 (l >> 4) + 0..7 of the step's 32).  The A operand of
// step i is therefore a[m][kb + 32 i + 8 o + 0..7] for row m = l & 15.
#pragma once
#include <stddef.h>
#include <stdint.h>

#if defined(__HIPCC__)
#define Q4_HD __host__ __device__
#else
#define Q4_HD
#endif

namespace q4mi {

constexpr int kTileK = 128;
constexpr int kTileBytes = 1152;
constexpr int kTileCodeBytes = 1024;
constexpr int kHalfBytes = 576;
constexpr int kHalfCodeBytes = 512;

// K padded to the 64-k granularity of the packed layout
Q4_HD inline int64_t padded_k(int64_t K) { return (K + 63) / 64 * 64; }
Q4_HD inline int64_t full_tiles(int64_t K) { return padded_k(K) / kTileK; }
Q4_HD inline bool has_half_tile(int64_t K) { return padded_k(K) % kTileK != 0; }
Q4_HD inline int64_t panel_bytes(int64_t K) {
  return full_tiles(K) * kTileBytes + (has_half_tile(K) ? kHalfBytes : 0);
}
// Zero guard behind the last panel when panels end in a half tile: a kernel
// may issue a full-tile load at a half tile (and never use its second half),
// which then stays inside the buffer.
Q4_HD inline int64_t packed_tail(int64_t K) { return has_half_tile(K) ? kTileBytes - kHalfBytes : 0; }
Q4_HD inline int64_t packed_matrix_bytes(int64_t N, int64_t K) { return N / 16 * panel_bytes(K) + packed_tail(K); }

enum Fmt { kNvfp4 = 0, kAffine = 1 };
// kAffineBits + b: the b-bit affine widths (b = 2, 3, 5, 6, 8); tiles of
// 256 b code bytes and 128 scale/bias bytes, K padded to whole tiles
constexpr int kAffineBits = 16;

// Workspace layout shared by every entry point, so that one zero-filled
// buffer can serve all of them: the first kWsCounterBytes hold only counters
// and keys that each call returns to zero; scratch (partial sums, h, o)
// starts at kWsCounterBytes.
constexpr size_t kWsCounterBytes = 32768;
constexpr size_t kWsRouteCounter = 0;        // u32: router arrival counter
constexpr size_t kWsArgmaxCounter = 64;      // u32: GEMM argmax completion counter
constexpr size_t kWsArgmaxKeys = 128;        // u64[16]: GEMM argmax keys
constexpr size_t kWsBlockCounters = 1024;    // u32[]: GEMM split-K arrival counters
constexpr int kMaxSplitBlocks = static_cast<int>((kWsCounterBytes - kWsBlockCounters) / 4);

struct GemmArgs {
  const uint8_t* w;          // packed weights
  int64_t panel_bytes;       // bytes per 16-row panel
  const uint16_t* a;         // activations [M][K] (f16 or bf16 bits)
  int M, K, N;
  int nfull;                 // full tiles in the packed layout
  int half;                  // 1 if a half tile follows the full ones
  int k_exact;               // 1 if every packed k < K (K % 64 == 0)
  float gscale;              // NVFP4 global scale (1 for affine)
  void* out;
  int out_dtype;
  int32_t* argmax;           // nullable
  unsigned* counter;         // argmax workspace: completion counter
  unsigned long long* keys;  // argmax workspace: per-row packed (value, index) keys
  // fused sampling (qgemm_nvfp4_sample): z = softcap(g acc) is what gets
  // stored (out may be null) and the row keys rank z / T + Gumbel noise, or
  // z itself for T = 0, in fp32
  int sample;
  float softcap;             // > 0: z = softcap tanh(y / softcap)
  float inv_temp;            // 1 / T, 0 for greedy
  unsigned seed_lo, seed_hi, offset;
};

struct GemmCfg {
  int P;   // panels per wave group
  int W;   // waves per workgroup
  int D;   // tiles of weight loads in flight per wave
  int KS;  // k-ranges (workgroups sharing a panel block; partials reduced in order)
  int KW;  // waves splitting a workgroup's k-range (LDS reduction, one group per wave)
  int PB;  // panels per workgroup block
  int RING;  // 1: each wave moves its own tiles' activations into an LDS ring (one group per wave, K % 64 == 0)
};

// Let kernel `fn` use `bytes` of dynamic LDS on the current device: raises the
// function's limit when this is more than was set before on that device, and
// never lowers it, so concurrent callers with different needs cannot undo
// each other.  Thread-safe; returns hipError_t as int.
int ensure_dynamic_lds(const void* fn, size_t bytes);

// kernel launchers (q4mi_gemm.hip); return hipError_t as int
GemmCfg choose_gemm_cfg(int fmt, int M, int64_t K, int64_t N);
size_t gemm_workspace(int fmt, int M, int64_t K, int64_t N);
int launch_gemm(int fmt, const GemmArgs& g, const GemmCfg& cfg, void* ws, void* stream);
int launch_dequant(int fmt, const uint8_t* w, int64_t panel_bytes, int64_t N, int64_t K, float g,
                   float* out, void* stream);
int launch_sample_uniforms(unsigned seed_lo, unsigned seed_hi, unsigned offset, int M, int64_t N, float* out,
                           void* stream);
// NVFP4 GEMM for M > 16 rows (q4mi_prefill.hip); uses w, panel_bytes, a, M, K,
// N, nfull, half, gscale, out, out_dtype of the arguments
int launch_prefill(const GemmArgs& g, void* stream);
// MoE block norms, router normalization and combine (q4mi_block.hip)
int launch_block_norm_in(const float* res, int T, int D, const float* w1, const float* w2, float eps, void* h1,
                         void* h2, void* stream);
// o1: the dense branch's outputs [T][2][D] (slot 0), o2 and rowof2 the
// experts' [T][k + 1][D] and [T][k] (grouped-MoE scratch layout)
int launch_block_combine(const float* o1, const float* o2, const int32_t* rowof2, int k, int T, int D,
                         const float* p1, const float* p2, const float* p, float eps, float* res, void* stream);
// affine 2/3/5/6/8-bit skinny GEMM (q4mi_affineb.hip)
int launch_affine_bits(int bits, const uint8_t* w, int64_t N, int64_t K, const uint16_t* a, int M, void* out,
                       int out_dtype, void* stream);
// stream-read ceiling (q4mi_ceiling.hip): bytes % 16 == 0, out[grid], depth in {1, 2, 4, 8}
int launch_stream_read(const void* src, size_t bytes, int grid, int mode, int depth, unsigned* out, void* stream);
// NVFP4 quantizer (q4mi_quant.hip); amax: one scratch word of the workspace
int launch_quantize(const float* w, int64_t N, int64_t K, float g_in, unsigned* amax, uint8_t* packed, float* g_out,
                    void* stream);

// Router grid: (16-expert column blocks) x (splits of D), workgroups of
// kRouteThreads threads (4 waves).  A workgroup computes the logits of its
// 16 experts for every token over its rows of D; its waves split those rows
// (a multiple of 16 each) and their partial sums are added in LDS in wave
// order.  The last workgroup to finish adds the D-splits' partial logits in
// split order and takes the top-k.
constexpr int kRouteThreads = 256;
constexpr int kRouteMaxSplits = 8;
constexpr int kRouteMaxRows = 1536;  // rows of D per workgroup (staged x: 96 KiB)
Q4_HD inline int route_eblocks(int E) { return (E + 15) / 16; }
Q4_HD inline int route_splits(int D) {
  const int s = (D + 255) / 256;
  return s < 1 ? 1 : (s > kRouteMaxSplits ? kRouteMaxSplits : s);
}
Q4_HD inline int route_rows(int D) {  // rows per split: a multiple of 64 (16 per wave)
  const int s = route_splits(D);
  return ((D + s - 1) / s + 63) / 64 * 64;
}
// staged x [rows][16] fp32, reused by the last workgroup for the logits
// [T][E] (T <= 64, E <= 256: at most 64 KiB); then the waves' partial sums
Q4_HD inline size_t route_lds_bytes(int D) {
  const size_t xs = static_cast<size_t>(route_rows(D)) * 64;
  return (xs < 65536 ? 65536 : xs) + 4096;
}

struct RouteArgs {
  const uint16_t* x;    // f16 [T][D]
  const float* wr;      // [D][E]
  int T, D, E, k, renormalize;
  float* logits;        // nullable [T][E]
  int32_t* idx;         // [T][k]
  float* w;             // [T][k]
  // The MoE block's routing (zscale non-NULL): the top-k and softmax are
  // taken over z = RMSNorm(logits; unit weights, eps) * zscale, the weights
  // multiplied by down_scale[idx] (when non-NULL), and the dense branch's
  // one-expert routing (expert 0, weight 1) written to didx, dw
  const float* zscale;
  const float* down_scale;
  float eps;
  int32_t* didx;
  float* dw;
  float* partial;       // workspace [splits][T][E]
  unsigned* counter;    // workspace counter
  int nsplit;           // splits of D
  int rows;             // rows of D per split (a multiple of 64)
  int partials_only;    // 1: write the partial logits and stop (the gate/up launch routes from them)
};
int launch_route(const RouteArgs& r, void* stream);

struct MoeArgs {
  int E, has_shared, D, F, T, k;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  int64_t gate_stride, down_stride;      // bytes per expert matrix
  int64_t gate_panel_bytes, down_panel_bytes;
  const float* g_gate;
  const float* g_up;
  const float* g_down;
  const uint16_t* x;       // f16 [T][D]
  const int32_t* idx;      // [T][k]
  const float* tw;         // [T][k]
  void* y;
  int out_dtype;
  uint16_t* h;             // workspace f16 [npairs][F], expert-sorted rows
  float* o;                // workspace fp32 [T][k + 1][D]: token t's slot s output (slot k: shared expert)
  int32_t* rowof;          // workspace [T * k]: pair -> scratch row (-1: none)
  int32_t* grp;            // workspace: the expert grouping, written by gate/up, read by down
  int combine;             // 1: a third launch sums each token's slots into y
  // Routing inside gate/up (rpart non-NULL; idx unused): every workgroup
  // sums the router's partial logits [rsplit][T][E] in split order (E % 4
  // == 0) and takes the top-k and softmax itself, over z = RMSNorm(logits;
  // eps) * zscale when zscale is non-NULL, the weights times down_scale[e]
  // when that is non-NULL and renormalized over the k when renorm; the
  // publishing workgroup writes them to ridx / rtw (tw must be rtw, for
  // down) and the summed logits to rlogits when non-NULL.  rconst: the
  // one-expert routing (expert 0, weight 1, k = 1) with no router, written
  // to ridx / rtw the same way.
  const float* rpart;
  int rsplit, renorm, rconst;
  const float* zscale;
  const float* down_scale;
  float eps;
  int32_t* ridx;
  float* rtw;
  float* rlogits;
};
// LDS the routed gate/up prologue borrows from the stash: the logits [T][E]
// and the scale vectors [E] each (bytes)
inline size_t moe_route_lds(int T, int E) { return (static_cast<size_t>(T) * E + 2 * static_cast<size_t>(E)) * 4; }
// The layers of one grouped launch (the second only for two-layer launches).
struct MoeLayers {
  MoeArgs l[2];
};
// the grouping table in the workspace (int32 words): nact, then act, cnt and
// base [E + 1] each, then tok and slot as int16 [T k + T] each
inline size_t moe_grp_words(int E, int T, int k) {
  return 4 + 3 * (static_cast<size_t>(E) + 1) + static_cast<size_t>(T) * (k + 1);
}
// One layer (m1 NULL: gate/up, down and, if m0.combine, the combine), or
// two layers of equal T and D sharing the gate/up and the down launch (no
// combine): the MoE block's experts (m0) and dense branch (m1).
int launch_moe(const MoeArgs& m0, const MoeArgs* m1, void* stream);
// whether a layer of T tokens, D and E experts can route inside gate/up
bool moe_gu_route_fits(int T, int D, int E);
// The per-device scratch array of moe_grouped_qgemm_noalloc (q4mi_moe.hip):
// its device address on the current device (looked up once per device) and
// its size.  Returns hipError_t as int.
constexpr int kMaxDevices = 64;
int moe_noalloc_scratch(void** ptr, size_t* bytes);

}  // namespace q4mi
