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

namespace q4mi {

constexpr int kTileK = 128;
constexpr int kTileBytes = 1152;
constexpr int kTileCodeBytes = 1024;
constexpr int kHalfBytes = 576;
constexpr int kHalfCodeBytes = 512;

// K padded to the 64-k granularity of the packed layout
inline int64_t padded_k(int64_t K) { return (K + 63) / 64 * 64; }
inline int64_t full_tiles(int64_t K) { return padded_k(K) / kTileK; }
inline bool has_half_tile(int64_t K) { return padded_k(K) % kTileK != 0; }
inline int64_t panel_bytes(int64_t K) {
  return full_tiles(K) * kTileBytes + (has_half_tile(K) ? kHalfBytes : 0);
}

enum Fmt { kNvfp4 = 0, kAffine = 1 };

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
};

struct GemmCfg {
  int P;   // panels per wave
  int KW;  // waves splitting K inside a workgroup
  int PW;  // independent panel groups (waves) per workgroup
};

// kernel launchers (q4mi_gemm.hip); return hipError_t as int
int launch_gemm(int fmt, const GemmArgs& g, const GemmCfg& cfg, void* stream);
GemmCfg choose_gemm_cfg(int fmt, int M, int64_t K, int64_t N);
int launch_dequant(int fmt, const uint8_t* w, int64_t panel_bytes, int64_t N, int64_t K, float g,
                   float* out, void* stream);

struct RouteArgs {
  const uint16_t* x;    // f16 [T][D]
  const float* wr;      // [D][E]
  int T, D, E, k, renormalize;
  float* logits;        // nullable [T][E]
  int32_t* idx;         // [T][k]
  float* w;             // [T][k]
  float* partial;       // workspace [nblk][T][E]
  unsigned* counter;    // workspace counter
  int nblk;             // workgroups splitting D
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
  uint16_t* h;             // workspace f16 [npairs][F]
  float* o;                // workspace fp32 [npairs][D]
};
int launch_moe(const MoeArgs& m, void* stream);

}  // namespace q4mi
