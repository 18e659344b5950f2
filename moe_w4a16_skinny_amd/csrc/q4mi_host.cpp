// Host side of libq4mi: argument validation, offline repack/unpack, workspace
// queries, and the extern "C" entry points that enqueue the HIP kernels.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "q4mi.h"
#include "q4mi_internal.h"

using namespace q4mi;

namespace q4mi {

int ensure_dynamic_lds(const void* fn, size_t bytes) {
  if (bytes <= 48 * 1024) return 0;  // within the default limit
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev)) return static_cast<int>(e);
  struct Set {
    const void* fn;
    int dev;
    size_t bytes;
  };
  static std::mutex mu;
  static std::vector<Set> done;
  std::lock_guard<std::mutex> lock(mu);
  Set* cur = nullptr;
  for (Set& d : done)
    if (d.fn == fn && d.dev == dev) cur = &d;
  if (cur && cur->bytes >= bytes) return 0;
  if (hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes))) {
    (void)hipGetLastError();  // do not leave the error for the next call
    return static_cast<int>(e);
  }
  if (cur)
    cur->bytes = bytes;
  else
    done.push_back(Set{fn, dev, bytes});
  return 0;
}

}  // namespace q4mi

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return Q4_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE_PTR(p)                                                              \
  do {                                                                              \
    if (!(p)) return fail(Q4_ERR_INVALID_ARG, "%s: %s is NULL", __func__, #p);     \
  } while (0)
#define REQUIRE_ALIGNED(p)                                                          \
  do {                                                                              \
    if (!aligned16(p))                                                              \
      return fail(Q4_ERR_ALIGNMENT, "%s: %s is not 16-byte aligned", __func__, #p); \
  } while (0)

int check_nk(const char* fn, int64_t N, int64_t K, int kmult) {
  if (N <= 0 || K <= 0) return fail(Q4_ERR_INVALID_ARG, "%s: N=%lld and K=%lld must be positive", fn, (long long)N, (long long)K);
  if (N % 16) return fail(Q4_ERR_UNSUPPORTED, "%s: N=%lld is not a multiple of 16", fn, (long long)N);
  if (K % kmult) return fail(Q4_ERR_UNSUPPORTED, "%s: K=%lld is not a multiple of %d", fn, (long long)K, kmult);
  if (N > (int64_t(1) << 30) || K > (int64_t(1) << 24))
    return fail(Q4_ERR_UNSUPPORTED, "%s: N=%lld or K=%lld too large", fn, (long long)N, (long long)K);
  return Q4_OK;
}

// ---- NVFP4 repack --------------------------------------------------------
// code byte (n, j) covers k = 2j (low nibble) and 2j + 1 (high nibble)
inline uint8_t code_byte(const uint8_t* codes, int64_t K, int64_t n, int64_t kk) {
  // kk is an even k; zero beyond K (padding)
  return kk < K ? codes[n * (K / 2) + kk / 2] : uint8_t(0);
}
inline uint8_t scale_byte(const uint8_t* scales, int64_t K, int64_t n, int64_t grp) {
  return grp < K / 16 ? scales[n * (K / 16) + grp] : uint8_t(0);
}

// Visit every (packed byte offset, canonical source) of one NVFP4 matrix.
// `code(off, n, kk)` handles one code byte (k = kk, kk+1); `scale(off, n, grp)` one scale byte.
template <class FC, class FS>
void nvfp4_walk(int64_t N, int64_t K, FC code, FS scale) {
  const int64_t nfull = full_tiles(K);
  const bool half = has_half_tile(K);
  const int64_t pb = panel_bytes(K);
  for (int64_t p = 0; p < N / 16; ++p) {
    for (int64_t t = 0; t < nfull + (half ? 1 : 0); ++t) {
      const bool is_half = t == nfull;
      const int64_t base = p * pb + t * kTileBytes;
      const int64_t kb = t * kTileK;
      const int steps = is_half ? 2 : 4;
      const int lane_bytes = steps * 4;
      for (int lane = 0; lane < 64; ++lane) {
        const int o = lane >> 4, c = lane & 15;
        const int64_t n = p * 16 + c;
        for (int i = 0; i < steps; ++i)
          for (int b = 0; b < 4; ++b)
            code(base + lane * lane_bytes + i * 4 + b, n, kb + 32 * i + 8 * o + 2 * b);
      }
      // scales: word (c, h) holds, in byte i, the scale of group kb/16 + 2i + h
      const int64_t sbase = base + (is_half ? kHalfCodeBytes : kTileCodeBytes);
      for (int c = 0; c < 16; ++c)
        for (int h = 0; h < 2; ++h)
          for (int i = 0; i < steps; ++i)
            scale(sbase + (c * 2 + h) * steps + i, p * 16 + c, kb / 16 + 2 * i + h);
    }
  }
}

// Affine: lane code dword i holds 8 codes e0..e7 (k = kb + 32i + 8o + j) with
// e_{2s} at nibble s and e_{2s+1} at nibble s + 4, so that
// ((d >> 4s) & 0x000F000F) is the pair (e_2s, e_2s+1) in the two 16-bit halves.
template <class FC, class FSB>
void affine_walk(int64_t N, int64_t K, FC code, FSB sb) {
  const int64_t nfull = full_tiles(K);
  const bool half = has_half_tile(K);
  const int64_t pb = panel_bytes(K);
  for (int64_t p = 0; p < N / 16; ++p) {
    for (int64_t t = 0; t < nfull + (half ? 1 : 0); ++t) {
      const bool is_half = t == nfull;
      const int64_t base = p * pb + t * kTileBytes;
      const int64_t kb = t * kTileK;
      const int steps = is_half ? 2 : 4;
      const int lane_bytes = steps * 4;
      for (int lane = 0; lane < 64; ++lane) {
        const int o = lane >> 4, c = lane & 15;
        const int64_t n = p * 16 + c;
        for (int i = 0; i < steps; ++i)
          code(base + lane * lane_bytes + i * 4, n, kb + 32 * i + 8 * o);
      }
      const int64_t sbase = base + (is_half ? kHalfCodeBytes : kTileCodeBytes);
      const int groups = is_half ? 1 : 2;
      for (int c = 0; c < 16; ++c)
        for (int gi = 0; gi < groups; ++gi)
          sb(sbase + (c * groups + gi) * 4, p * 16 + c, kb / 64 + gi);
    }
  }
}

inline uint32_t affine_word_from_codes(const uint8_t e[8]) {
  uint32_t d = 0;
  for (int s = 0; s < 4; ++s) {
    d |= uint32_t(e[2 * s] & 15) << (4 * s);
    d |= uint32_t(e[2 * s + 1] & 15) << (16 + 4 * s);
  }
  return d;
}

}  // namespace

extern "C" {

int q4_abi_version(void) { return Q4MI_ABI_VERSION; }

const char* q4_last_error(void) { return g_last_error.c_str(); }

size_t q4_nvfp4_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 || K % 16) return 0;
  return size_t(packed_matrix_bytes(N, K));
}

int q4_nvfp4_repack(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, void* packed,
                    size_t packed_bytes) {
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  REQUIRE_PTR(packed);
  if (int rc = check_nk(__func__, N, K, 16)) return rc;
  if (packed_bytes < q4_nvfp4_packed_bytes(N, K))
    return fail(Q4_ERR_INVALID_ARG, "%s: packed_bytes=%zu < %zu", __func__, packed_bytes, q4_nvfp4_packed_bytes(N, K));
  uint8_t* out = static_cast<uint8_t*>(packed);
  std::memset(out + N / 16 * panel_bytes(K), 0, size_t(packed_tail(K)));
  nvfp4_walk(N, K,
             [&](int64_t off, int64_t n, int64_t kk) { out[off] = code_byte(codes, K, n, kk); },
             [&](int64_t off, int64_t n, int64_t grp) { out[off] = scale_byte(scales, K, n, grp); });
  return ok();
}

size_t q4_nvfp4_quantize_workspace_bytes(void) { return kWsCounterBytes + 256; }

int q4_nvfp4_quantize(const float* w, int64_t N, int64_t K, float global_scale, void* packed, size_t packed_bytes,
                      float* g_out, void* ws, size_t ws_bytes, void* stream) {
  REQUIRE_PTR(w);
  REQUIRE_PTR(packed);
  if (int rc = check_nk(__func__, N, K, 16)) return rc;
  if (packed_bytes < q4_nvfp4_packed_bytes(N, K))
    return fail(Q4_ERR_INVALID_ARG, "%s: packed_bytes=%zu < %zu", __func__, packed_bytes, q4_nvfp4_packed_bytes(N, K));
  if (global_scale != global_scale || global_scale > 3.0e38f || global_scale < -3.0e38f)
    return fail(Q4_ERR_INVALID_ARG, "%s: global_scale=%g is not finite", __func__, double(global_scale));
  if (full_tiles(K) + 1 > 65535) return fail(Q4_ERR_UNSUPPORTED, "%s: K=%lld too large", __func__, (long long)K);
  REQUIRE_ALIGNED(w);
  REQUIRE_ALIGNED(packed);
  unsigned* amax = nullptr;
  if (!(global_scale > 0.0f)) {  // the global scale comes from the tensor's amax: one scratch word
    if (!ws) return fail(Q4_ERR_WORKSPACE, "%s: ws is NULL", __func__);
    if (ws_bytes < q4_nvfp4_quantize_workspace_bytes())
      return fail(Q4_ERR_WORKSPACE, "%s: ws_bytes=%zu < %zu", __func__, ws_bytes, q4_nvfp4_quantize_workspace_bytes());
    REQUIRE_ALIGNED(ws);
    amax = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kWsCounterBytes);
  }
  if (int e = launch_quantize(w, N, K, global_scale > 0.0f ? global_scale : 0.0f, amax,
                              static_cast<uint8_t*>(packed), g_out, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

int q4_nvfp4_unpack(const void* packed, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales) {
  REQUIRE_PTR(packed);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scales);
  if (int rc = check_nk(__func__, N, K, 16)) return rc;
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  nvfp4_walk(N, K,
             [&](int64_t off, int64_t n, int64_t kk) {
               if (kk < K) codes[n * (K / 2) + kk / 2] = in[off];
             },
             [&](int64_t off, int64_t n, int64_t grp) {
               if (grp < K / 16) scales[n * (K / 16) + grp] = in[off];
             });
  return ok();
}

size_t q4_affine4_packed_bytes(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % 16 || K % 64) return 0;
  return size_t(packed_matrix_bytes(N, K));
}

int q4_affine4_repack(const uint8_t* codes, const uint16_t* scale_bf16, const uint16_t* bias_bf16,
                      int64_t N, int64_t K, void* packed, size_t packed_bytes) {
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scale_bf16);
  REQUIRE_PTR(bias_bf16);
  REQUIRE_PTR(packed);
  if (int rc = check_nk(__func__, N, K, 64)) return rc;
  if (packed_bytes < q4_affine4_packed_bytes(N, K))
    return fail(Q4_ERR_INVALID_ARG, "%s: packed_bytes=%zu < %zu", __func__, packed_bytes, q4_affine4_packed_bytes(N, K));
  uint8_t* out = static_cast<uint8_t*>(packed);
  std::memset(out + N / 16 * panel_bytes(K), 0, size_t(packed_tail(K)));
  const int64_t G = K / 64;
  affine_walk(
      N, K,
      [&](int64_t off, int64_t n, int64_t k0) {
        uint8_t e[8];
        for (int j = 0; j < 8; ++j) {
          const uint8_t byte = codes[n * (K / 2) + (k0 + j) / 2];
          e[j] = ((k0 + j) & 1) ? uint8_t(byte >> 4) : uint8_t(byte & 15);
        }
        const uint32_t d = affine_word_from_codes(e);
        std::memcpy(out + off, &d, 4);
      },
      [&](int64_t off, int64_t n, int64_t grp) {
        const uint16_t s = scale_bf16[n * G + grp], b = bias_bf16[n * G + grp];
        std::memcpy(out + off, &s, 2);
        std::memcpy(out + off + 2, &b, 2);
      });
  return ok();
}

int q4_affine4_unpack(const void* packed, int64_t N, int64_t K, uint8_t* codes, uint16_t* scale_bf16,
                      uint16_t* bias_bf16) {
  REQUIRE_PTR(packed);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scale_bf16);
  REQUIRE_PTR(bias_bf16);
  if (int rc = check_nk(__func__, N, K, 64)) return rc;
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  const int64_t G = K / 64;
  affine_walk(
      N, K,
      [&](int64_t off, int64_t n, int64_t k0) {
        uint32_t d;
        std::memcpy(&d, in + off, 4);
        for (int s = 0; s < 4; ++s) {
          const uint8_t lo = (d >> (4 * s)) & 15, hi = (d >> (16 + 4 * s)) & 15;
          // elements 2s and 2s+1 form one canonical byte (2s even)
          codes[n * (K / 2) + (k0 + 2 * s) / 2] = uint8_t(lo | (hi << 4));
        }
      },
      [&](int64_t off, int64_t n, int64_t grp) {
        std::memcpy(&scale_bf16[n * G + grp], in + off, 2);
        std::memcpy(&bias_bf16[n * G + grp], in + off + 2, 2);
      });
  return ok();
}

// ---- GEMMs ---------------------------------------------------------------

size_t qgemm_nvfp4_workspace_bytes(int M, int64_t K, int64_t N, int want_argmax) {
  if (M < 1 || M > 16 || N <= 0 || K <= 0 || N % 16 || K % 16) return 0;
  const size_t b = gemm_workspace(kNvfp4, M, K, N);
  return (b > kWsCounterBytes || want_argmax) ? b : 0;  // counters alone serve only the argmax
}

size_t qgemm_affine4_workspace_bytes(int M, int64_t K, int64_t N) {
  if (M < 1 || M > 16 || N <= 0 || K <= 0 || N % 16 || K % 64) return 0;
  const size_t b = gemm_workspace(kAffine, M, K, N);
  return b > kWsCounterBytes ? b : 0;
}

constexpr int kMaxPrefillRows = 65536;  // M limit of the NVFP4 GEMM for M > 16

struct SampleSpec {  // qgemm_nvfp4_sample's extra arguments
  float softcap, temperature;
  uint64_t seed;
  uint32_t offset;
};

static int gemm_common(int fmt, const char* fn, const void* w_packed, float gscale, const void* a, int M,
                       int64_t K, int64_t N, void* out, int out_dtype, int32_t* argmax, void* ws,
                       size_t ws_bytes, void* stream, const SampleSpec* sp = nullptr) {
  if (!w_packed) return fail(Q4_ERR_INVALID_ARG, "%s: w_packed is NULL", fn);
  if (!a) return fail(Q4_ERR_INVALID_ARG, "%s: a is NULL", fn);
  if (!out && !sp) return fail(Q4_ERR_INVALID_ARG, "%s: out is NULL", fn);
  if (sp && !argmax) return fail(Q4_ERR_INVALID_ARG, "%s: token is NULL", fn);
  if (sp && !(sp->temperature >= 0.0f && sp->temperature <= 3.0e38f))
    return fail(Q4_ERR_INVALID_ARG, "%s: temperature=%g is not a finite number >= 0", fn, double(sp->temperature));
  if (sp && !(sp->softcap <= 3.0e38f))  // NaN or inf
    return fail(Q4_ERR_INVALID_ARG, "%s: softcap=%g is not finite", fn, double(sp->softcap));
  // more than 16 rows: NVFP4 only, without the fused argmax or sampling
  const bool prefill = fmt == kNvfp4 && M > 16 && !argmax && !sp;
  if (M < 1 || M > (prefill ? kMaxPrefillRows : 16))
    return fail(Q4_ERR_UNSUPPORTED, "%s: M=%d outside 1..16 (1..%d for NVFP4 without argmax or sampling)", fn, M,
                kMaxPrefillRows);
  if (int rc = check_nk(fn, N, K, fmt == kNvfp4 ? 16 : 64)) return rc;
  if (fmt == kNvfp4 && out_dtype != Q4_F32 && out_dtype != Q4_F16 && out_dtype != Q4_BF16)
    return fail(Q4_ERR_INVALID_ARG, "%s: out_dtype=%d is not Q4_F32, Q4_F16 or Q4_BF16", fn, out_dtype);
  if (fmt == kAffine && out_dtype != Q4_F32 && out_dtype != Q4_BF16)
    return fail(Q4_ERR_INVALID_ARG, "%s: out_dtype=%d is not Q4_F32 or Q4_BF16", fn, out_dtype);
  if (!aligned16(w_packed)) return fail(Q4_ERR_ALIGNMENT, "%s: w_packed is not 16-byte aligned", fn);
  if (!aligned16(a)) return fail(Q4_ERR_ALIGNMENT, "%s: a is not 16-byte aligned", fn);
  if (out && !aligned16(out)) return fail(Q4_ERR_ALIGNMENT, "%s: out is not 16-byte aligned", fn);
  const size_t need = fmt == kNvfp4 ? qgemm_nvfp4_workspace_bytes(M, K, N, argmax != nullptr)
                                    : qgemm_affine4_workspace_bytes(M, K, N);
  if (need) {
    if (!ws) return fail(Q4_ERR_WORKSPACE, "%s: ws is NULL but %zu bytes are needed", fn, need);
    if (ws_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: ws_bytes=%zu < %zu", fn, ws_bytes, need);
    if (!aligned16(ws)) return fail(Q4_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  }
  if (argmax && !aligned16(argmax)) return fail(Q4_ERR_ALIGNMENT, "%s: argmax is not 16-byte aligned", fn);
  GemmArgs g{};
  g.w = static_cast<const uint8_t*>(w_packed);
  g.panel_bytes = panel_bytes(K);
  g.a = static_cast<const uint16_t*>(a);
  g.M = M;
  g.K = int(K);
  g.N = int(N);
  g.nfull = int(full_tiles(K));
  g.half = has_half_tile(K) ? 1 : 0;
  g.k_exact = (K % 64) == 0;
  g.gscale = gscale;
  g.out = out;
  g.out_dtype = out_dtype;
  g.argmax = argmax;
  g.counter = argmax ? reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kWsArgmaxCounter) : nullptr;
  g.keys = argmax ? reinterpret_cast<unsigned long long*>(static_cast<char*>(ws) + kWsArgmaxKeys) : nullptr;
  if (sp) {
    g.sample = 1;
    g.softcap = sp->softcap > 0.0f ? sp->softcap : 0.0f;
    g.inv_temp = sp->temperature > 0.0f ? static_cast<float>(1.0 / double(sp->temperature)) : 0.0f;
    g.seed_lo = static_cast<unsigned>(sp->seed & 0xFFFFFFFFu);
    g.seed_hi = static_cast<unsigned>(sp->seed >> 32);
    g.offset = sp->offset;
  }
  if (prefill) {
    // one workgroup per 64 x 128 block (or a smaller measured shape): keep the grid within int range
    if ((int64_t(M) + 15) / 16 * ((N + 127) / 128) > (int64_t(1) << 30))
      return fail(Q4_ERR_UNSUPPORTED, "%s: M=%d x N=%lld too large for one launch", fn, M, (long long)N);
    if (int e = launch_prefill(g, stream)) return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", fn, e);
    return ok();
  }
  const GemmCfg cfg = choose_gemm_cfg(fmt, M, K, N);
  if (int e = launch_gemm(fmt, g, cfg, ws, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", fn, e);
  return ok();
}

int qgemm_nvfp4(const void* w_packed, float global_scale, const void* a, int M, int64_t K, int64_t N, void* out,
                int out_dtype, int32_t* argmax, void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(kNvfp4, __func__, w_packed, global_scale, a, M, K, N, out, out_dtype, argmax, ws, ws_bytes,
                     stream);
}

int qgemm_nvfp4_sample(const void* w_packed, float global_scale, const void* a, int M, int64_t K, int64_t N,
                       float softcap, float temperature, uint64_t seed, uint32_t offset, void* logits, int out_dtype,
                       int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  const SampleSpec sp{softcap, temperature, seed, offset};
  return gemm_common(kNvfp4, __func__, w_packed, global_scale, a, M, K, N, logits, out_dtype, token, ws, ws_bytes,
                     stream, &sp);
}

int q4_sample_uniforms(uint64_t seed, uint32_t offset, int M, int64_t N, float* out, void* stream) {
  REQUIRE_PTR(out);
  if (M < 1 || N < 1 || N > (int64_t(1) << 31) - 1 || int64_t(M) * N > (int64_t(1) << 40))
    return fail(Q4_ERR_UNSUPPORTED, "%s: M=%d N=%lld out of range", __func__, M, (long long)N);
  if (int e = launch_sample_uniforms(static_cast<unsigned>(seed & 0xFFFFFFFFu), static_cast<unsigned>(seed >> 32),
                                     offset, M, N, out, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

int qgemm_affine4(const void* w_packed, const void* a, int M, int64_t K, int64_t N, void* out, int out_dtype,
                  void* ws, size_t ws_bytes, void* stream) {
  return gemm_common(kAffine, __func__, w_packed, 1.0f, a, M, K, N, out, out_dtype, nullptr, ws, ws_bytes, stream);
}

int q4_stream_read(const void* src, size_t bytes, int grid, int mode, int depth, uint32_t* out, void* stream) {
  REQUIRE_PTR(src);
  REQUIRE_PTR(out);
  if (bytes == 0 || bytes % 16) return fail(Q4_ERR_INVALID_ARG, "%s: bytes=%zu is not a positive multiple of 16", __func__, bytes);
  if (grid < 1 || grid > 65536) return fail(Q4_ERR_INVALID_ARG, "%s: grid=%d outside 1..65536", __func__, grid);
  if (mode < 0 || mode > 2) return fail(Q4_ERR_INVALID_ARG, "%s: mode=%d is not 0, 1 or 2", __func__, mode);
  if (mode < 2 && depth != 1 && depth != 2 && depth != 4 && depth != 8)
    return fail(Q4_ERR_INVALID_ARG, "%s: depth=%d is not 1, 2, 4 or 8", __func__, depth);
  if (mode == 2 && (bytes / 16 + size_t(grid) - 1) / size_t(grid) > size_t(512) * 32)
    return fail(Q4_ERR_INVALID_ARG, "%s: mode 2 reads at most 256 KiB per workgroup (grid=%d)", __func__, grid);
  REQUIRE_ALIGNED(src);
  if (int e = launch_stream_read(src, bytes, grid, mode, depth, out, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

int q4_dequant_nvfp4(const void* w_packed, float global_scale, int64_t N, int64_t K, float* out, void* stream) {
  REQUIRE_PTR(w_packed);
  REQUIRE_PTR(out);
  if (int rc = check_nk(__func__, N, K, 16)) return rc;
  REQUIRE_ALIGNED(w_packed);
  REQUIRE_ALIGNED(out);
  if (int e = launch_dequant(kNvfp4, static_cast<const uint8_t*>(w_packed), panel_bytes(K), N, K, global_scale, out,
                             stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

int q4_dequant_affine4(const void* w_packed, int64_t N, int64_t K, float* out, void* stream) {
  REQUIRE_PTR(w_packed);
  REQUIRE_PTR(out);
  if (int rc = check_nk(__func__, N, K, 64)) return rc;
  REQUIRE_ALIGNED(w_packed);
  REQUIRE_ALIGNED(out);
  if (int e = launch_dequant(kAffine, static_cast<const uint8_t*>(w_packed), panel_bytes(K), N, K, 1.0f, out, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

// ---- router --------------------------------------------------------------

size_t moe_route_workspace_bytes(int T, int D, int E) {
  if (T < 1 || D < 1 || E < 1 || E > 256) return 0;
  return kWsCounterBytes + size_t(route_splits(D)) * size_t(T) * size_t(E) * sizeof(float);
}

}  // extern "C"

// Every condition moe_route_topk refuses, checked without enqueueing anything.
static int route_check(const char* fn, const void* x, const float* w_router, int T, int D, int E, int k,
                       const float* logits, const int32_t* topk_idx, const float* topk_w, const void* ws,
                       size_t ws_bytes) {
  if (!x || !w_router || !topk_idx || !topk_w)
    return fail(Q4_ERR_INVALID_ARG, "%s: x, w_router, topk_idx and topk_w must not be NULL", fn);
  if (T < 1 || D < 1 || E < 1 || k < 1)
    return fail(Q4_ERR_INVALID_ARG, "%s: T=%d D=%d E=%d k=%d must be positive", fn, T, D, E, k);
  if (T > 64) return fail(Q4_ERR_UNSUPPORTED, "%s: T=%d > 64", fn, T);
  if (E > 256) return fail(Q4_ERR_UNSUPPORTED, "%s: E=%d > 256", fn, E);
  if (k > E || k > 16) return fail(Q4_ERR_UNSUPPORTED, "%s: k=%d must be <= E=%d and <= 16", fn, k, E);
  if (D % 8) return fail(Q4_ERR_UNSUPPORTED, "%s: D=%d is not a multiple of 8", fn, D);
  if (route_rows(D) > kRouteMaxRows)
    return fail(Q4_ERR_UNSUPPORTED, "%s: D=%d > %d", fn, D, kRouteMaxSplits * kRouteMaxRows);
  if (!aligned16(x) || !aligned16(w_router) || !aligned16(topk_idx) || !aligned16(topk_w) ||
      (logits && !aligned16(logits)))
    return fail(Q4_ERR_ALIGNMENT, "%s: x, w_router, topk_idx, topk_w and logits must be 16-byte aligned", fn);
  if (!ws) return fail(Q4_ERR_WORKSPACE, "%s: ws is NULL", fn);
  if (!aligned16(ws)) return fail(Q4_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  if (ws_bytes < moe_route_workspace_bytes(T, D, E))
    return fail(Q4_ERR_WORKSPACE, "%s: ws_bytes=%zu < %zu", fn, ws_bytes, moe_route_workspace_bytes(T, D, E));
  return Q4_OK;
}

// partial: where the partial logits go (NULL: the workspace past its
// counters); partials_only: stop there (the routed gate/up takes the top-k)
static int route_enqueue(const char* fn, const void* x, const float* w_router, int T, int D, int E, int k,
                         int renormalize, float* logits, int32_t* topk_idx, float* topk_w, void* ws, void* stream,
                         const q4_moe_block_desc* blk = nullptr, int32_t* didx = nullptr, float* dw = nullptr,
                         float* partial = nullptr, bool partials_only = false) {
  RouteArgs r{};
  if (blk) {  // the MoE block's routing: scores normalized and scaled, weights times the down scale
    r.zscale = blk->router_scale;
    r.down_scale = blk->down_scale;
    r.eps = blk->eps;
    r.didx = didx;
    r.dw = dw;
  }
  r.x = static_cast<const uint16_t*>(x);
  r.wr = w_router;
  r.T = T;
  r.D = D;
  r.E = E;
  r.k = k;
  r.renormalize = renormalize ? 1 : 0;
  r.logits = logits;
  r.idx = topk_idx;
  r.w = topk_w;
  r.counter = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + kWsRouteCounter);
  r.partial = partial ? partial : reinterpret_cast<float*>(static_cast<char*>(ws) + kWsCounterBytes);
  r.partials_only = partials_only ? 1 : 0;
  r.nsplit = route_splits(D);
  r.rows = route_rows(D);
  if (int e = launch_route(r, stream)) return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", fn, e);
  return Q4_OK;
}

extern "C" {

int moe_route_topk(const void* x, const float* w_router, int T, int D, int E, int k, int renormalize, float* logits,
                   int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = route_check(__func__, x, w_router, T, D, E, k, logits, topk_idx, topk_w, ws, ws_bytes)) return rc;
  if (int rc = route_enqueue(__func__, x, w_router, T, D, E, k, renormalize, logits, topk_idx, topk_w, ws, stream))
    return rc;
  return ok();
}

// ---- grouped MoE ---------------------------------------------------------

// scratch after the counter region: h [npairs][F] f16, o [T][k + 1][D] fp32,
// rowof [T k] int32, the grouping table (moe_grp_words int32)
static size_t moe_ws_layout(const q4_moe_desc* w, int T, int k, size_t* h_off, size_t* o_off, size_t* r_off,
                            size_t* g_off) {
  const size_t npairs = size_t(T) * size_t(k) + (w->has_shared ? size_t(T) : 0);
  const size_t hbytes = (npairs * size_t(w->F) * 2 + 255) / 256 * 256;
  const size_t obytes = (size_t(T) * (size_t(k) + 1) * size_t(w->D) * 4 + 255) / 256 * 256;
  const size_t rbytes = (size_t(T) * size_t(k) * 4 + 255) / 256 * 256;
  const size_t gbytes = (moe_grp_words(w->E, T, k) * 4 + 255) / 256 * 256;
  *h_off = kWsCounterBytes;
  *o_off = *h_off + hbytes;
  *r_off = *o_off + obytes;
  *g_off = *r_off + rbytes;
  return *g_off + gbytes;
}

size_t moe_workspace_bytes(const q4_moe_desc* w, int T, int k) {
  if (!w || T < 1 || k < 1 || w->D < 1 || w->F < 1) return 0;
  size_t h, o, r;
  size_t g;
  return moe_ws_layout(w, T, k, &h, &o, &r, &g);
}

}  // extern "C"

// Every condition moe_grouped_qgemm refuses except those on its workspace,
// checked without enqueueing anything.
static int moe_check_shape(const char* fn, const q4_moe_desc* w, const void* x, const int32_t* topk_idx,
                           const float* topk_w, int T, int k, const void* y, int out_dtype) {
  if (!w) return fail(Q4_ERR_INVALID_ARG, "%s: w is NULL", fn);
  if (!x || !topk_idx || !topk_w || !y)
    return fail(Q4_ERR_INVALID_ARG, "%s: x, topk_idx, topk_w and y must not be NULL", fn);
  if (!w->gate_packed || !w->up_packed || !w->down_packed || !w->g_gate || !w->g_up || !w->g_down)
    return fail(Q4_ERR_INVALID_ARG, "%s: a weight or global-scale pointer of the descriptor is NULL", fn);
  if (w->E < 1 || w->D < 1 || w->F < 1 || (w->has_shared != 0 && w->has_shared != 1))
    return fail(Q4_ERR_INVALID_ARG, "%s: bad descriptor (E=%d D=%d F=%d has_shared=%d)", fn, w->E, w->D, w->F,
                w->has_shared);
  if (T < 1 || T > 16) return fail(Q4_ERR_UNSUPPORTED, "%s: T=%d outside 1..16", fn, T);
  if (k < 1 || k > w->E || k > 64) return fail(Q4_ERR_UNSUPPORTED, "%s: k=%d outside 1..min(E=%d, 64)", fn, k, w->E);
  if (w->D % 64 || w->F % 64)
    return fail(Q4_ERR_UNSUPPORTED, "%s: D=%d and F=%d must be multiples of 64", fn, w->D, w->F);
  if (w->E > 1024) return fail(Q4_ERR_UNSUPPORTED, "%s: E=%d > 1024", fn, w->E);
  if (out_dtype != Q4_F32 && out_dtype != Q4_F16)
    return fail(Q4_ERR_INVALID_ARG, "%s: out_dtype=%d is not Q4_F32 or Q4_F16", fn, out_dtype);
  if (!aligned16(x) || !aligned16(topk_idx) || !aligned16(topk_w) || !aligned16(y) || !aligned16(w->gate_packed) ||
      !aligned16(w->up_packed) || !aligned16(w->down_packed))
    return fail(Q4_ERR_ALIGNMENT, "%s: x, topk_idx, topk_w, y and the packed weights must be 16-byte aligned", fn);
  return Q4_OK;
}

// ... and with them
static int moe_check(const char* fn, const q4_moe_desc* w, const void* x, const int32_t* topk_idx,
                     const float* topk_w, int T, int k, const void* y, int out_dtype, const void* ws,
                     size_t ws_bytes) {
  if (int rc = moe_check_shape(fn, w, x, topk_idx, topk_w, T, k, y, out_dtype)) return rc;
  if (!ws) return fail(Q4_ERR_WORKSPACE, "%s: ws is NULL", fn);
  if (!aligned16(ws)) return fail(Q4_ERR_ALIGNMENT, "%s: ws is not 16-byte aligned", fn);
  size_t h_off, o_off, r_off, g_off;
  const size_t need = moe_ws_layout(w, T, k, &h_off, &o_off, &r_off, &g_off);
  if (ws_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: ws_bytes=%zu < %zu", fn, ws_bytes, need);
  return Q4_OK;
}

// The kernels' view of one grouped layer over workspace ws.
static MoeArgs moe_args(const q4_moe_desc* w, const void* x, const int32_t* topk_idx, const float* topk_w, int T,
                        int k, void* y, int out_dtype, void* ws, bool combine) {
  size_t h_off, o_off, r_off, g_off;
  (void)moe_ws_layout(w, T, k, &h_off, &o_off, &r_off, &g_off);
  MoeArgs m{};
  m.E = w->E;
  m.has_shared = w->has_shared;
  m.D = w->D;
  m.F = w->F;
  m.T = T;
  m.k = k;
  m.gate = static_cast<const uint8_t*>(w->gate_packed);
  m.up = static_cast<const uint8_t*>(w->up_packed);
  m.down = static_cast<const uint8_t*>(w->down_packed);
  m.gate_stride = int64_t(q4_nvfp4_packed_bytes(w->F, w->D));
  m.down_stride = int64_t(q4_nvfp4_packed_bytes(w->D, w->F));
  m.gate_panel_bytes = panel_bytes(w->D);
  m.down_panel_bytes = panel_bytes(w->F);
  m.g_gate = w->g_gate;
  m.g_up = w->g_up;
  m.g_down = w->g_down;
  m.x = static_cast<const uint16_t*>(x);
  m.idx = topk_idx;
  m.tw = topk_w;
  m.y = y;
  m.out_dtype = out_dtype;
  m.h = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + h_off);
  m.o = reinterpret_cast<float*>(static_cast<char*>(ws) + o_off);
  m.rowof = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + r_off);
  m.grp = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + g_off);
  m.combine = combine ? 1 : 0;
  return m;
}

static int moe_enqueue(const char* fn, const q4_moe_desc* w, const void* x, const int32_t* topk_idx,
                       const float* topk_w, int T, int k, void* y, int out_dtype, void* ws, void* stream) {
  const MoeArgs m = moe_args(w, x, topk_idx, topk_w, T, k, y, out_dtype, ws, true);
  if (int e = launch_moe(m, nullptr, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", fn, e);
  return Q4_OK;
}

extern "C" {

int moe_grouped_qgemm(const q4_moe_desc* w, const void* x, const int32_t* topk_idx, const float* topk_w, int T,
                      int k, void* y, int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = moe_check(__func__, w, x, topk_idx, topk_w, T, k, y, out_dtype, ws, ws_bytes)) return rc;
  if (int rc = moe_enqueue(__func__, w, x, topk_idx, topk_w, T, k, y, out_dtype, ws, stream)) return rc;
  return ok();
}

int moe_grouped_qgemm_noalloc(const q4_moe_desc* w, const void* x, const int32_t* topk_idx, const float* topk_w,
                              int T, int k, void* y, int out_dtype, void* stream) {
  if (int rc = moe_check_shape(__func__, w, x, topk_idx, topk_w, T, k, y, out_dtype)) return rc;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  if (int e = moe_noalloc_scratch(&scratch, &scratch_bytes))
    return fail(Q4_ERR_HIP, "%s: the scratch array's device address is not available (hip error %d)", __func__, e);
  const size_t need = moe_workspace_bytes(w, T, k);
  if (need > scratch_bytes)
    return fail(Q4_ERR_UNSUPPORTED, "%s: this shape needs %zu bytes of scratch, more than the %zu of the "
                "library's per-device array (use moe_grouped_qgemm with a workspace)", __func__, need, scratch_bytes);
  if (int rc = moe_enqueue(__func__, w, x, topk_idx, topk_w, T, k, y, out_dtype, scratch, stream)) return rc;
  return ok();
}

// ---- router + grouped MoE in one call -------------------------------------

static size_t route_part_bytes(int T, int D, int E) {
  return (size_t(route_splits(D)) * size_t(T) * size_t(E) * sizeof(float) + 255) / 256 * 256;
}

size_t moe_route_grouped_workspace_bytes(const q4_moe_desc* w, int T, int k) {
  const size_t m = moe_workspace_bytes(w, T, k);
  if (!m || w->E > 256) return 0;
  return m + route_part_bytes(T, w->D, w->E);
}

int moe_route_grouped_qgemm(const q4_moe_desc* w, const void* x, const float* w_router, int T, int k,
                            int renormalize, float* logits, int32_t* topk_idx, float* topk_w, void* y,
                            int out_dtype, void* ws, size_t ws_bytes, void* stream) {
  if (int rc = moe_check_shape(__func__, w, x, topk_idx, topk_w, T, k, y, out_dtype)) return rc;
  const size_t mws = moe_workspace_bytes(w, T, k);
  // the router's own conditions, its workspace taken as the whole of ws
  if (int rc = route_check(__func__, x, w_router, T, w->D, w->E, k, logits, topk_idx, topk_w, ws, ws_bytes))
    return rc;
  const size_t need = moe_route_grouped_workspace_bytes(w, T, k);
  if (ws_bytes < need) return fail(Q4_ERR_WORKSPACE, "%s: ws_bytes=%zu < %zu", __func__, ws_bytes, need);
  // the partial logits past the layer's scratch (gate/up reads them while it writes h)
  float* part = reinterpret_cast<float*>(static_cast<char*>(ws) + mws);
  if (moe_gu_route_fits(T, w->D, w->E)) {
    if (int rc = route_enqueue(__func__, x, w_router, T, w->D, w->E, k, renormalize, nullptr, topk_idx, topk_w, ws,
                               stream, nullptr, nullptr, nullptr, part, true))
      return rc;
    MoeArgs m = moe_args(w, x, nullptr, topk_w, T, k, y, out_dtype, ws, true);
    m.rpart = part;
    m.rsplit = route_splits(w->D);
    m.renorm = renormalize ? 1 : 0;
    m.ridx = topk_idx;
    m.rtw = topk_w;
    m.rlogits = logits;
    if (int e = launch_moe(m, nullptr, stream))
      return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  } else {  // the router's own top-k, then the layer
    if (int rc = route_enqueue(__func__, x, w_router, T, w->D, w->E, k, renormalize, logits, topk_idx, topk_w, ws,
                               stream, nullptr, nullptr, nullptr, part, false))
      return rc;
    if (int rc = moe_enqueue(__func__, w, x, topk_idx, topk_w, T, k, y, out_dtype, ws, stream)) return rc;
  }
  return ok();
}

// ---- affine 2/3/5/6/8-bit ------------------------------------------------
}  // extern "C"
namespace {
bool affine_bits_ok(int bits) { return bits == 2 || bits == 3 || bits == 5 || bits == 6 || bits == 8; }
int64_t affb_tiles(int64_t K) { return (K + kTileK - 1) / kTileK; }
int64_t affb_tile_bytes(int bits) { return 256 * int64_t(bits) + 128; }

// A lane's 4 * bits code bytes come in pieces of affb_piece(bits) bytes
// (16, 8 or 4: the widest load that divides them); piece j of lane l of a
// tile sits at j * 64 * piece + l * piece, so that each load instruction of
// a wave reads one contiguous block.
int affb_piece(int bits) { return bits % 4 == 0 ? 16 : (bits % 2 == 0 ? 8 : 4); }

// Visit every lane chunk and scale/bias word of the b-bit layout.
// chunk(at, n, kb, o): the lane's 4 * bits bytes for row n, k = kb + 32 i +
// 8 o + j, byte x of its bit stream at offset at(x) of the packed buffer
// sb(off, n, grp): the (scale, bias) word of group grp of row n
template <class FC, class FSB>
void affine_bits_walk(int64_t N, int64_t K, int bits, FC chunk, FSB sb) {
  const int64_t nt = affb_tiles(K), tb = affb_tile_bytes(bits), pb = nt * tb;
  const int pc = affb_piece(bits);
  for (int64_t p = 0; p < N / 16; ++p)
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t base = p * pb + t * tb;
      for (int lane = 0; lane < 64; ++lane) {
        auto at = [&](int x) { return base + int64_t(x / pc) * 64 * pc + int64_t(lane) * pc + x % pc; };
        chunk(at, p * 16 + (lane & 15), t * kTileK, lane >> 4);
      }
      for (int c = 0; c < 16; ++c)
        for (int gi = 0; gi < 2; ++gi) sb(base + 256 * bits + (c * 2 + gi) * 4, p * 16 + c, t * 2 + gi);
    }
}
}  // namespace
extern "C" {

size_t q4_affine_bits_packed_bytes(int64_t N, int64_t K, int bits) {
  if (!affine_bits_ok(bits) || N <= 0 || K <= 0 || N % 16 || K % 64) return 0;
  return size_t(N / 16) * size_t(affb_tiles(K) * affb_tile_bytes(bits));
}

int q4_affine_bits_repack(const uint8_t* codes, const uint16_t* scale_bf16, const uint16_t* bias_bf16, int64_t N,
                          int64_t K, int bits, void* packed, size_t packed_bytes) {
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scale_bf16);
  REQUIRE_PTR(bias_bf16);
  REQUIRE_PTR(packed);
  if (!affine_bits_ok(bits)) return fail(Q4_ERR_UNSUPPORTED, "%s: bits=%d not in {2, 3, 5, 6, 8}", __func__, bits);
  if (int rc = check_nk(__func__, N, K, 64)) return rc;
  const size_t need = q4_affine_bits_packed_bytes(N, K, bits);
  if (packed_bytes < need) return fail(Q4_ERR_INVALID_ARG, "%s: packed_bytes=%zu < %zu", __func__, packed_bytes, need);
  for (int64_t i = 0; i < N * K; ++i)
    if (codes[i] >> bits) return fail(Q4_ERR_INVALID_ARG, "%s: code %d at %lld exceeds %d bits", __func__, codes[i],
                                      (long long)i, bits);
  uint8_t* out = static_cast<uint8_t*>(packed);
  const int64_t G = K / 64;
  affine_bits_walk(
      N, K, bits,
      [&](auto at, int64_t n, int64_t kb, int o) {
        uint8_t dst[32] = {};  // the lane's bit stream (4 * bits <= 32 bytes)
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 8; ++j) {
            const int64_t k = kb + 32 * i + 8 * o + j;
            const unsigned q = k < K ? codes[n * K + k] : 0u;
            const int bit = 8 * bits * i + bits * j;
            for (int b = 0; b < bits; ++b)
              if (q >> b & 1u) dst[(bit + b) >> 3] |= uint8_t(1u << ((bit + b) & 7));
          }
        for (int x = 0; x < 4 * bits; ++x) out[at(x)] = dst[x];
      },
      [&](int64_t off, int64_t n, int64_t grp) {
        const uint16_t sv = grp < G ? scale_bf16[n * G + grp] : 0, bv = grp < G ? bias_bf16[n * G + grp] : 0;
        std::memcpy(out + off, &sv, 2);
        std::memcpy(out + off + 2, &bv, 2);
      });
  return ok();
}

int q4_affine_bits_unpack(const void* packed, int64_t N, int64_t K, int bits, uint8_t* codes, uint16_t* scale_bf16,
                          uint16_t* bias_bf16) {
  REQUIRE_PTR(packed);
  REQUIRE_PTR(codes);
  REQUIRE_PTR(scale_bf16);
  REQUIRE_PTR(bias_bf16);
  if (!affine_bits_ok(bits)) return fail(Q4_ERR_UNSUPPORTED, "%s: bits=%d not in {2, 3, 5, 6, 8}", __func__, bits);
  if (int rc = check_nk(__func__, N, K, 64)) return rc;
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  const int64_t G = K / 64;
  affine_bits_walk(
      N, K, bits,
      [&](auto at, int64_t n, int64_t kb, int o) {
        uint8_t src[32];
        for (int x = 0; x < 4 * bits; ++x) src[x] = in[at(x)];
        for (int i = 0; i < 4; ++i)
          for (int j = 0; j < 8; ++j) {
            const int64_t k = kb + 32 * i + 8 * o + j;
            if (k >= K) continue;
            const int bit = 8 * bits * i + bits * j;
            unsigned q = 0;
            for (int b = 0; b < bits; ++b) q |= unsigned(src[(bit + b) >> 3] >> ((bit + b) & 7) & 1u) << b;
            codes[n * K + k] = uint8_t(q);
          }
      },
      [&](int64_t off, int64_t n, int64_t grp) {
        if (grp >= G) return;
        std::memcpy(&scale_bf16[n * G + grp], in + off, 2);
        std::memcpy(&bias_bf16[n * G + grp], in + off + 2, 2);
      });
  return ok();
}

int qgemm_affine_bits(const void* w_packed, const void* a, int M, int64_t K, int64_t N, int bits, void* out,
                      int out_dtype, void* stream) {
  REQUIRE_PTR(w_packed);
  REQUIRE_PTR(a);
  REQUIRE_PTR(out);
  if (!affine_bits_ok(bits)) return fail(Q4_ERR_UNSUPPORTED, "%s: bits=%d not in {2, 3, 5, 6, 8}", __func__, bits);
  if (M < 1 || M > 16) return fail(Q4_ERR_UNSUPPORTED, "%s: M=%d outside 1..16", __func__, M);
  if (int rc = check_nk(__func__, N, K, 64)) return rc;
  if (out_dtype != Q4_F32 && out_dtype != Q4_BF16)
    return fail(Q4_ERR_INVALID_ARG, "%s: out_dtype=%d is not Q4_F32 or Q4_BF16", __func__, out_dtype);
  REQUIRE_ALIGNED(w_packed);
  REQUIRE_ALIGNED(a);
  REQUIRE_ALIGNED(out);
  if (int e = launch_affine_bits(bits, static_cast<const uint8_t*>(w_packed), N, K, static_cast<const uint16_t*>(a), M,
                                 out, out_dtype, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

// ---- MoE block -----------------------------------------------------------
// The block's workspace: the experts' grouped-MoE workspace (sub2, which the
// router uses before them; at offset 0, so the router's arrival counter is in
// the buffer's counter region), the dense layer's (sub1: the grouped-MoE
// kernels use no counters, only scratch above the counter region, which needs
// no zero-fill), then the normed inputs and the routings.  The
// two expert layers' outputs stay in their own workspaces until the block's
// combine reads them.
struct BlockWs {
  size_t sub2, part, sub1, h1, h2, idx, w, didx, dw, total;
};
static size_t up256(size_t x) { return (x + 255) / 256 * 256; }
static BlockWs block_ws(const q4_moe_block_desc* b, int T, int k) {
  BlockWs L{};
  const int D = b->experts.D, E = b->experts.E;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  L.sub2 = take(std::max(moe_route_workspace_bytes(T, D, E), moe_workspace_bytes(&b->experts, T, k)));
  L.part = take(size_t(route_splits(D)) * size_t(T) * size_t(E) * sizeof(float));
  L.sub1 = take(moe_workspace_bytes(&b->dense, T, 1));
  L.h1 = take(size_t(T) * D * 2);
  L.h2 = take(size_t(T) * D * 2);
  L.idx = take(size_t(T) * k * 4);
  L.w = take(size_t(T) * k * 4);
  L.didx = take(size_t(T) * 4);
  L.dw = take(size_t(T) * 4);
  L.total = o;
  return L;
}

size_t moe_block_workspace_bytes(const q4_moe_block_desc* b, int T, int k) {
  if (!b || T < 1 || T > 64 || k < 1 || k > 64 || b->experts.D < 1 || b->experts.E < 1 || b->experts.F < 1 ||
      b->dense.F < 1)
    return 0;
  return block_ws(b, T, k).total;
}

int moe_block_forward(const q4_moe_block_desc* b, float* residual, int T, int k, int32_t* topk_idx_out,
                      float* topk_w_out, void* ws, size_t ws_bytes, void* stream) {
  // every refusal, of this entry and of the calls it makes below, comes
  // before the first launch: on error nothing is enqueued
  REQUIRE_PTR(b);
  REQUIRE_PTR(residual);
  REQUIRE_PTR(b->w_router);
  REQUIRE_PTR(b->router_scale);
  REQUIRE_PTR(b->ffn_norm);
  REQUIRE_PTR(b->post_ffw_norm_1);
  REQUIRE_PTR(b->pre_ffw_norm_2);
  REQUIRE_PTR(b->post_ffw_norm_2);
  REQUIRE_PTR(b->post_ffw_norm);
  if (!(b->eps > 0.0f && b->eps < 3.0e38f))
    return fail(Q4_ERR_INVALID_ARG, "%s: eps=%g must be finite and > 0", __func__, double(b->eps));
  if (b->experts.has_shared != 0)
    return fail(Q4_ERR_INVALID_ARG, "%s: the routed experts may not have a shared expert (the dense branch is it)",
                __func__);
  if (b->dense.E != 1 || b->dense.has_shared != 0 || b->dense.D != b->experts.D)
    return fail(Q4_ERR_INVALID_ARG, "%s: dense must be a one-expert layer (E=1, has_shared=0) of D=%d", __func__,
                b->experts.D);
  if (T < 1 || k < 1) return fail(Q4_ERR_INVALID_ARG, "%s: T=%d and k=%d must be positive", __func__, T, k);
  if (T > 16) return fail(Q4_ERR_UNSUPPORTED, "%s: T=%d outside 1..16", __func__, T);
  if (b->experts.E > 256) return fail(Q4_ERR_UNSUPPORTED, "%s: E=%d > 256", __func__, b->experts.E);
  if (b->experts.D > 4096) return fail(Q4_ERR_UNSUPPORTED, "%s: D=%d > 4096", __func__, b->experts.D);
  REQUIRE_ALIGNED(residual);
  if ((topk_idx_out && !aligned16(topk_idx_out)) || (topk_w_out && !aligned16(topk_w_out)))
    return fail(Q4_ERR_ALIGNMENT, "%s: topk_idx_out and topk_w_out must be 16-byte aligned", __func__);
  if (!ws) return fail(Q4_ERR_WORKSPACE, "%s: ws is NULL", __func__);
  REQUIRE_ALIGNED(ws);
  const BlockWs L = block_ws(b, T, k);
  if (ws_bytes < L.total) return fail(Q4_ERR_WORKSPACE, "%s: ws_bytes=%zu < %zu", __func__, ws_bytes, L.total);
  char* base = static_cast<char*>(ws);
  const int D = b->experts.D, E = b->experts.E;
  int32_t* idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t*>(base + L.idx);
  float* w = topk_w_out ? topk_w_out : reinterpret_cast<float*>(base + L.w);
  const void* h1 = base + L.h1;
  const void* h2 = base + L.h2;
  int32_t* didx = reinterpret_cast<int32_t*>(base + L.didx);
  float* dw = reinterpret_cast<float*>(base + L.dw);
  void* ws1 = base + L.sub1;
  void* ws2 = base + L.sub2;
  const size_t ws2_bytes = L.sub1 - L.sub2, ws1_bytes = L.h1 - L.sub1;
  // the expert layers leave their per-slot outputs in their workspaces (no
  // combine launch of their own); y is required by the checks, never written
  size_t h_off, o1_off, r1_off, g_off, o2_off, r2_off;
  (void)moe_ws_layout(&b->dense, T, 1, &h_off, &o1_off, &r1_off, &g_off);
  (void)moe_ws_layout(&b->experts, T, k, &h_off, &o2_off, &r2_off, &g_off);
  const float* o1 = reinterpret_cast<const float*>(static_cast<char*>(ws1) + o1_off);
  const float* o2 = reinterpret_cast<const float*>(static_cast<char*>(ws2) + o2_off);
  const int32_t* rowof2 = reinterpret_cast<const int32_t*>(static_cast<char*>(ws2) + r2_off);
  if (int rc = route_check(__func__, h2, b->w_router, T, D, E, k, nullptr, idx, w, ws2, ws2_bytes)) return rc;
  if (int rc = moe_check(__func__, &b->dense, h1, didx, dw, T, 1, residual, Q4_F32, ws1, ws1_bytes)) return rc;
  if (int rc = moe_check(__func__, &b->experts, h2, idx, w, T, k, residual, Q4_F32, ws2, ws2_bytes)) return rc;
  if (int e = launch_block_norm_in(residual, T, D, b->ffn_norm, b->pre_ffw_norm_2, b->eps, base + L.h1, base + L.h2,
                                   stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  // the router's partial logits in their own region: the routed gate/up
  // reads them while it writes the layers' scratch
  float* part = reinterpret_cast<float*>(base + L.part);
  const bool routed = moe_gu_route_fits(T, D, E);
  if (int rc = route_enqueue(__func__, h2, b->w_router, T, D, E, k, 0, nullptr, idx, w, ws2, stream, b, didx, dw,
                             part, routed))
    return rc;
  // the experts and the dense branch share the gate/up and the down launch
  MoeArgs me = moe_args(&b->experts, h2, idx, w, T, k, residual, Q4_F32, ws2, false);
  MoeArgs md = moe_args(&b->dense, h1, didx, dw, T, 1, residual, Q4_F32, ws1, false);
  if (routed) {  // gate/up takes the top-k from the partials; the dense branch's routing is constant
    me.rpart = part;
    me.rsplit = route_splits(D);
    me.zscale = b->router_scale;
    me.down_scale = b->down_scale;
    me.eps = b->eps;
    me.ridx = idx;
    me.rtw = w;
    md.rconst = 1;
    md.ridx = didx;
    md.rtw = dw;
  }
  if (int e = launch_moe(me, &md, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  if (int e = launch_block_combine(o1, o2, rowof2, k, T, D, b->post_ffw_norm_1, b->post_ffw_norm_2, b->post_ffw_norm,
                                   b->eps, residual, stream))
    return fail(Q4_ERR_HIP, "%s: kernel launch failed (hip error %d)", __func__, e);
  return ok();
}

}  // extern "C"
