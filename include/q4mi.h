/*
 * q4mi.h -- C ABI of libq4mi.so: W4A16 skinny GEMMs (NVFP4 and MLX-style
 * affine 4-bit) and a grouped top-k MoE layer for AMD MI355X (gfx950).
 *
 * Pages that define the operations:
 *   [README] gemma-cuda-hybrid README, "Everything it has" and "Why it's
 *            NVIDIA-only": NVFP4 W4A16 decode (E2M1 codes, E4M3 scale per
 *            16 weights, fp32 global scale), one GEMM for every M <= 16
 *            product, weights repacked offline into the matrix-unit operand
 *            order, a grouped MoE over 128 experts top-8 plus one shared.
 *   [ISSUE]  TensorFold issue "Proposal: Gemma 4 on CUDA", "Why now":
 *            qlinear's MLX affine 4-bit path (groups of 64), activation rows
 *            with 64-value group sums, tree_round's argmax; "Gates": the
 *            float64 bound per kernel.
 *   [DOC]    TensorSharp docs, Gemma 4, 3.2 "Per-layer (MoE)", 4.6 "MoE"
 *            and 14 "Completed: Expert-batched FFN (GEGLU)": router matmul,
 *            softmax, top-k, gated expert FFN, weighted combine.
 *
 * Conventions for every entry point:
 *   - Status: Q4_OK (0) or a negative Q4_ERR_*; q4_last_error() then holds a
 *     message naming the refused argument (thread-local, valid until this
 *     thread's next call).  On any error nothing has been enqueued, except
 *     Q4_ERR_HIP, which reports a failed launch.
 *   - Memory: the caller owns every buffer.  "host" pointers are CPU memory,
 *     "device" pointers are GPU memory of the current HIP device, 16-byte
 *     aligned.  Inputs are read only; outputs are fully overwritten and must
 *     not alias inputs.  The library allocates and frees nothing and never
 *     synchronizes: GPU entry points enqueue on `stream` (a hipStream_t; NULL
 *     is the null stream) and return.
 *   - Canonical weight layouts (row n = one output, groups run along K):
 *       NVFP4 codes  u8[N][K/2], element 2j in the low nibble of byte j;
 *             scales u8[N][K/16] (OCP E4M3FN bytes); global scale fp32.
 *       affine codes u8[N][K/2] (same nibble order); scale, bias bf16
 *             (uint16 bit patterns) [N][K/64]; w = q*scale + bias.
 *     The packed layouts produced by the repack calls are private to the
 *     library; only their byte sizes are part of the ABI.
 *   - Workspaces: an entry point that needs device scratch takes (ws,
 *     ws_bytes) and has a *_workspace_bytes query.  A workspace must be
 *     zero-filled before its first use.  Its first 32 KiB hold only counters,
 *     which every call leaves at zero; scratch lives above them.  One buffer
 *     of the largest queried size can therefore serve every entry point, as
 *     long as the calls that share it are ordered on one stream (calls that
 *     overlap in time on a shared workspace race).
 *   - Entries are re-entrant: any number of host threads may call them at
 *     once (each with its own workspace, or ordered on one stream).
 */
#ifndef Q4MI_H
#define Q4MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4MI_ABI_VERSION 4

enum {
  Q4_OK = 0,
  Q4_ERR_INVALID_ARG = -1, /* null pointer, bad size, bad enum value        */
  Q4_ERR_UNSUPPORTED = -2, /* shape outside what the kernels handle          */
  Q4_ERR_ALIGNMENT = -3,   /* device pointer not 16-byte aligned             */
  Q4_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the query    */
  Q4_ERR_HIP = -5          /* the HIP runtime reported an error at launch    */
};

enum { Q4_F16 = 1, Q4_BF16 = 2, Q4_F32 = 3 };

/* Version of this header's ABI (Q4MI_ABI_VERSION). */
int q4_abi_version(void);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* q4_last_error(void);

/* ---------------------------------------------------------------------------
 * Offline repack (host memory in and out, pure CPU, deterministic).
 * [README]: the weights are reordered once, offline, into the order in
 * which the matrix unit consumes them, so that the hot loop issues only wide
 * contiguous loads.  Here the order is that of the gfx950 16x16x32 MFMA B
 * operand: per 16 output rows, 128-k tiles of 1152 bytes (1 KiB of codes
 * where each lane's 16 bytes are one 16-byte load, then the tile's scales),
 * and one 576-byte half tile when K % 128 == 64.  A matrix whose panels end
 * in a half tile is followed by a 576-byte zero guard (part of the packed
 * size), so that a full-tile load issued at the last half tile stays inside
 * the buffer.
 * ------------------------------------------------------------------------- */

/* Bytes of the packed NVFP4 matrix [N][K]; 0 if N % 16 != 0, K % 16 != 0 or
 * either is not positive.  K is padded internally to a multiple of 64 with
 * zero codes and zero scales (which contribute exactly 0). */
size_t q4_nvfp4_packed_bytes(int64_t N, int64_t K);

/* Pack canonical NVFP4 (host codes u8[N][K/2], host scales u8[N][K/16])
 * into host `packed` of `packed_bytes` >= q4_nvfp4_packed_bytes(N, K).
 * Errors: INVALID_ARG (null, sizes), UNSUPPORTED (N % 16, K % 16). */
int q4_nvfp4_repack(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                    void* packed, size_t packed_bytes);

/* Inverse of q4_nvfp4_repack (host memory), for tests and inspection. */
int q4_nvfp4_unpack(const void* packed, int64_t N, int64_t K, uint8_t* codes, uint8_t* scales);

/* Bytes of device workspace q4_nvfp4_quantize needs when it computes the
 * global scale itself (one scratch word past the counter area). */
size_t q4_nvfp4_quantize_workspace_bytes(void);

/* NVFP4 quantizer on the device [README: the NVFP4 quantization kernel of
 * its kernel list; "Why it's NVIDIA-only": E2M1 x E4M3/16 x fp32 global].
 * Quantizes fp32 weights and writes them in the packed layout of
 * q4_nvfp4_repack (the result equals q4_nvfp4_repack of the codes and
 * scales it chose):
 *   g = global_scale if > 0, else amax|w| / (448 * 6) (fp32)
 *   s = E4M3(amax of the 16-group / 6 / g), nearest even, saturating at 448
 *   code = E2M1(w / (e4m3(s) * g)), nearest even, saturating at 6; +0 for a
 *          group whose decoded scale is 0
 * each step one fp32 operation in that order.
 *   w        device fp32 [N][K] row-major, 16-byte aligned, finite values
 *   packed   device buffer of packed_bytes >= q4_nvfp4_packed_bytes(N, K)
 *   g_out    device fp32[1] receiving g, or NULL
 *   ws       device workspace of q4_nvfp4_quantize_workspace_bytes() bytes
 *            when global_scale <= 0 (NULL otherwise); no zero-fill needed
 * Errors: INVALID_ARG (NULL w or packed, short packed buffer, non-finite
 * global_scale), UNSUPPORTED (N % 16, K % 16, K too large), ALIGNMENT,
 * WORKSPACE, HIP. */
int q4_nvfp4_quantize(const float* w, int64_t N, int64_t K, float global_scale, void* packed,
                      size_t packed_bytes, float* g_out, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the packed affine matrix [N][K]; 0 unless N % 16 == 0 and K % 64 == 0. */
size_t q4_affine4_packed_bytes(int64_t N, int64_t K);

/* Pack canonical affine 4-bit (host codes u8[N][K/2], scale and bias as bf16
 * bit patterns u16[N][K/64]) into host `packed`.  [ISSUE "Why now"]. */
int q4_affine4_repack(const uint8_t* codes, const uint16_t* scale_bf16, const uint16_t* bias_bf16,
                      int64_t N, int64_t K, void* packed, size_t packed_bytes);

/* Inverse of q4_affine4_repack (host memory). */
int q4_affine4_unpack(const void* packed, int64_t N, int64_t K, uint8_t* codes,
                      uint16_t* scale_bf16, uint16_t* bias_bf16);

/* ---------------------------------------------------------------------------
 * Skinny GEMMs.  y[m][n] = sum_k a[m][k] * w[n][k], 1 <= M <= 16 (NVFP4
 * also more rows, see qgemm_nvfp4).
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace qgemm_nvfp4 needs for this shape (0 if none):
 * the fused argmax's counter and keys, and, for shapes whose K is split
 * across workgroups, the fp32 partial sums and their arrival counters.
 * Depends only on (M, K, N, want_argmax) and the Q4MI_GEMM_CFG override. */
size_t qgemm_nvfp4_workspace_bytes(int M, int64_t K, int64_t N, int want_argmax);

/* Same for qgemm_affine4. */
size_t qgemm_affine4_workspace_bytes(int M, int64_t K, int64_t N);

/* NVFP4 W4A16 GEMM [README "Everything it has": the M <= 16 GEMM with
 * in-register FP4 -> f16 dequant; "Why it's NVIDIA-only": E2M1 x E4M3/16 x
 * fp32 global].  Each weight is e2m1(code) * e4m3(scale) * global_scale.
 * More rows (17 <= M <= 65536, argmax NULL) -- prompt chunks and large
 * verify blocks [README, repository layout: the engine's prefill beside
 * decode; DOC 3.3 "Decode vs prefill": prefill runs many tokens at once]
 * -- run a
 * matrix-core kernel with 64 x 128 output blocks; it needs no workspace
 * (the query returns 0) and its results obey the same error bound.
 *   w_packed  device, from q4_nvfp4_repack of the [N][K] weights
 *   a         device f16 [M][K] row-major
 *   out       device [M][N] row-major of out_dtype (Q4_F32, Q4_F16 or Q4_BF16)
 *   argmax    device int32[M] or NULL (M <= 16 only).  If set, argmax[m] is the index of the
 *             largest value of row m of `out` as stored, lowest index on ties,
 *             NaN values skipped (-1 if the whole row is NaN) -- tree_round's
 *             argmax of [ISSUE "Why now"], fused into the GEMM.
 *   ws        device workspace of ws_bytes >= the query (NULL if the query is
 *             0); it must be zero-filled before its first use, and every call
 *             leaves its counters at zero again.
 * Errors: INVALID_ARG, UNSUPPORTED (M outside 1..16 with argmax, outside
 * 1..65536 without, N % 16, K % 16), ALIGNMENT, WORKSPACE, HIP. */
int qgemm_nvfp4(const void* w_packed, float global_scale, const void* a, int M, int64_t K,
                int64_t N, void* out, int out_dtype, int32_t* argmax, void* ws, size_t ws_bytes,
                void* stream);

/* NVFP4 lm_head with fused sampling: the GEMM of qgemm_nvfp4, then per row
 * one token.  [DOC 4.8 "Logit softcap"]: z = softcap * tanh(y / softcap) if
 * softcap > 0, else z = y.  [README "Everything it has"]: temperature
 * sampling by the Gumbel-max trick, temperature 0 being greedy:
 *   token[m] = argmax_n (z[m][n] / temperature + G[m][n])   (temperature > 0)
 *   token[m] = argmax_n z[m][n]                              (temperature == 0)
 * in fp32, lowest index on ties, NaN scores skipped (-1 if all are NaN).
 * G = -ln(-ln U), U = (2 (x >> 9) + 1) 2^-24 from Philox4x32-10 (Salmon et
 * al., SC 2011) with key (seed & 0xffffffff, seed >> 32), counter (n, m / 4,
 * offset, 0), word m % 4.  Advance `offset` (or change the seed) per step.
 *   logits   device [M][N] of out_dtype (Q4_F32, Q4_F16, Q4_BF16) receiving z,
 *            or NULL to skip storing the logits
 *   token    device int32[M]
 *   ws       as for qgemm_nvfp4 with want_argmax = 1
 * Errors: as qgemm_nvfp4; INVALID_ARG also for temperature < 0, NaN or inf,
 * a NaN or infinite softcap, or a NULL token. */
int qgemm_nvfp4_sample(const void* w_packed, float global_scale, const void* a, int M, int64_t K,
                       int64_t N, float softcap, float temperature, uint64_t seed, uint32_t offset,
                       void* logits, int out_dtype, int32_t* token, void* ws, size_t ws_bytes,
                       void* stream);

/* MLX-style affine 4-bit W4A16 GEMM [ISSUE "Why now": qlinear's affine
 * path in groups of 64 with activation group sums].  w = q*scale + bias per
 * 64 weights along K; the product is computed as
 *   sum_g scale[n,g] * sum_{k in g} a[m,k] q[n,k] + bias[n,g] * sum_{k in g} a[m,k].
 *   w_packed  device, from q4_affine4_repack
 *   a         device bf16 [M][K] row-major
 *   out       device [M][N] of out_dtype (Q4_F32 or Q4_BF16)
 *   ws        device workspace of ws_bytes >= qgemm_affine4_workspace_bytes
 *             (NULL if that is 0), zero-filled before first use as above
 * Errors: INVALID_ARG, UNSUPPORTED (M outside 1..16, N % 16, K % 64),
 * ALIGNMENT, WORKSPACE, HIP. */
int qgemm_affine4(const void* w_packed, const void* a, int M, int64_t K, int64_t N, void* out,
                  int out_dtype, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Top-k MoE.  [DOC 3.2, 4.6]; [README]: 128 experts, top-8, one shared.
 * ------------------------------------------------------------------------- */

/* Bytes of device workspace moe_route_topk needs. */
size_t moe_route_workspace_bytes(int T, int D, int E);

/* Router: logits[t][e] = sum_d x[t][d] * w_router[d][e] in fp32; the k
 * experts with the largest logits (decreasing, ties to the lower index);
 * their softmax probabilities over all E experts (renormalized to sum 1 over
 * the k if `renormalize`).
 *   x        device f16 [T][D];  w_router device fp32 [D][E]
 *   logits   device fp32 [T][E] or NULL
 *   topk_idx device int32 [T][k];  topk_w device fp32 [T][k]
 *   ws       device workspace (see above: its counters start at zero and are
 *            left at zero)
 * Errors: INVALID_ARG, UNSUPPORTED (T outside 1..64, E outside 1..256,
 * k > E or k > 16, D % 8, D > 12288),
 * ALIGNMENT, WORKSPACE, HIP. */
int moe_route_topk(const void* x, const float* w_router, int T, int D, int E, int k,
                   int renormalize, float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                   size_t ws_bytes, void* stream);

/* Expert weights of one MoE layer.  Experts 0..E-1 are routed; if has_shared,
 * expert E is the shared expert that every token uses with weight 1.
 * gate/up are [F][D] and down is [D][F] per expert, each packed with
 * q4_nvfp4_repack and stored expert after expert (stride
 * q4_nvfp4_packed_bytes of the matrix).  g_* are device fp32 arrays of the
 * per-matrix global scales, one per expert (E + has_shared entries). */
typedef struct {
  int E, has_shared, D, F;
  const void* gate_packed;
  const void* up_packed;
  const void* down_packed;
  const float* g_gate;
  const float* g_up;
  const float* g_down;
} q4_moe_desc;

/* Bytes of device workspace moe_grouped_qgemm needs for T tokens, top-k. */
size_t moe_workspace_bytes(const q4_moe_desc* w, int T, int k);

/* Grouped MoE expert FFN [README "Everything it has": grouped, weight-resident
 * MoE without atomics; DOC 14: expert-batched GEGLU].  For each token t:
 *   y[t] = sum_{j<k} topk_w[t][j] * FFN_{topk_idx[t][j]}(x[t]) + FFN_shared(x[t])
 *   FFN_e(v) = W_down,e (gelu_tanh(W_gate,e v) * (W_up,e v))
 * The (token, slot) pairs are grouped by expert on the device so each active
 * expert's weights are streamed once; h is kept in f16 between the two
 * projections; the combine sums in a fixed order (deterministic).
 *   x        device f16 [T][D]; topk_idx device int32 [T][k] (each in 0..E-1);
 *   topk_w   device fp32 [T][k]; y device [T][D] of out_dtype (Q4_F32, Q4_F16)
 *   ws       device workspace of ws_bytes >= moe_workspace_bytes (scratch for
 *            h and the per-pair expert outputs; no zero-fill needed)
 * Errors: INVALID_ARG, UNSUPPORTED (T outside 1..16, k outside 1..min(E, 64),
 * D % 64, F % 64, E > 1024), ALIGNMENT, WORKSPACE, HIP.  Expert indices live
 * on the device and are not validated: pairs whose index is outside 0..E-1
 * are dropped, and so are pairs beyond the 16th routed to one expert (only
 * possible if a token names the same expert twice). */
int moe_grouped_qgemm(const q4_moe_desc* w, const void* x, const int32_t* topk_idx,
                      const float* topk_w, int T, int k, void* y, int out_dtype, void* ws,
                      size_t ws_bytes, void* stream);

/* moe_grouped_qgemm without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same kernels and results, with
 * their scratch (h, the per-pair outputs, the expert grouping) in an 8 MiB
 * array that the library keeps on each GPU it runs on until the process
 * ends.  The call allocates nothing; the caller passes the inputs and y as
 * for moe_grouped_qgemm.  All calls on one GPU share that GPU's array, so
 * calls that overlap in time on one GPU (other streams, other threads)
 * race; calls ordered on one stream do not.  The array needs no clearing:
 * every call writes all the scratch it reads.
 * Errors: those of moe_grouped_qgemm (no WORKSPACE), and UNSUPPORTED when
 * moe_workspace_bytes(w, T, k) exceeds 8 MiB (T = 16, k = 16 fit up to
 * D = F = 4096). */
int moe_grouped_qgemm_noalloc(const q4_moe_desc* w, const void* x, const int32_t* topk_idx,
                              const float* topk_w, int T, int k, void* y, int out_dtype, void* stream);

/* Bytes of device workspace moe_route_grouped_qgemm needs (0 if E > 256):
 * moe_workspace_bytes plus the router's partial logits. */
size_t moe_route_grouped_workspace_bytes(const q4_moe_desc* w, int T, int k);

/* The router and the grouped MoE layer in one call [DOC 3.2 "Per-layer
 * (MoE)": router matmul, softmax, top-k, then the chosen experts' FFNs
 * summed with the routing weights]: the results of moe_route_topk(x,
 * w_router, T, w->D, w->E, k, renormalize, logits, topk_idx, topk_w)
 * followed by moe_grouped_qgemm(w, x, topk_idx, topk_w, T, k, y).  The
 * router kernel writes only its partial logits; every gate/up workgroup
 * sums them (in the router's order, so the logits are the same bits) and
 * takes the top-k and softmax itself before building the expert grouping,
 * one launch and one cross-workgroup handoff fewer than the two calls (the
 * same indices; the weights equal moe_route_topk's up to the order of the
 * softmax sums).  Shapes whose scores do not fit the gate/up launch's LDS
 * beside x (E % 4 != 0, or T E too large) take the two calls' path.
 *   x, w_router, logits (or NULL), topk_idx, topk_w  as for moe_route_topk
 *            (topk_idx and topk_w are outputs here)
 *   y, out_dtype  as for moe_grouped_qgemm
 *   ws       device workspace of ws_bytes >= moe_route_grouped_workspace_bytes,
 *            its first 32 KiB of counters at zero (left at zero)
 * Errors: those of moe_route_topk and moe_grouped_qgemm; nothing is
 * enqueued on an error other than HIP. */
int moe_route_grouped_qgemm(const q4_moe_desc* w, const void* x, const float* w_router, int T, int k,
                            int renormalize, float* logits, int32_t* topk_idx, float* topk_w, void* y,
                            int out_dtype, void* ws, size_t ws_bytes, void* stream);

/* MLX-style affine weights at 2, 3, 5, 6 or 8 bits [ISSUE "Why now":
 * qlinear's MLX affine paths at 2, 3, 5, 6 and 8 bits beside 4, groups of
 * 64; "Steps" 3 and 9: the other MLX widths; the 4-bit width has the entry
 * points above].  w = q * scale + bias per 64-value group.
 *   codes  host u8 [N][K], one code per byte, each < 2^bits
 *   scale_bf16, bias_bf16  host bf16 bit patterns [N][K/64]
 * Packed layout: per 16-row panel, 128-k tiles (K padded to 128 with zero
 * codes and zero scale/bias) of 256 * bits code bytes, lane (c, o) of the
 * MFMA (lane 16 o + c) owning 4 * bits bytes that hold row c's codes at
 * k = 32 i + 8 o + j as one little-endian bit stream (code (i, j) at bit
 * 8 bits i + bits j), stored in pieces of P = 16 (bits 8), 8 (bits 2, 6)
 * or 4 (bits 3, 5) bytes: piece j of lane l at byte 64 P j + P l of the
 * tile; then 128 bytes of (bf16 scale | bf16 bias << 16) words, row c's two
 * groups at 8 c.  packed_bytes = N / 16 * ceil(K / 128) * (256 bits + 128).
 * Errors: INVALID_ARG (NULL, short buffer, a code >= 2^bits), UNSUPPORTED
 * (bits, N % 16, K % 64). */
size_t q4_affine_bits_packed_bytes(int64_t N, int64_t K, int bits);
int q4_affine_bits_repack(const uint8_t* codes, const uint16_t* scale_bf16, const uint16_t* bias_bf16, int64_t N,
                          int64_t K, int bits, void* packed, size_t packed_bytes);
int q4_affine_bits_unpack(const void* packed, int64_t N, int64_t K, int bits, uint8_t* codes,
                          uint16_t* scale_bf16, uint16_t* bias_bf16);

/* y[m][n] = sum_k a[m][k] * (q[n][k] * s + b) for the b-bit layout above,
 * 1 <= M <= 16, fp32 accumulation; no workspace.
 *   w_packed device, from q4_affine_bits_repack;  a device bf16 [M][K]
 *   out      device [M][N] of out_dtype (Q4_F32 or Q4_BF16)
 * Errors: INVALID_ARG, UNSUPPORTED (bits, M, N % 16, K % 64), ALIGNMENT, HIP. */
int qgemm_affine_bits(const void* w_packed, const void* a, int M, int64_t K, int64_t N, int bits, void* out,
                      int out_dtype, void* stream);

/* The whole Gemma-4 MoE block around the experts [DOC 3.2 "Per-layer (MoE)",
 * DOC 4.6 "MoE"; DOC 14 "Completed": ffn_down_exps.scale folded into the
 * routing weights].  With RMSNorm(v; w) = v / sqrt(mean(v^2) + eps) * w per
 * token row:
 *   h1 = RMSNorm(r; ffn_norm)                b1 = dense FFN(h1)
 *   h2 = RMSNorm(r; pre_ffw_norm_2)          z  = RMSNorm(h2 . W_r; 1) * router_scale
 *   idx = top-k of softmax(z) (ties to the lower index), w = softmax(z)[idx] * down_scale[idx]
 *   b2 = sum_j w_j FFN_idx_j(h2)
 *   r += RMSNorm(RMSNorm(b1; post_ffw_norm_1) + RMSNorm(b2; post_ffw_norm_2); post_ffw_norm)
 * The FFNs are those of moe_grouped_qgemm (gated GELU-tanh, h in f16); h1 and
 * h2 enter them as f16. */
typedef struct {
  q4_moe_desc experts;        /* routed experts, has_shared = 0 */
  q4_moe_desc dense;          /* the dense branch as a one-expert layer: E = 1, has_shared = 0,
                                 F = its width, same D */
  const float* w_router;      /* device fp32 [D][E] */
  const float* router_scale;  /* device fp32 [E] (ffn_gate_inp.scale) */
  const float* down_scale;    /* device fp32 [E] (ffn_down_exps.scale) or NULL for 1 */
  const float* ffn_norm;      /* device fp32 [D] each */
  const float* post_ffw_norm_1;
  const float* pre_ffw_norm_2;
  const float* post_ffw_norm_2;
  const float* post_ffw_norm;
  float eps;                  /* RMSNorm epsilon (> 0; 1e-6 in the tests) */
} q4_moe_block_desc;

/* Bytes of device workspace moe_block_forward needs (0 on invalid shapes). */
size_t moe_block_workspace_bytes(const q4_moe_block_desc* b, int T, int k);

/* One MoE block on the residual stream, in place.
 *   residual     device fp32 [T][D], updated r <- r + update
 *   topk_idx_out device int32 [T][k] receiving the experts the block chose
 *                (decreasing z, ties to the lower index), or NULL
 *   topk_w_out   device fp32 [T][k] receiving their weights
 *                softmax(z)[idx] * down_scale[idx], or NULL; with these, a
 *                caller sees the routing the outputs were computed with
 *                (several are valid where scores tie within rounding)
 *   ws           device workspace of ws_bytes >= moe_block_workspace_bytes;
 *                its first 32 KiB of counters start and end at zero, as for
 *                the other entry points
 * The block runs 5 launches on `stream`: the two input norms, the router
 * (moe_route_topk's kernel, writing its partial logits), one gate/up and
 * one down launch of moe_grouped_qgemm's kernels that serve both the
 * experts and the dense branch (each layer in its own part of the
 * workspace; every gate/up workgroup normalizes and scales the scores and
 * takes the top-k itself, as moe_route_grouped_qgemm does), and the
 * combine, which sums each token's expert outputs itself.
 * Errors: INVALID_ARG (NULL pointers, eps <= 0 or not finite, dense not a
 * one-expert layer, D mismatch, has_shared set, T or k < 1), UNSUPPORTED
 * (T > 16, E > 256, D > 4096), the errors of moe_route_topk and
 * moe_grouped_qgemm for these shapes (k > min(E, 16), D % 64, F % 64, ...),
 * ALIGNMENT, WORKSPACE, HIP.  Every refusal happens before the first
 * launch. */
int moe_block_forward(const q4_moe_block_desc* b, float* residual, int T, int k, int32_t* topk_idx_out,
                      float* topk_w_out, void* ws, size_t ws_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Test exports: the same device dequantization the GEMMs use, written out.
 * ------------------------------------------------------------------------- */

/* out[m][n] (device fp32 [M][N]) = the uniform U that qgemm_nvfp4_sample
 * draws for row m, column n with this seed and offset. */
int q4_sample_uniforms(uint64_t seed, uint32_t offset, int M, int64_t N, float* out, void* stream);

/* out[n][k] (device fp32 [N][K]) = fp32(e2m1 * e4m3 * g) from the packed matrix. */
int q4_dequant_nvfp4(const void* w_packed, float global_scale, int64_t N, int64_t K, float* out,
                     void* stream);

/* out[n][k] (device fp32 [N][K]) = fmaf(q, scale, bias) from the packed matrix. */
int q4_dequant_affine4(const void* w_packed, int64_t N, int64_t K, float* out, void* stream);

/* ---------------------------------------------------------------------------
 * Measurement export.  [README "Why it's NVIDIA-only": the kernels are tuned
 * against the bandwidth the memory really delivers.]  The stream-read
 * ceiling: reads `bytes` of device memory at `src` with the loads the
 * weight-streaming kernels issue (16-byte non-temporal loads, each wave
 * instruction covering 1 KiB) and nothing else, so that its duration is the
 * floor for streaming that many bytes.
 *   src    device, 16-byte aligned, `bytes` readable (a positive multiple of 16)
 *   grid   workgroups of 256 threads, 1..65536
 *   mode   0: grid-stride (consecutive waves read consecutive KiB);
 *          1: workgroup b reads the b-th of `grid` contiguous chunks;
 *          2: one batch per lane: 512-thread workgroups, workgroup b
 *             reading the b-th of `grid` contiguous chunks (at most 256 KiB
 *             each), every lane issuing all its loads at once
 *   depth  loads per lane per batch in modes 0 and 1 (1, 2, 4 or 8), each
 *          lane keeping two batches in flight; ignored in mode 2
 *   out    device u32[grid]: the XOR of each workgroup's words
 * Errors: INVALID_ARG (NULL, bytes, grid, mode, depth), ALIGNMENT, HIP. */
int q4_stream_read(const void* src, size_t bytes, int grid, int mode, int depth, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* Q4MI_H */
