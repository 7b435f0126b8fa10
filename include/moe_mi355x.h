/*
 * moe_mi355x.h -- C ABI of the MI355X (gfx950) routed-expert MoE FFN library
 * (libmoe_mi355x.so).
 *
 * The library runs one Hy4-shaped MoE layer on packed low-bit expert weights: a
 * bf16 router picks k of E routed experts per token, the routed SwiGLU experts run
 * directly on STQ1_0 or MXFP4 weights, one bf16 shared expert runs on every token,
 * and the outputs are combined.  Shapes follow "Hy4-preview Flash-MoE STQ1_0"
 * (anemll), Package details table: 256 routed experts per MoE block, 8 selected
 * per token, 1 shared expert, embedding width 6144, MoE intermediate width 2048.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller.  The library never
 *   allocates, frees or keeps any of them; it only enqueues kernels.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Every
 *   call is asynchronous on that stream; the host never waits inside a call.
 * - Return codes report the synchronous argument checks (null pointers, shapes the
 *   kernels do not support, short workspaces) and launch errors.  A fault inside a
 *   kernel surfaces as MOE_ERR_HIP on a later call or at the caller's next
 *   synchronisation.  With the environment variable MOE_MI355X_DEBUG_SYNC=1 every
 *   call synchronises its stream and reports such faults itself.
 * - Inputs are never written.  Outputs must not alias inputs, except that
 *   `residual` may equal `out_f32` in moe_combine.
 * - bf16 and fp16 values travel as their uint16_t bit patterns.
 * - The library keeps no state between calls apart from the path counters of
 *   moe_get_counters (atomically updated; calls on different streams are safe).
 *
 * Weight layouts (expert-major: expert e's matrix follows expert e-1's)
 * -------------------------------------------------------------------
 * STQ1_0 ("Hy4-preview-GGUF" (AngelSlim) section 3, The format; "Hy4-preview
 * Flash-MoE STQ1_0", How the STQ1_0 packing works): 256-weight blocks of 64 groups
 * of four weights; each group has exactly one zero and three values in {-d,+d};
 * one binary16 scale d per block; 42 bytes per 256 weights.  Our bit layout of the
 * 5-bit group pattern p = 8*z + s (z = zero lane 0..3, bit i of s = 1 when the i-th
 * non-zero lane in ascending lane order is -d):
 *   codes  : 40 bytes per block -- bytes 0..31: byte i = (p[2i] & 15) | (p[2i+1] & 15) << 4;
 *            bytes 32..39: little-endian 64-bit word, bit g = p[g] >> 4.
 *   scales : one uint16 (binary16 bits) per block, same block order.
 *   Blocks run over the row-major [out][in] matrix, flattened, so a matrix of n
 *   weights owns n/256 blocks (n % 256 == 0).
 * MXFP4 ("Hy4-preview-SF-WFP4AFP8" (siliconflow), Quant Diff table: FP4 E2M1
 * weights, group 32, UE8M0 scales):
 *   codes  : [out][in/2] bytes, element 2i in the low nibble (E2M1: bit 3 sign).
 *   scales : [out][in/32] UE8M0 bytes (value 2^(v-127)), groups along `in`.
 * MXFP4_TILED: the MXFP4 bytes of each matrix reordered for the prefill GEMMs' matrix
 * cores (made by moe_mxfp4_pack_tiles; same values, same size).  With R = out and
 * S = in/128 K steps, for tile t < R/16, step j < S, lane l < 64:
 *   codes  : bytes 1024*(t*S + j) + 16*l .. +15 = row 16t + l%16, codes bytes
 *            64j + 16*(l/16) .. +15 of that row in the MXFP4 layout;
 *   scales : bytes 64*(t*S + j) + 4*r .. +3 = row 16t + r, scale bytes 4j .. 4j+3.
 *   Needs out % 16 == 0 and in % 128 == 0.
 * BF16 (shared expert, router): [out][in] uint16 bf16 bits.
 * Gate and up are [I][H] (out = I, in = H); down is [H][I].
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_MI355X_API __attribute__((visibility("default")))

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad or inconsistent shape            */
  MOE_ERR_UNSUPPORTED = 2,  /* valid request this build has no kernel for         */
  MOE_ERR_WORKSPACE = 3,    /* workspace missing or smaller than moe_workspace_size */
  MOE_ERR_HIP = 4           /* a HIP runtime call or kernel launch failed         */
} moe_status;

typedef enum { MOE_W_STQ1_0 = 1, MOE_W_MXFP4 = 2, MOE_W_BF16 = 3, MOE_W_MXFP4_TILED = 4,
               MOE_W_MXFP8 = 5 } moe_wfmt;
/* MOE_W_MXFP8 (shared expert only; "Hy4-preview-SF-WFP4AFP8", Quant Diff table: the shared
 * experts' gate/up/down are MXFP8 W8A8 group 32): codes [N][K] E4M3 bytes (0x7F / 0xFF,
 * the NaN codes, are not valid weights), scales [N][K/32] UE8M0 bytes. */

/* Layer dimensions: T tokens, hidden H, expert intermediate I, E routed experts,
 * k experts per token.  Limits: 1 <= k <= min(E, 32), E <= 1024, H % 32 == 0,
 * I % 32 == 0; STQ1_0 needs (I*H) % 256 == 0; MXFP4 and MXFP4_TILED need H % 128 == 0
 * and I % 128 == 0.  T == 0 is allowed and enqueues nothing. */
typedef struct { int32_t T, H, I, E, k; } moe_dims;

/* One weight family (gate, up or down) of `n` experts, expert-major. */
typedef struct { const void* codes; const void* scales; } moe_mat;

/* The three families of a set of experts (E routed experts, or 1 shared). */
typedef struct {
  int32_t fmt;          /* moe_wfmt of all three families                      */
  int32_t reserved;
  moe_mat gate, up, down;
} moe_experts;

/* Counter slots of moe_get_counters. */
enum {
  MOE_CNT_ROUTE_GEMV = 0,      /* router logits computed from x             */
  MOE_CNT_ROUTE_TOPK = 1,      /* top-k launches                            */
  MOE_CNT_PERMUTE = 2,
  MOE_CNT_STQ_GATEUP_MFMA = 3, /* STQ1_0 fused-decode gate/up, MFMA path    */
  MOE_CNT_STQ_DOWN_MFMA = 4,
  MOE_CNT_STQ_GENERIC = 5,     /* STQ1_0 slow path (blocks straddling rows) */
  MOE_CNT_MX_QUANT = 6,
  MOE_CNT_MX_GATEUP_MFMA = 7,
  MOE_CNT_MX_DOWN_MFMA = 8,
  MOE_CNT_BF16_GATEUP = 9,     /* shared expert                             */
  MOE_CNT_BF16_DOWN = 10,
  MOE_CNT_COMBINE = 11,
  MOE_CNT_RMSNORM = 12,
  MOE_CNT_DEQUANT = 13,
  MOE_CNT_BF16_GEMM = 14,      /* shared expert, prefill grouped GEMM path  */
  MOE_CNT_DECODE_FUSED = 15,   /* moe_layer_decode (fused kernels)          */
  MOE_CNT_STQ_GEMM = 16,       /* STQ1_0 prefill grouped GEMMs (fp16 MFMA)  */
  MOE_CNT_ROWSCALE = 17,       /* activation rows to fp16 / bf16 hi + lo    */
  MOE_CNT_MXFP8_SHARED = 18,   /* MXFP8 shared expert GEMMs (gate/up, down) */
  MOE_CNT_SLOTS = 19
};

MOE_MI355X_API const char* moe_status_str(moe_status s);
MOE_MI355X_API const char* moe_version(void);

/* Path counters: out[MOE_CNT_SLOTS] receives how many times each kernel variant
 * was launched since load or the last reset (host-side counts, no device work). */
MOE_MI355X_API moe_status moe_get_counters(uint64_t* out);
MOE_MI355X_API moe_status moe_reset_counters(void);

/* Opt-in kernel timing: while enabled the library records a HIP event pair on the launch
 * stream around each of its main kernels (slots: 0..3 the kernels of moe_layer_decode -- routing,
 * gate/up, down, and beyond 4 tokens the separate combine --, 4/5/6 MX quantisation, MXFP4
 * gate/up and down GEMMs, 7/8 the STQ1_0
 * prefill gate/up and down GEMMs, 9/10 the shared expert's prefill gate/up and down GEMMs,
 * 11 the activation conversions of the prefill GEMMs).  Enabling
 * creates the event pools once (host objects, no device memory).  moe_profile_read waits
 * for the recorded events, writes the average duration in microseconds and the number of
 * launches per slot (16 slots) and clears the records.  Timing adds two event records per
 * kernel; leave it off outside measurement. */
MOE_MI355X_API moe_status moe_profile_enable(int32_t on);
MOE_MI355X_API moe_status moe_profile_read(double* avg_us, int64_t* count);

/* ---------------------------------------------------------------------------
 * Route.  Router logits l[t][e] = sum_h x[t][h] * Wr[e][h] (+ logit_bias[e]) in
 * fp32 from bf16 operands (the router stays BF16: "Hy4-preview-SF-WFP4AFP8", BF16
 * row of the Quant Diff table), then the k largest logits per token ("Hy4-preview
 * Flash-MoE STQ1_0": 8 selected experts per token, --moe-topk 8).  The pages give
 * no routing function; this library takes softmax over all experts, keeps the top
 * k and renormalises, i.e. topk_w[t][j] = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 * over the selected slots.  Slots are ordered by descending logit, ties to the
 * lower expert index.  A NaN logit ranks above every number and all NaNs tie (a NaN
 * in x[t] makes the row NaN: experts 0 .. k-1 are selected, with NaN weights), so
 * every id is in [0, E).  Without logits_in, T is at most 524280 (MOE_ERR_UNSUPPORTED
 * past it).
 *   x_bf16      [T][H] bf16, ignored when logits_in != NULL
 *   wr_bf16     [E][H] bf16, ignored when logits_in != NULL
 *   logit_bias  [E] fp32 or NULL (added to the logits in both modes)
 *   logits_in   [T][E] fp32 or NULL: when given, the router GEMV is skipped
 *   logits_out  [T][E] fp32 or NULL: receives the (biased) logits
 *   topk_ids    [T][k] int32 out, topk_w [T][k] fp32 out
 * ------------------------------------------------------------------------- */
MOE_MI355X_API moe_status moe_route(const moe_dims* d, const uint16_t* x_bf16,
                                    const uint16_t* wr_bf16, const float* logit_bias,
                                    const float* logits_in, float* logits_out,
                                    int32_t* topk_ids, float* topk_w, void* stream);

/* ---------------------------------------------------------------------------
 * Permute: group the P = T*k (token, slot) pairs by expert, stably, so each
 * expert's rows are contiguous (the expert-major order the Flash-MoE sidecar
 * streams).  Pair f = t*k + j.  expert_offsets[e] = number of pairs with expert
 * below e (expert_offsets[E] = P); within one expert pairs keep increasing f;
 * sorted_pair[pos] = f and pair_pos[f] = pos.  Deterministic (no atomics decide
 * the order).  A pair whose id lies outside [0, E) (moe_route never gives one;
 * moe_remap_ids gives -1 for an expert without a slot) is not routed: pair_pos[f] = -1,
 * expert_offsets[E] counts only the routed pairs, sorted_pair is -1 from
 * expert_offsets[E] on, moe_expert_ffn never sees the pair and moe_combine adds
 * nothing for it.  One workgroup; no workspace.
 *   topk_ids [P] int32; sorted_pair [P], expert_offsets [E+1], pair_pos [P] int32 out
 * ------------------------------------------------------------------------- */
MOE_MI355X_API moe_status moe_permute(const moe_dims* d, const int32_t* topk_ids,
                                      int32_t* sorted_pair, int32_t* expert_offsets,
                                      int32_t* pair_pos, void* stream);

/* Workspace bytes moe_expert_ffn needs for routed format `routed_fmt` with or
 * without a shared expert (host-only, no device work). */
MOE_MI355X_API moe_status moe_workspace_size(const moe_dims* d, int32_t routed_fmt,
                                             int32_t has_shared, size_t* bytes);

/* Byte offsets of the workspace regions, so tests can read the intermediates:
 *   offs[0] h of the routed pairs, fp32 [P][I] (STQ1_0 path)
 *   offs[1] h of the shared expert, fp32 [T][I]
 *   offs[2] x as E4M3 codes [T][H]          (MXFP4 and MXFP4_TILED paths)
 *   offs[3] x UE8M0 scales  [T][H/32]       (MXFP4 path)
 *   offs[4] h as E4M3 codes [P][I]          (MXFP4 path, sorted-pair order)
 *   offs[5] h UE8M0 scales  [P][I/32]       (MXFP4 path)
 *   offs[6] total bytes
 * Unused regions get offset (size_t)-1. */
MOE_MI355X_API moe_status moe_workspace_offsets(const moe_dims* d, int32_t routed_fmt,
                                                int32_t has_shared, size_t* offs);

/* ---------------------------------------------------------------------------
 * Expert FFN.  For every routed pair at sorted position pos (token t =
 * sorted_pair[pos] / k, expert e with expert_offsets[e] <= pos < expert_offsets[e+1]):
 *   g = Wg[e] a_t,  u = Wu[e] a_t,  h = silu(g) * u,  y_pairs[pos] = Wd[e] h
 * (SwiGLU expert MLP: gate_proj / up_proj / down_proj of the routed experts).
 *   STQ1_0: a_t = bf16 x[t]; weights decoded in registers; fp32 accumulation;
 *           h kept in fp32.
 *   MXFP4:  a_t = x[t] MX-quantised to E4M3 with group-32 UE8M0 scales along H, and
 *           h MX-quantised the same way along I before the down projection (every
 *           routed-expert linear of the WFP4AFP8 recipe takes FP8 E4M3 group-32
 *           activations); FP8 x FP4 products on the scaled MFMA, fp32 accumulation.
 *   MXFP4_TILED: the MXFP4 computation, bit for bit, on weights in the tiled layout
 *           (the layout the GEMMs stream fastest; the MXFP4 path reads row-major rows).
 * Kernels by token count: MXFP4 always runs the grouped GEMMs; STQ1_0 runs the decode-shaped
 * kernels below 128 tokens and grouped GEMMs on the fp16 MFMA from 128 (x scaled per row by
 * a power of two into fp16, h as fp16 hi + lo: results within the same tolerance); the bf16
 * shared expert switches at 256 tokens.  The environment variable MOE_MI355X_PREFILL_MIN_T,
 * read once, overrides both thresholds (measurement).
 * When `shared` is non-NULL (one expert) y_shared[t] = the same SwiGLU for every token:
 *   MOE_W_BF16: bf16 weights on bf16 x[t], h kept in fp32;
 *   MOE_W_MXFP8: W8A8 -- x[t] MX-quantised to E4M3 along H and h along I, as for MXFP4
 *           routed experts; E4M3 x E4M3 products (exact in the bf16 MFMA), fp32 sums.
 *           Runs on the prefill GEMMs at every token count.
 *   x_bf16 [T][H]; sorted_pair [P]; expert_offsets [E+1] (from moe_permute)
 *   y_pairs [P][H] fp32 out (sorted-pair order); y_shared [T][H] fp32 out or NULL
 *   ws / ws_bytes: device workspace of at least moe_workspace_size bytes.
 * Size limits (MOE_ERR_UNSUPPORTED past them; split the tokens over several calls):
 * every activation operand of the grouped GEMMs stays within 2^31 bytes -- routed STQ1_0
 * 2 T H and 4 P I, routed MXFP4 T H and P I, a shared expert on the GEMMs 2 T H and 4 T I
 * (at hidden 6144, intermediate 2048, top-8: 32768 tokens for STQ1_0, 131072 for MXFP4,
 * 174762 for the shared expert); the decode-shaped kernels take up to 524280 tokens (the
 * generic STQ1_0 kernel, for H or I not a multiple of 256, 65535).
 * ------------------------------------------------------------------------- */
MOE_MI355X_API moe_status moe_expert_ffn(const moe_dims* d, const moe_experts* routed,
                                         const moe_experts* shared, const uint16_t* x_bf16,
                                         const int32_t* sorted_pair,
                                         const int32_t* expert_offsets, float* y_pairs,
                                         float* y_shared, void* ws, size_t ws_bytes,
                                         void* stream);

/* ---------------------------------------------------------------------------
 * Combine: out[t] = y_shared[t] + sum_j topk_w[t][j] * y_pairs[pair_pos[t*k + j]]
 * (+ residual[t]), summed in that order in fp32; a slot with pair_pos -1 (not routed
 * by moe_permute) adds nothing.  The shared expert is always on
 * and ungated (the Flash-MoE package lists one shared expert per MoE block and no
 * gate for it).
 *   y_pairs [P][H]; topk_w [T][k]; pair_pos [P]; y_shared [T][H] or NULL;
 *   residual [T][H] or NULL (may equal out_f32); out_f32 [T][H] out;
 *   out_bf16 [T][H] out (round to nearest even) or NULL.
 * ------------------------------------------------------------------------- */
MOE_MI355X_API moe_status moe_combine(const moe_dims* d, const float* y_pairs,
                                      const float* topk_w, const int32_t* pair_pos,
                                      const float* y_shared, const float* residual,
                                      float* out_f32, uint16_t* out_bf16, void* stream);

/* ---------------------------------------------------------------------------
 * Fused decode layer: the same computation as moe_route + moe_permute + moe_expert_ffn
 * + moe_combine for STQ1_0 or MXFP4 (row-major or tiled) routed experts and an optional
 * bf16 shared expert, in three kernels (the fused top-8 MoE operator idea of "Hy4-preview
 * Flash-MoE STQ1_0", Important runtime choices: --slot8).  Every intermediate the four calls expose is
 * written to the same caller buffers (logits_out, topk_ids, topk_w, sorted_pair,
 * expert_offsets, pair_pos, y_pairs, y_shared), then out_f32 (and out_bf16 when
 * non-NULL) = combine (+ residual; residual may equal out_f32).  The router runs from
 * x (no logits_in).  Numerics: router logits are summed in a different order than
 * moe_route's, so they may differ from it in the last bits; everything else follows the
 * four-call definitions.
 * MXFP4 routed experts follow moe_expert_ffn's MXFP4 definition: x and h MX-quantised to
 * E4M3 (group 32 along H, resp. I) before their projections.
 * The shared expert must be bf16 (an MXFP8 one returns MOE_ERR_UNSUPPORTED: use the four
 * calls).
 * Limits: T <= 64, k <= 32, E <= 256, and (H, I) one of the compiled shapes (512, 256),
 * (1024, 512), (2048, 1024), (4096, 2048), (6144, 2048), (8192, 2048); MXFP4 routed
 * experts at T <= 4 also T k (I + I/32) <= 81920 (every pair's FP8 h fits the small-batch
 * down kernel's LDS; beyond 4 tokens h is staged per unit of <= 16 pairs).
 * Workspace: at least moe_layer_decode_workspace_size bytes.  It holds atomic ticket
 * counters (used beyond 4 tokens: one per 16-token tile and one for the permutation) that
 * MUST be zero before the first call on a given workspace (clear the buffer once after
 * allocating it); every call leaves them zero.  Calls sharing one workspace must
 * not overlap in time.  Returns MOE_ERR_UNSUPPORTED outside the limits.
 * ------------------------------------------------------------------------- */
MOE_MI355X_API moe_status moe_layer_decode_workspace_size(const moe_dims* d, int32_t has_shared,
                                                          size_t* bytes);
/* Byte offsets of the fused decode workspace regions, so tests can read intermediates
 * (host-only):
 *   offs[6] routed h: STQ1_0 bf16 hi [P][I] (lo half at offs[7]); MXFP4 E4M3 codes [P][I]
 *           then UE8M0 scales [P][I/32], in sorted-pair order
 *   offs[8] shared h, bf16 hi [T][I] then lo [T][I]
 *   offs[9] MXFP4: x as E4M3 codes [T][H] then UE8M0 scales [T][H/32]
 *   offs[10] total bytes (offs[0..5]: work lists, ticket counters, router partials) */
MOE_MI355X_API moe_status moe_layer_decode_workspace_offsets(const moe_dims* d, int32_t has_shared,
                                                             size_t* offs);
MOE_MI355X_API moe_status moe_layer_decode(
    const moe_dims* d, const moe_experts* routed, const moe_experts* shared,
    const uint16_t* x_bf16, const uint16_t* wr_bf16, const float* logit_bias, float* logits_out,
    int32_t* topk_ids, float* topk_w, int32_t* sorted_pair, int32_t* expert_offsets,
    int32_t* pair_pos, float* y_pairs, float* y_shared, const float* residual, float* out_f32,
    uint16_t* out_bf16, void* ws, size_t ws_bytes, void* stream);

/* The same fused decode layer with no workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): it calls no allocating routine and uses, as its workspace, a scratch array of
 * 8 MiB that the library holds on every device it runs on until the process ends.  Same
 * arguments, limits and results as moe_layer_decode (bit for bit), plus: the workspace
 * moe_layer_decode_workspace_size reports for these dims must fit 8 MiB (at hidden 6144,
 * intermediate 2048, top-8 every T <= 64 does), else MOE_ERR_UNSUPPORTED.  Each call first
 * enqueues a small kernel that zeroes the scratch's ticket counters.  All calls on one device
 * share its array: calls that overlap in time on one device (other streams, other host
 * threads) race and give wrong results; serialise them. */
MOE_MI355X_API moe_status moe_layer_decode_noalloc(
    const moe_dims* d, const moe_experts* routed, const moe_experts* shared,
    const uint16_t* x_bf16, const uint16_t* wr_bf16, const float* logit_bias, float* logits_out,
    int32_t* topk_ids, float* topk_w, int32_t* sorted_pair, int32_t* expert_offsets,
    int32_t* pair_pos, float* y_pairs, float* y_shared, const float* residual, float* out_f32,
    uint16_t* out_bf16, void* stream);

/* ---------------------------------------------------------------------------
 * Helpers (same conventions).
 * ------------------------------------------------------------------------- */

/* Pack STQ1_0: zpos [n_blocks*64] zero lanes (0..3), signs [n_blocks*64] sign fields
 * (0..7, bit i = i-th non-zero lane negative), d_f16 [n_blocks] binary16 bits ->
 * codes [n_blocks*40], scales [n_blocks].  Values outside those ranges are masked
 * to their low bits. */
MOE_MI355X_API moe_status moe_stq1_pack(const uint8_t* zpos, const uint8_t* signs,
                                        const uint16_t* d_f16, int64_t n_blocks,
                                        uint8_t* codes, uint16_t* scales, void* stream);

/* STQ1_0 encoders ("Hy4-preview-GGUF" (AngelSlim), section 3, Our encoder): a float
 * matrix (flattened row-major [N][K], n_weights % 256 == 0) -> STQ1_0 blocks of 256
 * consecutive weights.  Importance of a weight: imatrix[flat index mod K] (K > 0), or 1
 * when imatrix is NULL.
 *   MOE_STQ1_ENC_UPSTREAM: d = the block's largest magnitude; in each group of four the
 *     lane of smallest |x| is zeroed (first lane on ties).
 *   MOE_STQ1_ENC_WLS: from that zero placement, 3 rounds of (the weighted least-squares
 *     scale d = sum(w sel x) / sum(w sel^2), then in each group the zero at the lane of
 *     smallest incremental cost w (x^2 - (|x| - d)^2)), and a final least-squares fit of d
 *     (d = amax when the kept lanes carry no weight).
 * Kept lanes take the sign of x (0 counts as positive); d is rounded to fp16 once.
 * Sums run in fp32 in a fixed order, so a zero placement at a near-tie of two lanes'
 * costs may differ from an exact computation.
 *   x [n_weights] fp32 (16-byte aligned); imatrix [K] fp32 (entries >= 0) or NULL;
 *   codes [n_weights/256*40] out (8-byte aligned), scales [n_weights/256] fp16 out.
 * A one-time weight preparation, not a per-step call. */
enum { MOE_STQ1_ENC_UPSTREAM = 0, MOE_STQ1_ENC_WLS = 1 };
MOE_MI355X_API moe_status moe_stq1_encode(const float* x, const float* imatrix, int64_t n_weights,
                                          int32_t K, int32_t method, uint8_t* codes,
                                          uint16_t* scales, void* stream);

/* ---------------------------------------------------------------------------
 * Expert slot bank ("Hy4-preview Flash-MoE STQ1_0", slot-bank mode: routed experts kept
 * expert-major outside the dense model and streamed into a fixed set of slots as the router
 * asks for them; 8 slots is the minimum for top-8, more slots cache more experts, misses are
 * read in bounded chunks).  For models larger than HBM: S device slots hold routed experts,
 * filled from caller-owned (pinned) host memory.  A step:
 *   1. moe_slot_bank_plan (host only): the step's expert ids (host array, e.g. topk_ids
 *      copied back) -> slot_of[E] (slot of every resident expert, -1 otherwise).  Resident
 *      experts are hits; each miss takes an empty slot, else the least recently used slot
 *      that no expert of this step holds (lowest slot on ties).  n_copies: the step's misses.
 *      MOE_ERR_UNSUPPORTED when the step has more distinct experts than slots (state
 *      unchanged).
 *   2. moe_slot_bank_fetch: enqueue every planned copy not yet fetched (every non-empty family
 *      buffer of each missing expert, in io_split chunks) host -> device on `stream`.  Copies
 *      of a plan that was not followed by a fetch, or of a fetch that returned an error, stay
 *      pending until a fetch succeeds, unless a later plan gave their slot to another expert.
 *   3. moe_remap_ids: topk_ids -> slot ids on the device (slot_of uploaded by the caller), then
 *      moe_permute / moe_expert_ffn with E = S on the slot arrays, and moe_combine as usual.
 * bytes[6]: per-expert bytes of gate codes, gate scales, up codes, up scales, down codes,
 * down scales (0 for a family buffer that does not exist).  host_src: all E experts
 * (expert-major, pinned host memory); dev_slots: S experts' worth of device memory in the
 * same layout.  The bank object is host state; it is not thread-safe. */
typedef struct moe_slot_bank moe_slot_bank;
MOE_MI355X_API moe_status moe_slot_bank_create(int32_t E, int32_t S, const uint64_t* bytes,
                                               int32_t io_split, moe_slot_bank** out);
MOE_MI355X_API moe_status moe_slot_bank_destroy(moe_slot_bank* bank);
MOE_MI355X_API moe_status moe_slot_bank_plan(moe_slot_bank* bank, const int32_t* ids_host,
                                             int64_t n, int32_t* slot_of_host, int32_t* n_copies);
MOE_MI355X_API moe_status moe_slot_bank_fetch(moe_slot_bank* bank, const moe_experts* host_src,
                                              const moe_experts* dev_slots, void* stream);
MOE_MI355X_API moe_status moe_slot_bank_stats(const moe_slot_bank* bank, uint64_t* hits,
                                              uint64_t* misses);
/* ids [n] -> out [n] = slot_of[ids] (device arrays; ids must be resident in slot_of). */
MOE_MI355X_API moe_status moe_remap_ids(const int32_t* ids, int64_t n, const int32_t* slot_of,
                                        int32_t* out, void* stream);

/* Decode STQ1_0 blocks to fp32 weights out [n_blocks*256] (exact). */
MOE_MI355X_API moe_status moe_stq1_dequant(const uint8_t* codes, const uint16_t* scales,
                                           int64_t n_blocks, float* out, void* stream);

/* Decode MXFP4 rows: codes [rows][K/2], scales [rows][K/32] -> out [rows][K] fp32 (exact). */
MOE_MI355X_API moe_status moe_mxfp4_dequant(const uint8_t* codes, const uint8_t* scales,
                                            int64_t rows, int32_t K, float* out, void* stream);

/* Reorder MXFP4 rows (codes [rows][K/2], scales [rows][K/32], rows % 16 == 0,
 * K % 128 == 0) into the MXFP4_TILED layout: tcodes [rows*K/2], tscales [rows*K/32].
 * A stack of matrices (E experts of `out` rows each) is one call with rows = E*out,
 * since tiles never straddle a matrix when out % 16 == 0.  codes and tcodes must be
 * 16-byte aligned, scales and tscales 4-byte aligned; outputs must not overlap the
 * inputs.  A one-time weight preparation for MOE_W_MXFP4_TILED, not a per-step call. */
MOE_MI355X_API moe_status moe_mxfp4_pack_tiles(const uint8_t* codes, const uint8_t* scales,
                                               int64_t rows, int32_t K, uint8_t* tcodes,
                                               uint8_t* tscales, void* stream);

/* MX-quantise rows of K (K % 32 == 0) into E4M3 codes q [rows][K] and UE8M0 scales
 * s [rows][K/32].  Input is either bf16 (x_bf16) or fp32 (x_f32); exactly one must be
 * non-NULL.  Rule (OCP MX v1.0 reading): X = floor(log2(amax)) - 8 clamped to
 * [-127, 127], scale byte X + 127; elements round to nearest even of v / 2^X,
 * saturated to +-448; the sign bit follows the input (a negative value that rounds
 * to zero gives 0x80); a group with amax == 0 stores scale 0 and zero codes. */
MOE_MI355X_API moe_status moe_mx_quant_act(int64_t rows, int32_t K, const uint16_t* x_bf16,
                                           const float* x_f32, uint8_t* q, uint8_t* s,
                                           void* stream);

/* The same MX quantisation of fp32 rows as moe_mx_quant_act (same rule, same outputs), with
 * every E4M3 code produced by the gfx950 scaled hardware conversion that the MXFP4 gate/up
 * epilogue uses for h, instead of the integer-rule encoder.  A check point for that
 * epilogue's encoder on chosen values (rounding ties, the saturating band, zeros, every group
 * exponent); not a per-step call.  x_f32 [rows][K] (16-byte aligned), q [rows][K] and
 * s [rows][K/32] out. */
MOE_MI355X_API moe_status moe_mx_quant_f32_hwcvt(int64_t rows, int32_t K, const float* x_f32,
                                                 uint8_t* q, uint8_t* s, void* stream);

/* Pre-norm for a residual stack of MoE layers: a[t] = bf16(r[t] / sqrt(mean(r[t]^2) + eps))
 * (norm weight 1), r [T][H] fp32, a [T][H] bf16 out. */
MOE_MI355X_API moe_status moe_rmsnorm_bf16(int32_t T, int32_t H, float eps, const float* r,
                                           uint16_t* a, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
