/*
 * moe_nvfp4.h -- C ABI of the NVFP4 routed-expert (mixture-of-experts) layer
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  The routed-expert layer of a Qwen-style MoE decoder whose
 * experts are NVFP4: E2M1 4-bit codes, one E4M3 scale per 16 consecutive
 * weights along the reduction dimension, one fp32 multiplier per matrix and,
 * for 4-bit activations, one fp32 activation input scale per matrix (page
 * "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)", section "What
 * is bit-exact and what is quantized").  512 routed experts with the top 10
 * chosen per token (same page, opening description).  The expert activations
 * run at 16, 8 or 4 bits (page "Infernix", section "Activation precision").
 *
 * Conventions shared by every entry point:
 *  - Pointers are DEVICE pointers unless marked [host].  The caller owns every
 *    buffer and keeps it alive until the work enqueued on the stream is done;
 *    the library keeps no pointer after a call returns.  It allocates nothing.
 *  - Calls validate their arguments on the host, enqueue kernels on stream
 *    `s` and return without synchronising.  A device fault surfaces at the
 *    caller's next synchronisation.
 *  - On error nothing is enqueued (except MOE_E_HIP, reported after a launch
 *    failed) and moe_last_error() describes it.  No C++ exception crosses
 *    this boundary.
 *  - bf16 tensors are passed as uint16_t bit patterns.  Matrices are row-major.
 *  - Packed NVFP4 rows hold element 2i in the low nibble of byte i.
 *  - Identical inputs give bitwise-identical outputs (no floating-point
 *    atomics).  Calls are re-entrant; calls on different streams may overlap.
 *  - Shapes: H and I are multiples of 32 and at most 4096; 1 <= k <= E <= 1024
 *    and k <= 64 (routing and the whole layer).
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_E_ARG = -1,          /* null pointer where one is required, bad enum */
  MOE_E_ALIGN = -2,        /* pointer not aligned as documented */
  MOE_E_SHAPE = -3,        /* size out of the documented range */
  MOE_E_UNSUPPORTED = -4,  /* valid but not implemented combination */
  MOE_E_WORKSPACE = -5,    /* workspace smaller than the *_workspace_bytes() figure */
  MOE_E_HIP = -6,          /* a HIP call or kernel launch failed */
  MOE_E_STALLED = -7       /* moe_layer_status: a wait inside a fused decode call gave up */
} moe_status;

/* Expert activation precision (page "Infernix", section "Activation precision"). */
typedef enum {
  MOE_A16 = 0, /* bf16 activations on the 4-bit weights (W4A16) */
  MOE_A8 = 1,  /* E4M3 activations, one fp32 scale per 16 (W4A8) */
  MOE_A4 = 2,  /* NVFP4 activations under the matrix's fp32 input scale (W4A4) */
  /* range markers, not modes: with them every int32 is a value of the type in
   * C and C++, so an out-of-range argument reaches the validation (MOE_E_ARG)
   * as the caller passed it */
  MOE_ACT_MODE_RANGE_MIN_ = -2147483647 - 1,
  MOE_ACT_MODE_RANGE_MAX_ = 2147483647
} moe_act_mode;

typedef enum {
  MOE_DT_BF16 = 0,
  MOE_DT_F32 = 1,
  MOE_DTYPE_RANGE_MIN_ = -2147483647 - 1, /* range markers, as for moe_act_mode */
  MOE_DTYPE_RANGE_MAX_ = 2147483647
} moe_dtype;

/* Encoding of the expert weights. */
typedef enum {
  /* NVFP4 (the routed experts of page "Qwen3.8-Flash-Next NVIDIA NVFP4 for
   * Infernix (bit-exact)", section "What is bit-exact and what is quantized") */
  MOE_FMT_NVFP4 = 0,
  /* q4_g64_fp16 (same page, section "Drafting only": the drafter's routed
   * experts): 4-bit two's complement codes (element 2i in the low nibble of byte
   * i), one fp16 scale per 64 consecutive values along the reduction dimension,
   * no per-matrix multiplier.  These experts compute in fp16: they take the
   * 16-bit mode (MOE_A16) only, with x rounded to fp16 (nearest even) at the
   * expert input and the intermediate held as fp16. */
  MOE_FMT_Q4G64 = 2
} moe_weight_format;

/* Arrangement of the NVFP4 block scales in memory (the codes are the same in
 * both).  The pages' checkpoint is repacked into the engine's own expert
 * layout without changing a bit (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for
 * Infernix (bit-exact)", section "What is bit-exact and what is quantized");
 * this library's own bit-preserving layout is MOE_LAYOUT_TILED.
 *   MOE_LAYOUT_CANONICAL: scale row [K/16] in K order: the two E4M3 scales of
 *     chunk c (values 32c .. 32c+31) at bytes 2c, 2c+1.
 *   MOE_LAYOUT_TILED: a scale row is cut into windows of 32 chunks (1024
 *     values, 64 bytes).  In a full window, chunk 4i + g (step i of 128
 *     values, piece g of 32) has its scale pair at pair position 8g + i of the
 *     window: piece g of all 8 steps is one contiguous 16-byte word, which one
 *     lane of the prefill matrix-core path loads for 8 steps at once.  A
 *     trailing window of fewer than 32 chunks keeps the canonical order.
 *     NVFP4 only, with H and I multiples of 128.  Produced by moe_nvfp4_repack;
 *     every entry point that takes moe_nvfp4_experts accepts either layout and
 *     gives bit-identical results. */
typedef enum { MOE_LAYOUT_CANONICAL = 0, MOE_LAYOUT_TILED = 1 } moe_layout;

/* One layer's experts, stacked over E.  The struct itself
 * lives in host memory; its pointers are device pointers.  16-byte alignment
 * is required for the code and scale arrays, 4-byte for the fp32 arrays.
 *   gu_codes   [E][2I][H/2]  gate rows 0..I-1, then up rows I..2I-1
 *   gu_scales  [E][2I][H/16] E4M3 block scales   (MOE_FMT_Q4G64: fp16 [E][2I][H/64])
 *   dn_codes   [E][H][I/2]
 *   dn_scales  [E][H][I/16]                      (MOE_FMT_Q4G64: fp16 [E][H][I/64])
 *   gu_wscale  [E][2]        fp32 multiplier of the gate and the up matrix (NVFP4 only)
 *   dn_wscale  [E]           fp32 multiplier of the down matrix (NVFP4 only)
 *   gu_inscale [E][2]        fp32 activation input scales (MOE_A4 only, else may be NULL)
 *   dn_inscale [E]           fp32 activation input scale of down (MOE_A4 only)
 *   fmt                      the encoding (a zero-filled struct is NVFP4); MOE_FMT_Q4G64
 *                            needs H and I multiples of 64
 *   layout                   the scale arrangement (moe_layout; zero: canonical)
 */
typedef struct {
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint8_t* dn_codes;
  const uint8_t* dn_scales;
  const float* gu_wscale;
  const float* dn_wscale;
  const float* gu_inscale;
  const float* dn_inscale;
  int32_t E, H, I;
  int32_t fmt;    /* moe_weight_format */
  int32_t layout; /* moe_layout */
} moe_nvfp4_experts;

/* The shared expert of a layer and its gate, BF16 (page "Qwen3.8-Flash-Next
 * NVIDIA NVFP4 for Infernix (bit-exact)", section "What is bit-exact and what
 * is quantized": the shared experts and the gates are BF16 dense
 * projections).  Read as a Qwen-style MoE block: one SwiGLU expert that every
 * token runs, whose output is scaled by sigmoid(x . gate) and added to the
 * routed experts' weighted sum.  Host struct of device pointers (16-byte
 * aligned); Is a multiple of 32 up to 1024, H the layer's.
 *   gu   [2Is][H] bf16  gate rows 0..Is-1, then up rows Is..2Is-1
 *   dn   [H][Is]  bf16
 *   gate [H]      bf16  the gate vector (one output) */
typedef struct {
  const uint16_t* gu;
  const uint16_t* dn;
  const uint16_t* gate;
  int32_t H, Is;
} moe_shared_expert;

/* Text of the last error on the calling thread; valid until the next call on it. */
const char* moe_last_error(void);

/* ------------------------------------------------------------------ router
 * moe_route_topk: router logits, softmax, top-k, renormalise.
 *   logits[t][e] = sum_h x[t][h] * w_router[e][h] (+ bias[e]), fp32 accumulate;
 *   the k largest logits per token in descending order (equal logits: lower
 *   expert first); topk_w[t][j] = p_j / sum of the chosen p with p the
 *   softmax over all E (equal to a softmax over the chosen logits).
 * The pages store the router in BF16 (page "Qwen3.8-Flash-Next NVIDIA NVFP4
 * for Infernix (bit-exact)", section "What is bit-exact and what is
 * quantized") and print no router formula; this is the Qwen-style reading.
 *   x        [T][H] bf16          w_router [E][H] bf16     bias [E] fp32 or NULL
 *   topk_ids [T][k] int32 (out)   topk_w   [T][k] fp32 (out)
 *   ws: moe_route_workspace_bytes(T, E) bytes (fp32 logits), 16-byte aligned.
 * NaN logits give unspecified ids.  T >= 1. */
size_t moe_route_workspace_bytes(int T, int E);
moe_status moe_route_topk(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                          int H, int E, int k, int32_t* topk_ids, float* topk_w, void* ws,
                          size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------------ permute
 * moe_permute: stable counting sort of the T*k (token, slot) pairs by expert.
 * Pair p = t*k + j.  expert_offsets [E+1] is the exclusive scan of the expert
 * histogram; sorted_pairs[expert_offsets[e] + r] is the r-th pair of expert e
 * in ascending p; pair_row[p] is the inverse (row of pair p in sorted order).
 * Ids outside [0, E) are dropped: not counted, pair_row[p] = -1, and
 * expert_offsets[E] counts the valid pairs only.  Bit-exact and deterministic.
 *   ws: moe_permute_workspace_bytes(T, k, E) bytes, 4-byte aligned (0 bytes, ws
 *   may be NULL, up to 2048 pairs; more pairs run on several workgroups and
 *   keep per-block expert counts there).  MOE_E_WORKSPACE if smaller. */
size_t moe_permute_workspace_bytes(int T, int k, int E);
moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E, int32_t* expert_offsets,
                       int32_t* sorted_pairs, int32_t* pair_row, void* ws, size_t ws_bytes,
                       hipStream_t s);

/* ------------------------------------------------------------------ quantizers
 * act_quant_nvfp4: NVFP4 per 16 along a row (the weight format of the page
 * "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)", section "What
 * is bit-exact and what is quantized", also used for 4-bit activations):
 *   t = f32(f32(bamax / 6) / g);  s = E4M3(t);  d = f32(dec(s) * g);
 *   code = E2M1(f32(v / d))   -- each op a correctly rounded fp32 op; E4M3 and
 *   E2M1 round to nearest with ties to the even code, saturate (448 / 6) and
 *   keep the sign; a block whose d is not positive gets all-zero codes.
 * g = global[row_group ? row_group[r] : 0].
 *   x [rows][cols] bf16 or fp32; codes [rows][cols/2]; scales [rows][cols/16].
 * cols % 32 == 0. */
moe_status act_quant_nvfp4(const void* x, moe_dtype xdt, int rows, int cols, const float* global,
                           const int32_t* row_group, uint8_t* codes, uint8_t* scales,
                           hipStream_t s);

/* act_quant_fp8: the 8-bit activation mode (page "Infernix", section
 * "Activation precision", --a8-activations), read as E4M3 codes with one fp32
 * scale per 16: s = f32(bamax / 448); code = E4M3(f32(v / s)); s == 0 gives
 * all-zero codes.  codes [rows][cols]; scales [rows][cols/16] fp32. */
moe_status act_quant_fp8(const void* x, moe_dtype xdt, int rows, int cols, uint8_t* codes,
                         float* scales, hipStream_t s);

/* q4g64_quantize: q4_g64_fp16 packing of fp32 rows (page "Qwen3.8-Flash-Next
 * NVIDIA NVFP4 for Infernix (bit-exact)", section "Drafting only": 4-bit, one
 * FP16 scale per 64, scales chosen by mean squared error from the exact
 * values).  Per group of 64 values with amax = max |v|: the candidates
 * d_j = fp16(f32(amax / m_j)), m_j = 7 + j/8 for j = 0..8; codes
 * q = clamp(RNE(f32(v / d_j)), -8, 7); the first candidate with the least
 * sum of (v - d_j q)^2 (double, in index order, each op rounded once) is kept;
 * candidates whose d is 0 or infinite are skipped; a group with none stores
 * d = 0 and q = 0.  x [rows][cols] fp32 (cols % 64 == 0); codes [rows][cols/2];
 * scales [rows][cols/64] fp16 bit patterns. */
moe_status q4g64_quantize(const float* x, int rows, int cols, uint8_t* codes, uint16_t* scales, hipStream_t s);

/* nvfp4_global_scale: per-matrix fp32 multiplier of NVFP4 packing,
 * global[m] = f32(amax(|x_m|) / 2688) (2688 = 6 * 448) for the n_mat
 * contiguous fp32 matrices of mat_elems elements each.  Deterministic. */
moe_status nvfp4_global_scale(const float* x, int n_mat, int64_t mat_elems, float* global,
                              hipStream_t s);

/* ------------------------------------------------------------------ experts
 * nvfp4_expert_ffn: every (token, expert) pair's SwiGLU expert in sorted order.
 * For sorted row r of expert e (token t = sorted_pairs[r] / k):
 *   g = x_t . Wgate_e,  u = x_t . Wup_e   (fp32 accumulate; x_t in the mode's
 *   precision: bf16 for A16, E4M3 per 16 for A8, NVFP4 per 16 under the
 *   matrix's input scale for A4);  h = silu(g) * u  (silu(z) = z / (1 + e^-z));
 *   h is held at the mode's precision (bf16 / E4M3 per 16 / NVFP4 per 16 under
 *   dn_inscale[e]);  y_pairs[r] = h . Wdown_e (fp32).
 * The page "Infernix releases" (release 2026.10.11, "Highlights") describes
 * the same stages on its GPU: narrow calls on one-column kernels with exact
 * FP4 products, the down pass chained on gate/up.
 *   w        [host] expert set          x [T][H] bf16
 *   expert_offsets [E+1], sorted_pairs [T*k] from moe_permute
 *   y_pairs  [T*k][H] fp32 (out; rows >= expert_offsets[E] are not written)
 *   ws: nvfp4_expert_ffn_workspace_bytes(mode, T, k, H, I) bytes, 16-byte aligned.
 * Workspace layout (P = T*k rows, byte offsets rounded up to 256):
 *   A16: h bf16 [P][I]
 *   A8 : x codes [T][H], x scales fp32 [T][H/16], h codes [P][I], h scales fp32 [P][I/16]
 *   A4 : x codes [P][2][H/2], x scales [P][2][H/16] (gate, up), h codes [P][I/2],
 *        h scales [P][I/16], work plan int32 [min(P, 1024) + P/32][4] (used
 *        when T > 8: chunks of at most 32 rows of one expert, each as expert,
 *        first sorted row, rows; unused entries have expert -1)  */
size_t nvfp4_expert_ffn_workspace_bytes(moe_act_mode mode, int T, int k, int H, int I);
moe_status nvfp4_expert_ffn(const moe_nvfp4_experts* w, moe_act_mode mode, const uint16_t* x,
                            int T, int k, const int32_t* expert_offsets,
                            const int32_t* sorted_pairs, float* y_pairs, void* ws,
                            size_t ws_bytes, hipStream_t s);

/* nvfp4_expert_ffn_stage: one stage of nvfp4_expert_ffn, same arguments and
 * workspace: stage 0 quantizes the activations (8/4-bit modes; a no-op for
 * A16), stage 1 runs gate/up + SwiGLU (writes the intermediate into ws),
 * stage 2 runs down (writes y_pairs).  Running 0, 1, 2 in order on one stream
 * equals nvfp4_expert_ffn; it lets a caller time or overlap the stages. */
moe_status nvfp4_expert_ffn_stage(const moe_nvfp4_experts* w, moe_act_mode mode, int stage,
                                  const uint16_t* x, int T, int k, const int32_t* expert_offsets,
                                  const int32_t* sorted_pairs, float* y_pairs, void* ws,
                                  size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------------ combine
 * moe_combine: out[t] = bf16( sum_j topk_w[t][j] * y_pairs[pair_row[t*k + j]] ),
 * j ascending, fp32 sum, one round-to-nearest-even to bf16.  Pairs with
 * pair_row < 0 contribute nothing.  With a residual x (bf16 [T][H], not NULL)
 * the result is the next layer's input bf16(x + bf16(sum)). */
moe_status moe_combine(const float* y_pairs, const int32_t* pair_row, const float* topk_w, int T,
                       int k, int H, const uint16_t* residual, uint16_t* out, hipStream_t s);

/* ------------------------------------------------------------------ shared expert
 * moe_shared_expert_forward: y[t] = sigmoid(x_t . gate) * (h_t . Wd^T) with
 * h_t = bf16(silu(x_t . Wg^T) * (x_t . Wu^T)), fp32 sums of bf16 products, the
 * intermediate rounded once to bf16 (the dense projections' activation
 * precision).  x [T][H] bf16; y [T][H] fp32 (out);
 * ws: moe_shared_expert_workspace_bytes(T, Is) bytes (the intermediate), 16-byte aligned.
 * moe_combine_shared: moe_combine with the shared expert's y (fp32 [T][H], not
 * NULL) added after the routed sum and before the rounding:
 *   out[t] = bf16( sum_j topk_w[t][j] * y_pairs[pair_row[t*k + j]] + shared_y[t] ). */
size_t moe_shared_expert_workspace_bytes(int T, int Is);
moe_status moe_shared_expert_forward(const moe_shared_expert* sw, const uint16_t* x, int T, float* y, void* ws,
                                     size_t ws_bytes, hipStream_t s);
moe_status moe_combine_shared(const float* y_pairs, const int32_t* pair_row, const float* topk_w, int T, int k,
                              int H, const float* shared_y, const uint16_t* residual, uint16_t* out,
                              hipStream_t s);

/* ------------------------------------------------------------------ whole layer
 * moe_layer_forward: route -> permute -> experts -> combine on one stream.
 *   out [T][H] bf16 = the layer output, or bf16(residual + output) when
 *   residual is not NULL (residual may equal x; out must not alias x).
 *   ws: moe_layer_workspace_bytes(mode, T, k, E, H, I) bytes, 256-byte aligned,
 *   zero-filled before its first use: up to 8 tokens the layer runs fused (one
 *   launch for 16- and 8-bit activations and up to 64 pairs, else the routing
 *   in one launch and the experts with the combine in another) and keeps
 *   inter-workgroup state in the workspace: counters, which every call leaves at
 *   zero, and words stamped with a per-call number, which need no reset.
 *   Calls sharing a workspace must not overlap.
 *   moe_layer_workspace_layout fills offsets[7] (bytes into ws) of topk_ids
 *   [T][k] int32, topk_w [T][k] fp32, expert_offsets [E+1] int32, sorted_pairs
 *   [T*k] int32, pair_row [T*k] int32, y_pairs [T*k][H] fp32, and the expert
 *   workspace (the nvfp4_expert_ffn layout above), so a caller can read them.
 * Returns MOE_E_SHAPE from the layout call for sizes out of range. */
moe_status moe_layer_workspace_layout(moe_act_mode mode, int T, int k, int E, int H, int I,
                                      size_t offsets[7]);
/* Byte offset in a layer workspace of a uint32 that counts waits of the fused
 * decode path which gave up (a stalled producer); it stays 0 in correct
 * operation.  Workgroups of one fused launch wait for each other; the waits are
 * bounded (about 0.7 s each) and the first to give up makes every other wait of
 * the launch give up at once, so a stalled launch still ends.  Its combine then
 * writes bf16 NaN for the outputs whose inputs it gave up on.  A non-zero count
 * makes every later fused call on the workspace give up at once (NaN outputs)
 * until the caller zero-fills the workspace again. */
size_t moe_layer_wait_timeouts_offset(void);

/* moe_layer_status: MOE_OK when no wait of a fused decode call on this layer
 * workspace has given up since it was zero-filled, else MOE_E_STALLED (the
 * outputs of those calls are unreliable).  It reads 4 bytes of ws after the
 * work already enqueued on s, and therefore SYNCHRONISES stream s: a health
 * check, not for a hot loop. */
moe_status moe_layer_status(const void* ws, hipStream_t s);

/* 1 when moe_layer_forward runs the fused decode path for these sizes (up
 * to 8 tokens, H/32 in 33..128, I/32 in 5..32), else 0 (per-stage kernels). */
int moe_layer_is_fused(int T, int H, int I);

/* Kernel launches of one moe_layer_forward call: 1 for the single-launch
 * decode layer (fused sizes, MOE_A16 or MOE_A8 with NVFP4 experts, T*k <= 64;
 * MOE_A8 quantizes x in the gate/up tiles), 2 for the fused two-kernel path
 * (routing, experts + combine; MOE_A8 quantizes x in the routing kernel,
 * MOE_A4 in the expert kernel's gate/up tiles; q4_g64_fp16 experts take this
 * path), 0 when the per-stage kernels run.  Under stream capture the single-launch layer is one graph node
 * too: it then takes its call number from the workspace and advances it itself
 * (a number baked into the launch would repeat on every replay). */
int moe_layer_launches(moe_act_mode mode, int T, int k, int H, int I);

/* Kernel launches of one moe_block_forward call with a shared expert of
 * intermediate width Is: 1 where the single-launch decode layer also runs the
 * shared expert (its conditions with MOE_A16, and Is a multiple of 32 up to 512: the shared
 * expert's weights then stream while the tokens are routed), else the shared
 * expert's two kernels plus moe_layer_launches (0 for the per-stage path). */
int moe_block_launches(moe_act_mode mode, int T, int k, int H, int I, int Is);
size_t moe_layer_workspace_bytes(moe_act_mode mode, int T, int k, int E, int H, int I);
moe_status moe_layer_forward(const moe_nvfp4_experts* w, moe_act_mode mode, const uint16_t* x,
                             const uint16_t* w_router, const float* router_bias, int T, int k,
                             const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes,
                             hipStream_t s);

/* moe_layer_forward_stage: one half of moe_layer_forward, same arguments and
 * workspace: stage 0 routes (router logits, top-k, permutation, and the
 * activation quantization of the 8/4-bit modes), stage 1 runs the experts and
 * the combine.  Stage 0 then stage 1 on one stream equals moe_layer_forward;
 * stage 1 needs the stage 0 of the same call before it.  It lets a caller time
 * the two halves (the fused decode path runs one kernel per half). */
moe_status moe_layer_forward_stage(const moe_nvfp4_experts* w, moe_act_mode mode, int stage,
                                   const uint16_t* x, const uint16_t* w_router,
                                   const float* router_bias, int T, int k,
                                   const uint16_t* residual, uint16_t* out, void* ws,
                                   size_t ws_bytes, hipStream_t s);

/* ------------------------------------------------------------------ no allocation
 * moe_layer_forward_noalloc: moe_layer_forward for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same layer, the same kernels and
 * results, bit for bit, but the workspace is a device array inside the
 * library (MOE_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on a GPU
 * until the process ends) instead of a caller's buffer.  The caller still
 * passes the inputs and the output.  The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).
 *  - Calls whose moe_layer_workspace_bytes exceeds MOE_NOALLOC_SCRATCH_BYTES
 *    return MOE_E_WORKSPACE (16 MiB holds, for example, every call of up to 64
 *    tokens at E = 512, k = 10, H = 3072, I = 512).
 *  - Every call on one GPU shares that GPU's array, which keeps the last call's
 *    contents: calls that overlap on one GPU (on different streams or threads)
 *    race and must not be made.
 *  - The array is zero-filled (a fill kernel on stream s) at the first call on
 *    each GPU, and again when reset is non-zero.  A fused decode call whose
 *    waits gave up (see moe_layer_wait_timeouts_offset) leaves bf16 NaN in out
 *    and makes every later call on the GPU give up too until a call with
 *    reset != 0.
 *  - Arguments and errors as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
moe_status moe_layer_forward_noalloc(const moe_nvfp4_experts* w, moe_act_mode mode, const uint16_t* x,
                                     const uint16_t* w_router, const float* router_bias, int T, int k,
                                     const uint16_t* residual, uint16_t* out, int reset, hipStream_t s);

/* ------------------------------------------------------------------ repack
 * moe_nvfp4_repack: the experts of src (canonical) into the tiled layout of dst
 * (see moe_layout), without changing a bit: every code byte is copied as is
 * and every scale byte moved to its tiled position (page "Qwen3.8-Flash-Next
 * NVIDIA NVFP4 for Infernix (bit-exact)", section "What is bit-exact and what
 * is quantized": the checkpoint is repacked into the engine's layout bit for
 * bit).  src and dst are host structs of device pointers; dst's code and scale
 * arrays are caller-allocated, of the same sizes as src's, and written here;
 * its fp32 arrays are not touched (they may be src's own).  dst's code arrays
 * may be src's (then they are not copied); its scale arrays must not overlap
 * src's.  Requirements: src->layout MOE_LAYOUT_CANONICAL, dst->layout
 * MOE_LAYOUT_TILED, both MOE_FMT_NVFP4 with equal E, H, I; H and I multiples
 * of 128 (else MOE_E_SHAPE); 16-byte aligned arrays (else MOE_E_ALIGN).
 * Enqueued on s; nothing is allocated. */
moe_status moe_nvfp4_repack(const moe_nvfp4_experts* src, const moe_nvfp4_experts* dst, hipStream_t s);

/* ------------------------------------------------------------------ test only
 * moe_debug_nvfp4_matmul: the expert kernels' product core without the
 * routing, the SwiGLU or the intermediate's rounding, for pinning it.  For one
 * NVFP4 matrix W (codes [N][K/2], E4M3 scales [N][K/16], fp32 multiplier
 * *wscale) and cols activation columns x:
 *   out[c][n] = wscale (* inscale, MOE_A4) * sum_k dec(W[n][k]) * x[c][k]
 * in fp32 accumulation, with x in the mode's stored form:
 *   MOE_A16  x bf16 [cols][K], x_scales NULL;
 *   MOE_A8   x E4M3 codes [cols][K], x_scales fp32 [cols][K/16];
 *   MOE_A4   x E2M1 codes [cols][K/2], x_scales E4M3 [cols][K/16], *inscale
 *            the fp32 input scale (a device pointer, as wscale).
 * core 0 runs the narrow path's tile (the one the down projection of calls of
 * up to 8 tokens uses; any K % 32 == 0 up to 4096, any N); core 1 the wide
 * path's matrix-core loop (MOE_A4; N % 16 == 0, K % 128 == 0) and needs
 * moe_debug_nvfp4_matmul_workspace_bytes(1, cols) bytes of ws (16-byte
 * aligned) for its chunk list; core 0 needs none (ws may be NULL).
 * Products of E2M1 weights with E2M1 (or small-integer) activations are exact,
 * so with unit scales the result is the exact integer row sum, bit for bit,
 * in any summation order (page "Infernix releases", release 2026.10.11,
 * "Highlights": FP4 products and their row sums stay exact). */
size_t moe_debug_nvfp4_matmul_workspace_bytes(int core, int cols);
/* moe_debug_q4g64_matmul: the same for q4_g64_fp16 weights (codes [N][K/2],
 * fp16 scales [N][K/64]) on the narrow tile, x bf16 [cols][K] rounded to fp16
 * as the experts take it: out[c][n] = sum_k dec(W[n][k]) * fp16(x[c][k]).
 * K % 64 == 0, K <= 4096. */
moe_status moe_debug_q4g64_matmul(const uint8_t* codes, const uint16_t* scales, int N, int K, const uint16_t* x,
                                  int cols, float* out, hipStream_t s);
moe_status moe_debug_nvfp4_matmul(int core, moe_act_mode mode, const uint8_t* codes, const uint8_t* scales,
                                  const float* wscale, int N, int K, const void* x, const void* x_scales,
                                  const float* inscale, int cols, float* out, void* ws, size_t ws_bytes,
                                  hipStream_t s);

/* moe_block_forward: moe_layer_forward plus the shared expert (sw, not NULL):
 *   out = bf16( routed weighted sum + sigmoid(x . gate) * shared expert(x) ),
 * or with a residual bf16(residual + out), on one stream (the shared expert's
 * two kernels first, then the layer's).  ws: moe_block_workspace_bytes(mode,
 * T, k, E, H, I, Is) bytes, 256-byte aligned, zero-filled before its first use
 * as for moe_layer_forward; moe_block_workspace_layout fills offsets[9]: the
 * seven of moe_layer_workspace_layout, then the shared expert's intermediate
 * (bf16 [T][Is]) and its gated output (fp32 [T][H]). */
size_t moe_block_workspace_bytes(moe_act_mode mode, int T, int k, int E, int H, int I, int Is);
moe_status moe_block_workspace_layout(moe_act_mode mode, int T, int k, int E, int H, int I, int Is,
                                      size_t offsets[9]);
moe_status moe_block_forward(const moe_nvfp4_experts* w, const moe_shared_expert* sw, moe_act_mode mode,
                             const uint16_t* x, const uint16_t* w_router, const float* router_bias, int T, int k,
                             const uint16_t* residual, uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s);

#ifdef __cplusplus
}
#endif
#endif
