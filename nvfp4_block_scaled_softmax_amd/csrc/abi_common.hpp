// Host-side helpers of the C ABI: the thread-local error text, argument
// checks and launch checks.  Every entry point validates before enqueuing.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdarg.h>
#include <string>

#include "../../include/moe_nvfp4.h"

namespace moe {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Checks after launches: any launch failure becomes MOE_E_HIP with HIP's text.
inline moe_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    set_error("%s: kernel launch failed: %s", what, hipGetErrorString(e));
    return MOE_E_HIP;
  }
  return MOE_OK;
}

#define MOE_REQUIRE(cond, code, ...) \
  do {                               \
    if (!(cond)) {                   \
      ::moe::set_error(__VA_ARGS__); \
      return code;                   \
    }                                \
  } while (0)

// The kernels' internal mode for q4_g64_fp16 experts (fp16 activations); the
// public modes are MOE_A16 / MOE_A8 / MOE_A4 = 0 / 1 / 2.
constexpr int kModeQ4 = 3;

// The mode the kernels run: the public activation mode, or kModeQ4 for
// q4_g64_fp16 experts (validated to come with MOE_A16).
inline moe_act_mode kernel_mode(const moe_nvfp4_experts& w, moe_act_mode mode) {
  return w.fmt == MOE_FMT_Q4G64 ? (moe_act_mode)kModeQ4 : mode;
}

constexpr int kMaxExperts = 1024;
constexpr int kMaxTopK = 64;   // experts per token: one wave lane each in the top-k
constexpr int kMaxDim = 4096;

inline bool dim_ok(int d) { return d >= 32 && d <= kMaxDim && d % 32 == 0; }

// Launchers implemented in the .hip files (no validation: callers validated).
moe_status launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                        int H, int E, int k, int32_t* ids, float* w, float* logits, hipStream_t s);
moe_status launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_row, void* ws, hipStream_t s);
size_t permute_workspace(int P, int E);
// stage_mask: bit 0 activation quantization, bit 1 gate/up + SwiGLU, bit 2 down.
// pair_row and ids (the permutation's inverse and the top-k ids, both [T*k];
// nullable together) let the 4-bit x quantization work per token.
moe_status launch_expert_ffn(const moe_nvfp4_experts& w, moe_act_mode mode, const uint16_t* x,
                             int T, int k, const int32_t* offsets, const int32_t* sorted_pairs,
                             float* y_pairs, void* ws, int stage_mask, hipStream_t s,
                             const int32_t* pair_row = nullptr, const int32_t* ids = nullptr);
moe_status launch_combine(const float* y_pairs, const int32_t* pair_row, const float* topk_w,
                          int T, int k, int H, const float* shared_y, const uint16_t* residual,
                          uint16_t* out, hipStream_t s);
// The shared expert (shared.hip): validation, workspace (its bf16 intermediate
// [T][Is]) and the two kernels writing the gated output y [T][H] fp32.
moe_status check_shared(const char* name, const moe_shared_expert* sw, int H);
size_t shared_workspace(int T, int Is);
moe_status launch_shared_expert(const moe_shared_expert& sw, const uint16_t* x, int T, void* h_ws, float* y,
                                hipStream_t s);
size_t expert_ffn_workspace(moe_act_mode mode, int T, int k, int H, int I);
// The fused decode layer (T <= 8): routing in one launch, experts + combine in
// another; its counter block must start at zero and is left at zero.
size_t decode_state_bytes();
size_t decode_timeouts_offset();
bool decode_fusable(int T, int H, int I);
int decode_launches(moe_act_mode mode, int T, int k, int H, int I);
// Whether the single launch also runs a block's shared expert of width Is.
bool decode_fuses_shared(moe_act_mode mode, int T, int k, int H, int I, int Is);
// stage_mask: bit 0 routing (+ activation quantization), bit 1 experts + combine.
// shared_y: the shared expert's gated output, computed before the call, or
// (with fuse_sw, when decode_fuses_shared) by the single launch itself into
// shared_y and sh_h (its intermediate).
moe_status launch_layer_decode(const moe_nvfp4_experts& w, moe_act_mode mode, int stage_mask,
                               const uint16_t* x, const uint16_t* w_router, const float* bias,
                               int T, int k, const uint16_t* residual, uint16_t* out,
                               int32_t* ids, float* tw, int32_t* offsets, int32_t* sorted,
                               int32_t* prow, float* y, float* logits, void* ffn_ws, void* state,
                               const float* shared_y, hipStream_t s,
                               const moe_shared_expert* fuse_sw = nullptr, void* sh_h = nullptr);

}  // namespace moe
