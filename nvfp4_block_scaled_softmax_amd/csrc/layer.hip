// The whole routed-expert layer on one stream (route -> permute -> experts ->
// combine), its workspace layout, and the thread-local error text.
#include <mutex>
#include <string>

#include "abi_common.hpp"

namespace moe {

static thread_local std::string g_error;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
}

void clear_error() { g_error.clear(); }

moe_status check_experts(const char* name, const moe_nvfp4_experts* w, moe_act_mode mode);

struct LayerLayout {
  size_t ids, w, offsets, sorted, pair_row, y, ffn, route, state, sh_h, sh_y, total;
};

// Is > 0: a shared expert of that intermediate size; its segments (bf16 h
// [T][Is], gated fp32 y [T][H]) come last, so every other offset is the same
// with or without it.
static bool layer_layout(moe_act_mode mode, int T, int k, int E, int H, int I, LayerLayout& L, int Is = 0) {
  if (T < 1 || k < 1 || k > kMaxTopK || E < 1 || E > kMaxExperts || k > E || !dim_ok(H) || !dim_ok(I) ||
      (int64_t)T * k > (1 << 24))
    return false;
  if (mode != MOE_A16 && mode != MOE_A8 && mode != MOE_A4) return false;
  const size_t P = (size_t)T * k;
  size_t o = 0;
  auto seg = [&](size_t bytes) { const size_t at = o; o = round_up(o + bytes, 256); return at; };
  // first, so its place does not depend on the call's sizes (one workspace
  // may serve calls of several token counts)
  L.state = seg(decode_state_bytes());   // zero before the first call, left zero by each call
  L.ids = seg(P * 4);
  L.w = seg(P * 4);
  L.offsets = seg((size_t)(E + 1) * 4);
  L.sorted = seg(P * 4);
  L.pair_row = seg(P * 4);
  L.y = seg(P * H * 4);
  L.ffn = seg(expert_ffn_workspace(mode, T, k, H, I));
  // router logits, dead after top-k; then the permutation's block counts
  const size_t route = (size_t)T * E * 4, perm = permute_workspace((int)P, E);
  L.route = seg(route > perm ? route : perm);
  L.sh_h = L.sh_y = 0;
  if (Is > 0) {
    L.sh_h = seg(shared_workspace(T, Is));
    L.sh_y = seg((size_t)T * H * 4);
  }
  L.total = o;
  return true;
}

}  // namespace moe

extern "C" const char* moe_last_error(void) { return moe::g_error.c_str(); }

extern "C" int moe_layer_is_fused(int T, int H, int I) { return moe::decode_fusable(T, H, I) ? 1 : 0; }

extern "C" int moe_layer_launches(moe_act_mode mode, int T, int k, int H, int I) {
  return moe::decode_launches(mode, T, k, H, I);
}

extern "C" int moe_block_launches(moe_act_mode mode, int T, int k, int H, int I, int Is) {
  if (moe::decode_fuses_shared(mode, T, k, H, I, Is)) return 1;
  const int n = moe::decode_launches(mode, T, k, H, I);
  return n > 0 ? n + 2 : 0;
}

extern "C" size_t moe_layer_wait_timeouts_offset(void) {
  return moe::decode_timeouts_offset();   // the state block is at the start of the workspace
}

extern "C" size_t moe_layer_workspace_bytes(moe_act_mode mode, int T, int k, int E, int H, int I) {
  moe::LayerLayout L;
  return moe::layer_layout(mode, T, k, E, H, I, L) ? L.total : 0;
}

extern "C" moe_status moe_layer_workspace_layout(moe_act_mode mode, int T, int k, int E, int H,
                                                 int I, size_t offsets[7]) {
  moe::clear_error();
  MOE_REQUIRE(offsets, MOE_E_ARG, "moe_layer_workspace_layout: null offsets");
  moe::LayerLayout L;
  MOE_REQUIRE(moe::layer_layout(mode, T, k, E, H, I, L), MOE_E_SHAPE,
              "moe_layer_workspace_layout: bad shape or mode");
  offsets[0] = L.ids;
  offsets[1] = L.w;
  offsets[2] = L.offsets;
  offsets[3] = L.sorted;
  offsets[4] = L.pair_row;
  offsets[5] = L.y;
  offsets[6] = L.ffn;
  return MOE_OK;
}

static moe_status layer_call(const char* name, const moe_nvfp4_experts* w, moe_act_mode mode,
                             int stage_mask, const uint16_t* x, const uint16_t* w_router,
                             const float* router_bias, int T, int k, const uint16_t* residual,
                             uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s,
                             const moe_shared_expert* sw = nullptr) {
  moe::clear_error();
  moe_status st = moe::check_experts(name, w, mode);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(x && w_router && out && ws, MOE_E_ARG, "%s: null pointer argument", name);
  if (sw && (st = moe::check_shared(name, sw, w->H)) != MOE_OK) return st;
  moe::LayerLayout L;
  MOE_REQUIRE(moe::layer_layout(mode, T, k, w->E, w->H, w->I, L, sw ? sw->Is : 0), MOE_E_SHAPE,
              "%s: bad shape T=%d k=%d", name, T, k);
  mode = moe::kernel_mode(*w, mode);   // (q4_g64_fp16 experts: the fp16 kernels; the layout is the same)
  MOE_REQUIRE(out != x, MOE_E_ARG, "%s: out must not alias x", name);
  MOE_REQUIRE(moe::aligned(x, 16) && moe::aligned(w_router, 16) && moe::aligned(out, 16) &&
                  moe::aligned(ws, 256) && (!residual || moe::aligned(residual, 16)) &&
                  (!router_bias || moe::aligned(router_bias, 4)),
              MOE_E_ALIGN, "%s: misaligned pointer (workspace needs 256 bytes)", name);
  MOE_REQUIRE(ws_bytes >= L.total, MOE_E_WORKSPACE, "%s: workspace %zu < %zu bytes", name,
              ws_bytes, L.total);
  uint8_t* b = static_cast<uint8_t*>(ws);
  int32_t* ids = reinterpret_cast<int32_t*>(b + L.ids);
  float* tw = reinterpret_cast<float*>(b + L.w);
  int32_t* offs = reinterpret_cast<int32_t*>(b + L.offsets);
  int32_t* sorted = reinterpret_cast<int32_t*>(b + L.sorted);
  int32_t* prow = reinterpret_cast<int32_t*>(b + L.pair_row);
  float* y = reinterpret_cast<float*>(b + L.y);
  // the shared expert needs no routing: the single decode launch runs it too
  // (decode_fuses_shared); otherwise its kernels go first, with the routing half
  float* shy = sw ? reinterpret_cast<float*>(b + L.sh_y) : nullptr;
  const bool fuse_sw = sw && stage_mask == 3 && moe::decode_fuses_shared(mode, T, k, w->H, w->I, sw->Is);
  if (sw && !fuse_sw && (stage_mask & 1) &&
      (st = moe::launch_shared_expert(*sw, x, T, b + L.sh_h, shy, s)) != MOE_OK)
    return st;
  if (moe::decode_fusable(T, w->H, w->I))
    return moe::launch_layer_decode(*w, mode, stage_mask, x, w_router, router_bias, T, k,
                                    residual, out, ids, tw, offs, sorted, prow, y,
                                    reinterpret_cast<float*>(b + L.route), b + L.ffn, b + L.state, shy, s,
                                    fuse_sw ? sw : nullptr, b + L.sh_h);
  if (stage_mask & 1) {
    if ((st = moe::launch_route(x, w_router, router_bias, T, w->H, w->E, k, ids, tw,
                                reinterpret_cast<float*>(b + L.route), s)) != MOE_OK)
      return st;
    if ((st = moe::launch_permute(ids, T, k, w->E, offs, sorted, prow, b + L.route, s)) != MOE_OK)
      return st;
    if ((st = moe::launch_expert_ffn(*w, mode, x, T, k, offs, sorted, y, b + L.ffn, 1, s, prow, ids)) != MOE_OK)
      return st;
  }
  if (stage_mask & 2) {
    if ((st = moe::launch_expert_ffn(*w, mode, x, T, k, offs, sorted, y, b + L.ffn, 6, s)) != MOE_OK)
      return st;
    return moe::launch_combine(y, prow, tw, T, k, w->H, shy, residual, out, s);
  }
  return MOE_OK;
}

extern "C" moe_status moe_layer_forward(const moe_nvfp4_experts* w, moe_act_mode mode,
                                        const uint16_t* x, const uint16_t* w_router,
                                        const float* router_bias, int T, int k,
                                        const uint16_t* residual, uint16_t* out, void* ws,
                                        size_t ws_bytes, hipStream_t s) {
  return layer_call("moe_layer_forward", w, mode, 3, x, w_router, router_bias, T, k, residual, out,
                    ws, ws_bytes, s);
}

extern "C" moe_status moe_layer_forward_stage(const moe_nvfp4_experts* w, moe_act_mode mode,
                                              int stage, const uint16_t* x,
                                              const uint16_t* w_router, const float* router_bias,
                                              int T, int k, const uint16_t* residual,
                                              uint16_t* out, void* ws, size_t ws_bytes,
                                              hipStream_t s) {
  if (stage != 0 && stage != 1) {
    moe::clear_error();
    moe::set_error("moe_layer_forward_stage: stage %d is not 0 or 1", stage);
    return MOE_E_ARG;
  }
  return layer_call("moe_layer_forward_stage", w, mode, 1 << stage, x, w_router, router_bias, T,
                    k, residual, out, ws, ws_bytes, s);
}

extern "C" moe_status moe_layer_status(const void* ws, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(ws, MOE_E_ARG, "moe_layer_status: null workspace");
  uint32_t v = 0u;
  hipError_t e = hipMemcpyAsync(&v, static_cast<const uint8_t*>(ws) + moe::decode_timeouts_offset(), 4,
                                hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  MOE_REQUIRE(e == hipSuccess, MOE_E_HIP, "moe_layer_status: %s", hipGetErrorString(e));
  MOE_REQUIRE(v == 0u, MOE_E_STALLED,
              "moe_layer_status: %u wait(s) of the fused decode path gave up on this workspace; "
              "the outputs of the calls since it was zero-filled are unreliable (NaN where seen)",
              v);
  return MOE_OK;
}

// ------------------------------------------------------------------ with the shared expert
extern "C" size_t moe_block_workspace_bytes(moe_act_mode mode, int T, int k, int E, int H, int I, int Is) {
  moe::LayerLayout L;
  if (Is < 32 || Is > 1024 || Is % 32 != 0) return 0;
  return moe::layer_layout(mode, T, k, E, H, I, L, Is) ? L.total : 0;
}

extern "C" moe_status moe_block_workspace_layout(moe_act_mode mode, int T, int k, int E, int H, int I, int Is,
                                                 size_t offsets[9]) {
  moe::clear_error();
  MOE_REQUIRE(offsets, MOE_E_ARG, "moe_block_workspace_layout: null offsets");
  moe::LayerLayout L;
  MOE_REQUIRE(Is >= 32 && Is <= 1024 && Is % 32 == 0 && moe::layer_layout(mode, T, k, E, H, I, L, Is), MOE_E_SHAPE,
              "moe_block_workspace_layout: bad shape or mode");
  const size_t v[9] = {L.ids, L.w, L.offsets, L.sorted, L.pair_row, L.y, L.ffn, L.sh_h, L.sh_y};
  for (int i = 0; i < 9; ++i) offsets[i] = v[i];
  return MOE_OK;
}

extern "C" moe_status moe_block_forward(const moe_nvfp4_experts* w, const moe_shared_expert* sw,
                                        moe_act_mode mode, const uint16_t* x, const uint16_t* w_router,
                                        const float* router_bias, int T, int k, const uint16_t* residual,
                                        uint16_t* out, void* ws, size_t ws_bytes, hipStream_t s) {
  if (!sw) {
    moe::clear_error();
    moe::set_error("moe_block_forward: null shared expert (use moe_layer_forward)");
    return MOE_E_ARG;
  }
  return layer_call("moe_block_forward", w, mode, 3, x, w_router, router_bias, T, k, residual, out, ws, ws_bytes,
                    s, sw);
}

// ------------------------------------------------------------------ no allocation
// moe_layer_forward_noalloc: moe_layer_forward with the library's own device
// scratch array as the workspace, for callers that cannot allocate.  Each GPU
// holds its own copy of `scratch` (a file-scope device array of kScratchBytes)
// until the process ends.  In host code the array's name is only a stand-in for
// the symbol: its device address on the current GPU comes from
// hipGetSymbolAddress, taken once per device on that device's first call and
// kept; kernels and fills get that address, never the name.

namespace moe {

constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

// Zero-fill of n16 16-byte words: a kernel, not hipMemsetAsync, so that a call
// recorded into a graph replays it correctly.
__global__ void __launch_bounds__(256) k_zero16(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

static moe_status zero_fill(void* p, size_t bytes, hipStream_t s) {
  hipLaunchKernelGGL(k_zero16, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p), bytes / 16);
  return check_launch("moe_layer_forward_noalloc (scratch fill)");
}

// This device's scratch address, zero-filled on stream s at the device's first
// call (the address is kept only once its fill is enqueued) or when asked to.
static moe_status scratch_for_device(void** ptr, bool reset, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  MOE_REQUIRE(e == hipSuccess, MOE_E_HIP, "moe_layer_forward_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  MOE_REQUIRE(dev >= 0 && dev < kMaxDevices, MOE_E_UNSUPPORTED, "moe_layer_forward_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  void* p = g_scratch_ptr[dev];
  const bool first = p == nullptr;
  if (first) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    MOE_REQUIRE(e == hipSuccess && p != nullptr, MOE_E_HIP,
                "moe_layer_forward_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  }
  if (first || reset) {   // the state block at its start must be zero before a fused call uses it
    moe_status st = zero_fill(p, kScratchBytes, s);
    if (st != MOE_OK) return st;
  }
  g_scratch_ptr[dev] = p;
  *ptr = p;
  return MOE_OK;
}

}  // namespace moe

extern "C" moe_status moe_layer_forward_noalloc(const moe_nvfp4_experts* w, moe_act_mode mode,
                                                const uint16_t* x, const uint16_t* w_router,
                                                const float* router_bias, int T, int k,
                                                const uint16_t* residual, uint16_t* out, int reset,
                                                hipStream_t s) {
  const char* name = "moe_layer_forward_noalloc";
  moe::clear_error();
  moe_status st = moe::check_experts(name, w, mode);
  if (st != MOE_OK) return st;
  const size_t need = moe_layer_workspace_bytes(mode, T, k, w->E, w->H, w->I);
  MOE_REQUIRE(need > 0, MOE_E_SHAPE, "%s: bad shape T=%d k=%d", name, T, k);
  MOE_REQUIRE(need <= moe::kScratchBytes, MOE_E_WORKSPACE,
              "%s: the call needs a %zu-byte workspace, above the %zu-byte device scratch; "
              "use moe_layer_forward with a workspace",
              name, need, moe::kScratchBytes);
  void* ws = nullptr;
  if ((st = moe::scratch_for_device(&ws, reset != 0, s)) != MOE_OK) return st;
  return layer_call(name, w, mode, 3, x, w_router, router_bias, T, k, residual, out, ws, moe::kScratchBytes, s);
}
