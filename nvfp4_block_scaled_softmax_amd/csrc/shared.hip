// The shared expert and its gate (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for
// Infernix (bit-exact)", section "What is bit-exact and what is quantized":
// shared experts and gates are BF16 dense projections): two kernels, gate/up +
// SwiGLU into a bf16 intermediate, then down times the gate's sigmoid, on the
// tiles of shared_common.hpp.
#include "shared_common.hpp"

namespace moe {

template <int CPL>
__global__ void __launch_bounds__(kTileThreads) k_shared_gateup(SharedArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  shared_gateup_tile<CPL, false>(a, blockIdx.x, lds);
}

template <int CPL>
__global__ void __launch_bounds__(kTileThreads) k_shared_down(SharedArgs a) {
  extern __shared__ __align__(16) uint8_t lds[];
  shared_down_tile<CPL, false>(a, blockIdx.x, lds, NoHook{});
}

template <int CPL>
static void launch_sgu(const SharedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_gateup<CPL>, dim3(a.Is / kShGuRows), dim3(kTileThreads),
                     (size_t)a.tg * a.H * 2, s, a);
}

template <int CPL>
static void launch_sdn(const SharedArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_shared_down<CPL>, dim3((a.H + kShDnRows - 1) / kShDnRows), dim3(kTileThreads),
                     (size_t)kShTok * a.Is * 2, s, a);
}

moe_status launch_shared(const SharedArgs& a, hipStream_t s) {
  switch (shared_gu_cpl(a.H)) {
#define GU(C) case C: launch_sgu<C>(a, s); break;
    GU(1) GU(2) GU(3) GU(4) GU(5) GU(6) GU(7) GU(8) GU(9) GU(10) GU(11) GU(12) GU(13) GU(14) GU(15) GU(16)
#undef GU
    default: set_error("shared expert: H=%d", a.H); return MOE_E_SHAPE;
  }
  moe_status st = check_launch("moe_shared_expert_forward (gate/up)");
  if (st != MOE_OK) return st;
  switch (shared_dn_cpl(a.Is)) {
#define DN(C) case C: launch_sdn<C>(a, s); break;
    DN(1) DN(2) DN(3) DN(4) DN(5) DN(6) DN(7) DN(8)
#undef DN
    default: set_error("shared expert: Is=%d", a.Is); return MOE_E_SHAPE;
  }
  return check_launch("moe_shared_expert_forward (down)");
}

size_t shared_workspace(int T, int Is) { return round_up((size_t)T * Is * 2, 256); }

moe_status check_shared(const char* name, const moe_shared_expert* sw, int H) {
  MOE_REQUIRE(sw, MOE_E_ARG, "%s: null shared expert", name);
  MOE_REQUIRE(sw->gu && sw->dn && sw->gate, MOE_E_ARG, "%s: null shared expert array", name);
  MOE_REQUIRE(sw->H == H && dim_ok(sw->H) && sw->Is >= 32 && sw->Is <= kShMaxIs && sw->Is % 32 == 0, MOE_E_SHAPE,
              "%s: bad shared expert shape H=%d Is=%d (Is: a multiple of 32 up to %d; H as the layer's)", name,
              sw->H, sw->Is, kShMaxIs);
  MOE_REQUIRE(aligned(sw->gu, 16) && aligned(sw->dn, 16) && aligned(sw->gate, 16), MOE_E_ALIGN,
              "%s: misaligned shared expert array", name);
  return MOE_OK;
}

SharedArgs make_shared_args(const moe_shared_expert& sw, const uint16_t* x, int T, void* h_ws, float* y) {
  SharedArgs a;
  a.gu = sw.gu;
  a.dn = sw.dn;
  a.gate = sw.gate;
  a.x = x;
  a.H = sw.H;
  a.Is = sw.Is;
  a.T = T;
  a.h = static_cast<uint16_t*>(h_ws);
  a.y = y;
  a.tg = shared_tok_group(sw.H);
  return a;
}

moe_status launch_shared_expert(const moe_shared_expert& sw, const uint16_t* x, int T, void* h_ws, float* y,
                                hipStream_t s) {
  return launch_shared(make_shared_args(sw, x, T, h_ws, y), s);
}

}  // namespace moe

extern "C" size_t moe_shared_expert_workspace_bytes(int T, int Is) {
  if (T < 1 || Is < 32 || Is > moe::kShMaxIs || Is % 32 != 0) return 0;
  return moe::shared_workspace(T, Is);
}

extern "C" moe_status moe_shared_expert_forward(const moe_shared_expert* sw, const uint16_t* x, int T, float* y,
                                                void* ws, size_t ws_bytes, hipStream_t s) {
  const char* name = "moe_shared_expert_forward";
  moe::clear_error();
  MOE_REQUIRE(sw, MOE_E_ARG, "%s: null shared expert", name);
  moe_status st = moe::check_shared(name, sw, sw->H);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(x && y && ws, MOE_E_ARG, "%s: null pointer argument", name);
  MOE_REQUIRE(T >= 1 && T <= (1 << 20), MOE_E_SHAPE, "%s: bad T=%d", name, T);
  MOE_REQUIRE(moe::aligned(x, 16) && moe::aligned(y, 16) && moe::aligned(ws, 16), MOE_E_ALIGN,
              "%s: misaligned pointer", name);
  const size_t need = moe::shared_workspace(T, sw->Is);
  MOE_REQUIRE(ws_bytes >= need, MOE_E_WORKSPACE, "%s: workspace %zu < %zu bytes", name, ws_bytes, need);
  return moe::launch_shared_expert(*sw, x, T, ws, y, s);
}
