// Router: logits = x . Wr^T (+ bias), softmax, top-k, renormalise.
//
// The router is stored BF16 (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for
// Infernix (bit-exact)", section "What is bit-exact and what is quantized");
// 512 experts, the top 10 per token (same page, opening description).  The
// pages print no router formula; this is the Qwen-style reading (softmax over
// all experts, the k largest, weights renormalised over the chosen ones).
//
// Decode (T <= 8): the 512 x H router matrix is one HBM stream.  One wave per
// expert row; x sits in LDS; bf16 pairs meet in v_dot2_f32_bf16 (exact
// products, fp32 sums).
// Wide calls: a bf16 MFMA GEMM (16x16x32), operands read straight from
// global memory in the MFMA lane layout (both are K-contiguous).
// Top-k: one wave per token, k rounds of a wave argmax (ties to lower index).
#include "route_common.hpp"

namespace moe {

__global__ void __launch_bounds__(256) k_router_logits_narrow(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wr,
                                                              const float* __restrict__ bias,
                                                              int T, int H, int E,
                                                              float* __restrict__ logits) {
  extern __shared__ __align__(16) uint8_t smem[];
  router_logits_wave<256>(x, wr, bias, T, H, E, blockIdx.x * 4 + threadIdx.x / kWave,
                     reinterpret_cast<uint4*>(smem), logits);
}

// Wide logits (prefill): workgroup = 32 tokens x 32 experts, 4 waves splitting
// K into four ranges; each wave accumulates the whole 32 x 32 tile over its
// range (2 x 2 MFMA tiles, K 32 per step), keeping three steps of operands in
// flight in four register sets (the body names each set at a fixed place, so
// no copy waits on a load; loads past the range re-read its last step).  The
// four partial tiles meet in LDS and are summed in wave order, so the result
// does not depend on timing.  Rows past T or E read clamped rows and are not
// stored.
constexpr int kRtSets = 4;

__global__ void __launch_bounds__(256) k_router_logits_mfma(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ wr,
                                                            const float* __restrict__ bias,
                                                            int T, int H, int E,
                                                            float* __restrict__ logits) {
  __shared__ float part[4][32 * 32];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int t0 = blockIdx.y * 32, e0 = blockIdx.x * 32;
  const int r = lane & 15, g = lane >> 4;
  const int total = H / 32, per = (total + 3) / 4;
  const int n = max(0, min(per, total - wave * per));   // this wave's steps (0 for tiny H)
  const int k_first = n > 0 ? wave * per : 0;             // keeps every read inside its row
  const uint16_t* xa[2];
  const uint16_t* wb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    xa[i] = x + (size_t)min(t0 + 16 * i + r, T - 1) * H + 8 * g + 32 * k_first;
    wb[i] = wr + (size_t)min(e0 + 16 * i + r, E - 1) * H + 8 * g + 32 * k_first;
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 fa[kRtSets][2], fb[kRtSets][2];
  auto load = [&](uint4 (&a)[2], uint4 (&b)[2], int st) {
    const int k = 32 * min(st, max(n - 1, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      a[i] = *reinterpret_cast<const uint4*>(xa[i] + k);
      b[i] = *reinterpret_cast<const uint4*>(wb[i] + k);
    }
  };
#pragma unroll
  for (int d = 0; d < kRtSets - 1; ++d) load(fa[d], fb[d], d);
  for (int s0 = 0; s0 < n; s0 += kRtSets) {
#pragma unroll
    for (int u = 0; u < kRtSets; ++u) {
      const int st = s0 + u;
      load(fa[(u + kRtSets - 1) % kRtSets], fb[(u + kRtSets - 1) % kRtSets], st + kRtSets - 1);
      __builtin_amdgcn_sched_barrier(0);
      if (st < n) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                bitcast<bf16x8>(fa[u][i]), bitcast<bf16x8>(fb[u][j]), acc[i][j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // C layout: lane holds rows (tokens) 4g + q, column (expert) r of each tile.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) part[wave][(16 * i + 4 * g + q) * 32 + 16 * j + r] = acc[i][j][q];
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int idx = u * 256 + threadIdx.x;
    const int t = t0 + idx / 32, e = e0 + idx % 32;
    if (t < T && e < E) {
      const float v = ((part[0][idx] + part[1][idx]) + part[2][idx]) + part[3][idx];
      logits[(size_t)t * E + e] = v + (bias ? bias[e] : 0.0f);
    }
  }
}

template <int S>
__global__ void __launch_bounds__(256) k_topk(const float* __restrict__ logits, int T, int E,
                                              int k, int32_t* __restrict__ ids,
                                              float* __restrict__ w) {
  __shared__ TopkScratch sc[4];
  const int t = blockIdx.x * 4 + threadIdx.x / kWave;
  if (t < T) topk_wave<S>(logits, t, E, k, ids, w, nullptr, &sc[threadIdx.x / kWave]);
}

static void launch_topk(const float* logits, int T, int E, int k, int32_t* ids, float* w,
                        hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
  if (E <= 64) hipLaunchKernelGGL(k_topk<1>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 128) hipLaunchKernelGGL(k_topk<2>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 256) hipLaunchKernelGGL(k_topk<4>, grid, block, 0, s, logits, T, E, k, ids, w);
  else if (E <= 512) hipLaunchKernelGGL(k_topk<8>, grid, block, 0, s, logits, T, E, k, ids, w);
  else hipLaunchKernelGGL(k_topk<16>, grid, block, 0, s, logits, T, E, k, ids, w);
}

moe_status launch_route(const uint16_t* x, const uint16_t* w_router, const float* bias, int T,
                        int H, int E, int k, int32_t* ids, float* w, float* logits,
                        hipStream_t s) {
  if (T <= kNarrowT) {
    const size_t lds = (size_t)T * H * 2;
    hipLaunchKernelGGL(k_router_logits_narrow, dim3((E + 3) / 4), dim3(256), lds, s, x, w_router,
                       bias, T, H, E, logits);
  } else {
    hipLaunchKernelGGL(k_router_logits_mfma, dim3((E + 31) / 32, (T + 31) / 32), dim3(256), 0, s,
                       x, w_router, bias, T, H, E, logits);
  }
  moe_status st = check_launch("moe_route_topk (logits)");
  if (st != MOE_OK) return st;
  launch_topk(logits, T, E, k, ids, w, s);
  return check_launch("moe_route_topk (top-k)");
}

}  // namespace moe

extern "C" size_t moe_route_workspace_bytes(int T, int E) {
  if (T < 1 || E < 1) return 0;
  return moe::round_up((size_t)T * E * sizeof(float), 256);
}

extern "C" moe_status moe_route_topk(const uint16_t* x, const uint16_t* w_router, const float* bias,
                                     int T, int H, int E, int k, int32_t* topk_ids, float* topk_w,
                                     void* ws, size_t ws_bytes, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(x && w_router && topk_ids && topk_w && ws, MOE_E_ARG,
              "moe_route_topk: null pointer argument");
  MOE_REQUIRE(T >= 1 && moe::dim_ok(H) && E >= 1 && E <= moe::kMaxExperts && k >= 1 && k <= E &&
                  k <= moe::kMaxTopK,
              MOE_E_SHAPE, "moe_route_topk: bad shape T=%d H=%d E=%d k=%d", T, H, E, k);
  MOE_REQUIRE(moe::aligned(x, 16) && moe::aligned(w_router, 16) && moe::aligned(ws, 16) &&
                  moe::aligned(topk_ids, 4) && moe::aligned(topk_w, 4) &&
                  (!bias || moe::aligned(bias, 4)),
              MOE_E_ALIGN, "moe_route_topk: misaligned pointer");
  MOE_REQUIRE(ws_bytes >= moe_route_workspace_bytes(T, E), MOE_E_WORKSPACE,
              "moe_route_topk: workspace %zu < %zu bytes", ws_bytes, moe_route_workspace_bytes(T, E));
  return moe::launch_route(x, w_router, bias, T, H, E, k, topk_ids, topk_w,
                           static_cast<float*>(ws), s);
}
