// The combine arithmetic shared by moe_combine and the fused decode kernel.
#pragma once
#include "device_common.hpp"

namespace moe {

// The weighted sum over token t's pairs in j order (fp32 fused multiply-adds)
// of four consecutive hidden values; load_y(r) gives them for sorted row r.
template <bool COH = false, typename LoadY>
__device__ __forceinline__ float4 combine_acc4(LoadY&& load_y, const int32_t* pair_row,
                                               const float* w, int t, int k) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int U = 8;
  for (int j0 = 0; j0 < k; j0 += U) {
    int r[U];
    float wj[U];
    float4 yv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      r[u] = j < k ? (int)hld32<COH>(pair_row, 4 * ((size_t)t * k + j)) : -1;
      wj[u] = j < k ? __builtin_bit_cast(float, hld32<COH>(w, 4 * ((size_t)t * k + j))) : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) yv[u] = r[u] >= 0 ? load_y(r[u]) : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u) {   // j ascending
      acc.x = __builtin_fmaf(wj[u], yv[u].x, acc.x);
      acc.y = __builtin_fmaf(wj[u], yv[u].y, acc.y);
      acc.z = __builtin_fmaf(wj[u], yv[u].z, acc.z);
      acc.w = __builtin_fmaf(wj[u], yv[u].w, acc.w);
    }
  }
  return acc;
}

// The sum rounded to bf16, then (with a residual: rr holds its four bf16
// values) the residual added in fp32 and rounded again.
__device__ __forceinline__ uint2 combine_round4(float4 acc, bool has_residual, uint2 rr) {
  uint32_t o0 = f32_to_bf16(acc.x), o1 = f32_to_bf16(acc.y);
  uint32_t o2 = f32_to_bf16(acc.z), o3 = f32_to_bf16(acc.w);
  if (has_residual) {
    o0 = f32_to_bf16(bf16_to_f32(rr.x & 0xFFFFu) + bf16_to_f32(o0));
    o1 = f32_to_bf16(bf16_to_f32(rr.x >> 16) + bf16_to_f32(o1));
    o2 = f32_to_bf16(bf16_to_f32(rr.y & 0xFFFFu) + bf16_to_f32(o2));
    o3 = f32_to_bf16(bf16_to_f32(rr.y >> 16) + bf16_to_f32(o3));
  }
  return make_uint2(o0 | (o1 << 16), o2 | (o3 << 16));
}

// The shared expert's gated output (fp32 [T][H], nullable) joins the routed
// sum after its last term, before the rounding.
__device__ __forceinline__ void add_shared4(float4& acc, const float* __restrict__ shared_y, int t, int H, int c) {
  if (shared_y) {
    const float4 sv = *reinterpret_cast<const float4*>(shared_y + (size_t)t * H + (size_t)c * 4);
    acc.x += sv.x;
    acc.y += sv.y;
    acc.z += sv.z;
    acc.w += sv.w;
  }
}

// out values of token t, hidden 4c .. 4c+3, from y_pairs in global memory.
template <bool COH = false>
__device__ __forceinline__ uint2 combine4(const float* __restrict__ y,
                                          const int32_t* __restrict__ pair_row,
                                          const float* __restrict__ w, int t, int k, int H, int c,
                                          const uint16_t* __restrict__ residual,
                                          const float* __restrict__ shared_y = nullptr) {
  float4 acc = combine_acc4<COH>(
      [&](int r) {
        return __builtin_bit_cast(float4, hld128<COH>(y, 4 * ((size_t)r * H) + 16 * (size_t)c));
      },
      pair_row, w, t, k);
  add_shared4(acc, shared_y, t, H, c);
  const uint2 rr = residual ? *reinterpret_cast<const uint2*>(residual + (size_t)t * H + (size_t)c * 4)
                            : make_uint2(0u, 0u);
  return combine_round4(acc, residual != nullptr, rr);
}

}  // namespace moe
