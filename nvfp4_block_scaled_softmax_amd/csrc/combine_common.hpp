// The combine arithmetic shared by moe_combine and the fused decode kernel.
#pragma once
#include "device_common.hpp"

namespace moe {

// out values of token t, hidden 4c .. 4c+3: the weighted sum over the token's
// pairs in j order (fp32 fused multiply-adds), rounded to bf16, then the
// optional residual add in fp32 of the two bf16 values, rounded again.
template <bool COH = false>
__device__ __forceinline__ uint2 combine4(const float* __restrict__ y,
                                          const int32_t* __restrict__ pair_row,
                                          const float* __restrict__ w, int t, int k, int H, int c,
                                          const uint16_t* __restrict__ residual) {
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  constexpr int U = 8;
  for (int j0 = 0; j0 < k; j0 += U) {
    int r[U];
    float wj[U];
    float4 yv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u;
      r[u] = j < k ? pair_row[(size_t)t * k + j] : -1;
      wj[u] = j < k ? w[(size_t)t * k + j] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      yv[u] = r[u] >= 0 ? __builtin_bit_cast(float4, hld128<COH>(y, 4 * ((size_t)r[u] * H) + 16 * (size_t)c))
                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < U; ++u) {   // j ascending
      acc.x = __builtin_fmaf(wj[u], yv[u].x, acc.x);
      acc.y = __builtin_fmaf(wj[u], yv[u].y, acc.y);
      acc.z = __builtin_fmaf(wj[u], yv[u].z, acc.z);
      acc.w = __builtin_fmaf(wj[u], yv[u].w, acc.w);
    }
  }
  uint32_t o0 = f32_to_bf16(acc.x), o1 = f32_to_bf16(acc.y);
  uint32_t o2 = f32_to_bf16(acc.z), o3 = f32_to_bf16(acc.w);
  if (residual) {
    const uint2 rr = *reinterpret_cast<const uint2*>(residual + (size_t)t * H + (size_t)c * 4);
    o0 = f32_to_bf16(bf16_to_f32(rr.x & 0xFFFFu) + bf16_to_f32(o0));
    o1 = f32_to_bf16(bf16_to_f32(rr.x >> 16) + bf16_to_f32(o1));
    o2 = f32_to_bf16(bf16_to_f32(rr.y & 0xFFFFu) + bf16_to_f32(o2));
    o3 = f32_to_bf16(bf16_to_f32(rr.y >> 16) + bf16_to_f32(o3));
  }
  return make_uint2(o0 | (o1 << 16), o2 | (o3 << 16));
}

}  // namespace moe
