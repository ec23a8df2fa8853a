// Combine: out[t] = bf16( sum_j w[t][j] * y[pair_row[t*k + j]] ), j ascending,
// optionally followed by the residual add bf16(x + out) of a decoder layer.
// One thread per 8 consecutive hidden values of a token: two 128-bit loads
// per chosen expert row, one 128-bit store.  No atomics: the order of the sum
// is fixed, so results are bitwise reproducible.
#include "abi_common.hpp"
#include "device_common.hpp"

namespace moe {

__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ pair_row,
                                                 const float* __restrict__ w, int T, int k, int H,
                                                 const uint16_t* __restrict__ residual,
                                                 uint16_t* __restrict__ out) {
  const int n8 = H / 8;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * n8) return;
  const int t = (int)(i / n8), c = (int)(i % n8);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < k; ++j) {
    const int r = pair_row[(size_t)t * k + j];
    if (r < 0) continue;
    const float wj = w[(size_t)t * k + j];
    const float4* p = reinterpret_cast<const float4*>(y + (size_t)r * H + (size_t)c * 8);
    const float4 a = p[0], b = p[1];
    acc[0] += wj * a.x; acc[1] += wj * a.y; acc[2] += wj * a.z; acc[3] += wj * a.w;
    acc[4] += wj * b.x; acc[5] += wj * b.y; acc[6] += wj * b.z; acc[7] += wj * b.w;
  }
  uint32_t o[4];
  uint4 res = make_uint4(0u, 0u, 0u, 0u);
  if (residual) res = *reinterpret_cast<const uint4*>(residual + (size_t)t * H + (size_t)c * 8);
  const uint32_t rw[4] = {res.x, res.y, res.z, res.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t lo = f32_to_bf16(acc[2 * q]), hi = f32_to_bf16(acc[2 * q + 1]);
    if (residual) {
      lo = f32_to_bf16(bf16_to_f32(rw[q] & 0xFFFFu) + bf16_to_f32(lo));
      hi = f32_to_bf16(bf16_to_f32(rw[q] >> 16) + bf16_to_f32(hi));
    }
    o[q] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4*>(out + (size_t)t * H + (size_t)c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

moe_status launch_combine(const float* y_pairs, const int32_t* pair_row, const float* topk_w,
                          int T, int k, int H, const uint16_t* residual, uint16_t* out,
                          hipStream_t s) {
  const int64_t n = (int64_t)T * (H / 8);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y_pairs,
                     pair_row, topk_w, T, k, H, residual, out);
  return check_launch("moe_combine");
}

}  // namespace moe

extern "C" moe_status moe_combine(const float* y_pairs, const int32_t* pair_row,
                                  const float* topk_w, int T, int k, int H,
                                  const uint16_t* residual, uint16_t* out, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(y_pairs && pair_row && topk_w && out, MOE_E_ARG, "moe_combine: null pointer argument");
  MOE_REQUIRE(T >= 1 && k >= 1 && k <= moe::kMaxExperts && moe::dim_ok(H), MOE_E_SHAPE,
              "moe_combine: bad shape T=%d k=%d H=%d", T, k, H);
  MOE_REQUIRE(moe::aligned(y_pairs, 16) && moe::aligned(out, 16) && moe::aligned(pair_row, 4) &&
                  moe::aligned(topk_w, 4) && (!residual || moe::aligned(residual, 16)),
              MOE_E_ALIGN, "moe_combine: misaligned pointer");
  return moe::launch_combine(y_pairs, pair_row, topk_w, T, k, H, residual, out, s);
}
