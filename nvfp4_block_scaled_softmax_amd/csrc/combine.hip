// Combine: out[t] = bf16( sum_j w[t][j] * y[pair_row[t*k + j]] ), j ascending,
// optionally followed by the residual add bf16(x + out) of a decoder layer.
// One thread per 4 consecutive hidden values of a token: every chosen expert
// row's 128-bit load is issued before the sum, then one 64-bit store.  No atomics: the order of the sum
// is fixed, so results are bitwise reproducible.
#include "abi_common.hpp"
#include "combine_common.hpp"

namespace moe {

__global__ void __launch_bounds__(256) k_combine(const float* __restrict__ y,
                                                 const int32_t* __restrict__ pair_row,
                                                 const float* __restrict__ w, int T, int k, int H,
                                                 const float* __restrict__ shared_y,
                                                 const uint16_t* __restrict__ residual,
                                                 uint16_t* __restrict__ out) {
  const int n4 = H / 4;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * n4) return;
  const int t = (int)(i / n4), c = (int)(i % n4);
  *reinterpret_cast<uint2*>(out + (size_t)t * H + (size_t)c * 4) =
      combine4(y, pair_row, w, t, k, H, c, residual, shared_y);
}

moe_status launch_combine(const float* y_pairs, const int32_t* pair_row, const float* topk_w,
                          int T, int k, int H, const float* shared_y, const uint16_t* residual,
                          uint16_t* out, hipStream_t s) {
  const int64_t n = (int64_t)T * (H / 4);
  hipLaunchKernelGGL(k_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, y_pairs,
                     pair_row, topk_w, T, k, H, shared_y, residual, out);
  return check_launch("moe_combine");
}

}  // namespace moe

static moe_status combine_entry(const char* name, const float* y_pairs, const int32_t* pair_row,
                                const float* topk_w, int T, int k, int H, const float* shared_y,
                                const uint16_t* residual, uint16_t* out, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(y_pairs && pair_row && topk_w && out, MOE_E_ARG, "%s: null pointer argument", name);
  MOE_REQUIRE(T >= 1 && k >= 1 && k <= moe::kMaxExperts && moe::dim_ok(H), MOE_E_SHAPE,
              "%s: bad shape T=%d k=%d H=%d", name, T, k, H);
  MOE_REQUIRE(moe::aligned(y_pairs, 16) && moe::aligned(out, 16) && moe::aligned(pair_row, 4) &&
                  moe::aligned(topk_w, 4) && (!residual || moe::aligned(residual, 16)) &&
                  (!shared_y || moe::aligned(shared_y, 16)),
              MOE_E_ALIGN, "%s: misaligned pointer", name);
  return moe::launch_combine(y_pairs, pair_row, topk_w, T, k, H, shared_y, residual, out, s);
}

extern "C" moe_status moe_combine(const float* y_pairs, const int32_t* pair_row,
                                  const float* topk_w, int T, int k, int H,
                                  const uint16_t* residual, uint16_t* out, hipStream_t s) {
  return combine_entry("moe_combine", y_pairs, pair_row, topk_w, T, k, H, nullptr, residual, out, s);
}

extern "C" moe_status moe_combine_shared(const float* y_pairs, const int32_t* pair_row, const float* topk_w,
                                         int T, int k, int H, const float* shared_y, const uint16_t* residual,
                                         uint16_t* out, hipStream_t s) {
  if (!shared_y) {
    moe::clear_error();
    moe::set_error("moe_combine_shared: null shared_y");
    return MOE_E_ARG;
  }
  return combine_entry("moe_combine_shared", y_pairs, pair_row, topk_w, T, k, H, shared_y, residual, out, s);
}
