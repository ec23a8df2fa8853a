// moe_nvfp4_repack: canonical NVFP4 experts into the tiled scale layout, bit
// for bit (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)",
// section "What is bit-exact and what is quantized": the checkpoint is
// repacked into the engine's expert layout without changing a bit).  Codes are
// copied as they are; each scale pair (the two E4M3 scales of a 32-value
// chunk) moves to its tiled position within its row (tiled_pair).
#include <algorithm>

#include "ffn_common.hpp"

namespace moe {

// One thread per scale pair of rows x nc pairs, grid-stride.
__global__ void __launch_bounds__(256)
    k_repack_scales(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, size_t rows, int nc) {
  const size_t n = rows * (size_t)nc;
  for (size_t i = blockIdx.x * (size_t)256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const size_t row = i / (size_t)nc;
    const int c = (int)(i - row * (size_t)nc);
    dst[row * (size_t)nc + (size_t)tiled_pair(c, nc)] = src[i];
  }
}

static moe_status repack_scales(const uint8_t* src, const uint8_t* dst, size_t rows, int nc, hipStream_t s) {
  const size_t n = rows * (size_t)nc;
  const size_t blocks = std::min<size_t>((n + 255) / 256, (size_t)1 << 20);
  hipLaunchKernelGGL(k_repack_scales, dim3((unsigned)blocks), dim3(256), 0, s, reinterpret_cast<const uint16_t*>(src),
                     reinterpret_cast<uint16_t*>(const_cast<uint8_t*>(dst)), rows, nc);
  return check_launch("moe_nvfp4_repack");
}

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

}  // namespace moe

extern "C" moe_status moe_nvfp4_repack(const moe_nvfp4_experts* src, const moe_nvfp4_experts* dst, hipStream_t s) {
  const char* name = "moe_nvfp4_repack";
  moe::clear_error();
  MOE_REQUIRE(src && dst, MOE_E_ARG, "%s: null expert set", name);
  MOE_REQUIRE(src->fmt == MOE_FMT_NVFP4 && dst->fmt == MOE_FMT_NVFP4, MOE_E_ARG, "%s: NVFP4 experts only", name);
  MOE_REQUIRE(src->layout == MOE_LAYOUT_CANONICAL && dst->layout == MOE_LAYOUT_TILED, MOE_E_ARG,
              "%s: src must be canonical (layout %d) and dst tiled (layout %d)", name, (int)src->layout,
              (int)dst->layout);
  MOE_REQUIRE(src->gu_codes && src->gu_scales && src->dn_codes && src->dn_scales && dst->gu_codes &&
                  dst->gu_scales && dst->dn_codes && dst->dn_scales,
              MOE_E_ARG, "%s: null code or scale array", name);
  MOE_REQUIRE(src->E == dst->E && src->H == dst->H && src->I == dst->I, MOE_E_SHAPE,
              "%s: shapes differ (E=%d/%d H=%d/%d I=%d/%d)", name, src->E, dst->E, src->H, dst->H, src->I, dst->I);
  MOE_REQUIRE(src->E >= 1 && src->E <= moe::kMaxExperts && moe::dim_ok(src->H) && moe::dim_ok(src->I) &&
                  src->H % 128 == 0 && src->I % 128 == 0,
              MOE_E_SHAPE, "%s: bad shape E=%d H=%d I=%d (H and I: multiples of 128)", name, src->E, src->H,
              src->I);
  MOE_REQUIRE(moe::aligned(src->gu_codes, 16) && moe::aligned(src->gu_scales, 16) && moe::aligned(src->dn_codes, 16) &&
                  moe::aligned(src->dn_scales, 16) && moe::aligned(dst->gu_codes, 16) &&
                  moe::aligned(dst->gu_scales, 16) && moe::aligned(dst->dn_codes, 16) &&
                  moe::aligned(dst->dn_scales, 16),
              MOE_E_ALIGN, "%s: misaligned array", name);
  const size_t E = (size_t)src->E, H = (size_t)src->H, I = (size_t)src->I;
  const size_t gu_sc = E * 2 * I * (H / 16), dn_sc = E * H * (I / 16);
  const size_t gu_cd = E * 2 * I * (H / 2), dn_cd = E * H * (I / 2);
  MOE_REQUIRE(!moe::overlap(dst->gu_scales, gu_sc, src->gu_scales, gu_sc) &&
                  !moe::overlap(dst->gu_scales, gu_sc, src->dn_scales, dn_sc) &&
                  !moe::overlap(dst->dn_scales, dn_sc, src->gu_scales, gu_sc) &&
                  !moe::overlap(dst->dn_scales, dn_sc, src->dn_scales, dn_sc) &&
                  !moe::overlap(dst->gu_scales, gu_sc, dst->dn_scales, dn_sc),
              MOE_E_ARG, "%s: dst scale arrays overlap src's or each other", name);
  if (dst->gu_codes != src->gu_codes) {
    MOE_REQUIRE(!moe::overlap(dst->gu_codes, gu_cd, src->gu_codes, gu_cd), MOE_E_ARG,
                "%s: dst gate/up codes partly overlap src's", name);
    MOE_REQUIRE(hipMemcpyAsync(const_cast<uint8_t*>(dst->gu_codes), src->gu_codes, gu_cd, hipMemcpyDeviceToDevice,
                               s) == hipSuccess,
                MOE_E_HIP, "%s: copy of the gate/up codes failed", name);
  }
  if (dst->dn_codes != src->dn_codes) {
    MOE_REQUIRE(!moe::overlap(dst->dn_codes, dn_cd, src->dn_codes, dn_cd), MOE_E_ARG,
                "%s: dst down codes partly overlap src's", name);
    MOE_REQUIRE(hipMemcpyAsync(const_cast<uint8_t*>(dst->dn_codes), src->dn_codes, dn_cd, hipMemcpyDeviceToDevice,
                               s) == hipSuccess,
                MOE_E_HIP, "%s: copy of the down codes failed", name);
  }
  moe_status st = moe::repack_scales(src->gu_scales, dst->gu_scales, E * 2 * I, (int)(H / 32), s);
  if (st != MOE_OK) return st;
  return moe::repack_scales(src->dn_scales, dst->dn_scales, E * H, (int)(I / 32), s);
}
