// Per-16 block quantizers (NVFP4 and the 8-bit activation mode) and the
// per-matrix NVFP4 multiplier.
//
// NVFP4: E2M1 codes, one E4M3 scale per 16, one fp32 multiplier per matrix
// (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix (bit-exact)", section
// "What is bit-exact and what is quantized"); 8-bit mode: page "Infernix",
// section "Activation precision".  One thread per block of 16: the block is
// 32 B (bf16) or 64 B (fp32) of contiguous input, so consecutive threads read
// consecutive memory.
#include "abi_common.hpp"
#include "device_common.hpp"

namespace moe {

template <bool F32>
__device__ __forceinline__ void load16(const void* x, size_t off, float* v) {
  if (F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(x) + off);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 u = p[q];
      v[4 * q + 0] = __uint_as_float(u.x);
      v[4 * q + 1] = __uint_as_float(u.y);
      v[4 * q + 2] = __uint_as_float(u.z);
      v[4 * q + 3] = __uint_as_float(u.w);
    }
  } else {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint4 u = p[q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = bf16_to_f32(w[i] & 0xFFFFu);
        v[8 * q + 2 * i + 1] = bf16_to_f32(w[i] >> 16);
      }
    }
  }
}

template <bool F32>
__global__ void __launch_bounds__(256) k_quant_nvfp4(const void* __restrict__ x, int rows, int cols,
                                                     const float* __restrict__ global,
                                                     const int32_t* __restrict__ row_group,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales) {
  const int nb = cols / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * nb) return;
  const int r = (int)(i / nb), b = (int)(i % nb);
  float v[16];
  load16<F32>(x, (size_t)r * cols + (size_t)b * 16, v);
  const float g = global[row_group ? row_group[r] : 0];
  uint32_t lo, hi;
  const uint32_t s = nvfp4_quant16(v, g, lo, hi);
  *reinterpret_cast<uint2*>(codes + (size_t)r * (cols / 2) + (size_t)b * 8) = make_uint2(lo, hi);
  scales[(size_t)r * nb + b] = (uint8_t)s;
}

template <bool F32>
__global__ void __launch_bounds__(256) k_quant_fp8(const void* __restrict__ x, int rows, int cols,
                                                   uint8_t* __restrict__ codes,
                                                   float* __restrict__ scales) {
  const int nb = cols / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)rows * nb) return;
  const int r = (int)(i / nb), b = (int)(i % nb);
  float v[16];
  load16<F32>(x, (size_t)r * cols + (size_t)b * 16, v);
  uint32_t w[4];
  const float s = fp8_quant16(v, w);
  *reinterpret_cast<uint4*>(codes + (size_t)r * cols + (size_t)b * 16) = make_uint4(w[0], w[1], w[2], w[3]);
  scales[(size_t)r * nb + b] = s;
}

// One workgroup per matrix: amax over mat_elems fp32 values, then amax / 2688.
__global__ void __launch_bounds__(1024) k_global_scale(const float* __restrict__ x,
                                                       int64_t mat_elems,
                                                       float* __restrict__ global) {
  __shared__ float red[1024 / kWave];
  const float4* p = reinterpret_cast<const float4*>(x + (size_t)blockIdx.x * mat_elems);
  const int64_t n4 = mat_elems / 4;
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n4; i += blockDim.x) {
    const float4 v = p[i];
    m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v.x), __builtin_fabsf(v.y)),
                                           __builtin_fmaxf(__builtin_fabsf(v.z), __builtin_fabsf(v.w))));
  }
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, kWave));
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float a = 0.0f;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) a = __builtin_fmaxf(a, red[w]);
    global[blockIdx.x] = __fdiv_rn(a, 2688.0f);
  }
}

}  // namespace moe

namespace {
moe_status check_quant_args(const char* name, const void* x, moe_dtype xdt, int rows, int cols) {
  MOE_REQUIRE(x, MOE_E_ARG, "%s: null input", name);
  MOE_REQUIRE(xdt == MOE_DT_BF16 || xdt == MOE_DT_F32, MOE_E_ARG, "%s: bad dtype %d", name, (int)xdt);
  MOE_REQUIRE(rows >= 1 && cols >= 32 && cols % 32 == 0 && (int64_t)rows * cols <= (1ll << 40),
              MOE_E_SHAPE, "%s: bad shape rows=%d cols=%d", name, rows, cols);
  MOE_REQUIRE(moe::aligned(x, 16), MOE_E_ALIGN, "%s: input not 16-byte aligned", name);
  return MOE_OK;
}
}  // namespace

extern "C" moe_status act_quant_nvfp4(const void* x, moe_dtype xdt, int rows, int cols,
                                      const float* global, const int32_t* row_group,
                                      uint8_t* codes, uint8_t* scales, hipStream_t s) {
  moe::clear_error();
  moe_status st = check_quant_args("act_quant_nvfp4", x, xdt, rows, cols);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(global && codes && scales, MOE_E_ARG, "act_quant_nvfp4: null pointer argument");
  MOE_REQUIRE(moe::aligned(codes, 8) && moe::aligned(global, 4) &&
                  (!row_group || moe::aligned(row_group, 4)),
              MOE_E_ALIGN, "act_quant_nvfp4: misaligned pointer");
  const int64_t n = (int64_t)rows * (cols / 16);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (xdt == MOE_DT_F32)
    hipLaunchKernelGGL(moe::k_quant_nvfp4<true>, dim3(grid), dim3(256), 0, s, x, rows, cols, global,
                       row_group, codes, scales);
  else
    hipLaunchKernelGGL(moe::k_quant_nvfp4<false>, dim3(grid), dim3(256), 0, s, x, rows, cols, global,
                       row_group, codes, scales);
  return moe::check_launch("act_quant_nvfp4");
}

extern "C" moe_status act_quant_fp8(const void* x, moe_dtype xdt, int rows, int cols,
                                    uint8_t* codes, float* scales, hipStream_t s) {
  moe::clear_error();
  moe_status st = check_quant_args("act_quant_fp8", x, xdt, rows, cols);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(codes && scales, MOE_E_ARG, "act_quant_fp8: null pointer argument");
  MOE_REQUIRE(moe::aligned(codes, 16) && moe::aligned(scales, 4), MOE_E_ALIGN,
              "act_quant_fp8: misaligned pointer");
  const int64_t n = (int64_t)rows * (cols / 16);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (xdt == MOE_DT_F32)
    hipLaunchKernelGGL(moe::k_quant_fp8<true>, dim3(grid), dim3(256), 0, s, x, rows, cols, codes,
                       scales);
  else
    hipLaunchKernelGGL(moe::k_quant_fp8<false>, dim3(grid), dim3(256), 0, s, x, rows, cols, codes,
                       scales);
  return moe::check_launch("act_quant_fp8");
}

extern "C" moe_status nvfp4_global_scale(const float* x, int n_mat, int64_t mat_elems,
                                         float* global, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(x && global, MOE_E_ARG, "nvfp4_global_scale: null pointer argument");
  MOE_REQUIRE(n_mat >= 1 && mat_elems >= 4 && mat_elems % 4 == 0, MOE_E_SHAPE,
              "nvfp4_global_scale: bad shape n_mat=%d mat_elems=%lld", n_mat, (long long)mat_elems);
  MOE_REQUIRE(moe::aligned(x, 16) && moe::aligned(global, 4), MOE_E_ALIGN,
              "nvfp4_global_scale: misaligned pointer");
  hipLaunchKernelGGL(moe::k_global_scale, dim3(n_mat), dim3(1024), 0, s, x, mat_elems, global);
  return moe::check_launch("nvfp4_global_scale");
}

// ------------------------------------------------------------------ q4_g64_fp16
// One thread per group of 64 values (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for
// Infernix (bit-exact)", section "Drafting only": 4-bit codes, one FP16 scale
// per 64, scales chosen by squared error from the exact values).  The nine
// candidate scales d = fp16(amax / m), m = 7, 7.125, ..., 8, are each scored
// by the sum of (v - d q)^2 in double, in index order, every operation rounded
// once (no contraction), and the first least-error candidate is kept: the
// choice is a deterministic function of the 64 fp32 values.
namespace moe {

__global__ void __launch_bounds__(256) k_q4g64_quantize(const float* __restrict__ x, int64_t n_groups,
                                                        uint8_t* __restrict__ codes, uint16_t* __restrict__ scales) {
#pragma clang fp contract(off)   // every product and sum below is rounded on its own, as defined
  const int64_t gi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gi >= n_groups) return;
  const uint4* src = reinterpret_cast<const uint4*>(x + gi * 64);
  float v[64];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const uint4 u = src[q];
    v[4 * q + 0] = __uint_as_float(u.x);
    v[4 * q + 1] = __uint_as_float(u.y);
    v[4 * q + 2] = __uint_as_float(u.z);
    v[4 * q + 3] = __uint_as_float(u.w);
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 64; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
  double best = __builtin_inf();
  uint32_t best_d = 0u;
  float best_df = 0.0f;
  for (int j = 0; j <= 8; ++j) {
    const float m = 7.0f + 0.125f * (float)j;
    const _Float16 dh = (_Float16)__fdiv_rn(amax, m);   // nearest even
    const float df = (float)dh;
    if (!(df > 0.0f) || __builtin_isinf(df)) continue;
    const double dd = (double)df;
    double err = 0.0;
    for (int i = 0; i < 64; ++i) {
      const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fdiv_rn(v[i], df)), -8.0f), 7.0f);
      const double e = __dsub_rn((double)v[i], __dmul_rn(dd, (double)q));
      err = __dadd_rn(err, __dmul_rn(e, e));
    }
    if (err < best) {
      best = err;
      best_d = (uint32_t)__builtin_bit_cast(uint16_t, dh);
      best_df = df;
    }
  }
  uint32_t w[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
  if (best_df > 0.0f) {
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      const float q = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(__fdiv_rn(v[i], best_df)), -8.0f), 7.0f);
      w[i / 8] |= ((uint32_t)(int)q & 15u) << (4 * (i % 8));
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes + gi * 32);
  dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
  dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  scales[gi] = (uint16_t)best_d;
}

}  // namespace moe

extern "C" moe_status q4g64_quantize(const float* x, int rows, int cols, uint8_t* codes, uint16_t* scales,
                                     hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(x && codes && scales, MOE_E_ARG, "q4g64_quantize: null pointer argument");
  MOE_REQUIRE(rows >= 1 && cols >= 64 && cols % 64 == 0, MOE_E_SHAPE, "q4g64_quantize: bad shape %d x %d", rows,
              cols);
  MOE_REQUIRE(moe::aligned(x, 16) && moe::aligned(codes, 16) && moe::aligned(scales, 2), MOE_E_ALIGN,
              "q4g64_quantize: misaligned pointer");
  const int64_t n = (int64_t)rows * (cols / 64);
  hipLaunchKernelGGL(moe::k_q4g64_quantize, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n, codes,
                     scales);
  return moe::check_launch("q4g64_quantize");
}
