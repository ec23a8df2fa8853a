// nvfp4_expert_ffn: activation quantization for the 8/4-bit modes, then the
// gate/up + SwiGLU and down kernels: the narrow path for calls of up to 8
// tokens, the MFMA grouped GEMM for wider 4-bit calls.
#include "ffn_common.hpp"

namespace moe {

// 4-bit mode: x of every sorted row, quantized under its expert's gate and up
// input scales.  One thread per (row, matrix, 16-block).
__global__ void __launch_bounds__(256) k_quant_x_a4_rows(FfnArgs a) {
  const int nb = a.H / 16;
  const int64_t P = (int64_t)a.T * a.k;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= P * 2 * nb) return;
  const int r = (int)(i / (2 * nb));
  const int m = (int)((i / nb) % 2);
  const int b = (int)(i % nb);
  if (r >= a.offsets[a.E]) return;
  const int e = expert_of_row(a.offsets, a.E, r);
  const int t = a.sorted_pairs[r] / a.k;
  const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H + (size_t)b * 16);
  float v[16];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const uint4 u = src[q];
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * q + 2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      v[8 * q + 2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
  }
  uint32_t lo, hi;
  const uint32_t s = nvfp4_quant16(v, a.gu_inscale[2 * e + m], lo, hi);
  const size_t row = (size_t)r * 2 + m;
  *reinterpret_cast<uint2*>(const_cast<uint8_t*>(a.xq_codes) + row * (a.H / 2) + (size_t)b * 8) =
      make_uint2(lo, hi);
  static_cast<uint8_t*>(const_cast<void*>(a.xq_scales))[row * nb + b] = (uint8_t)s;
}

// 4-bit mode inside the whole layer, where the permutation's pair rows and the
// top-k ids are at hand: one workgroup per token, one thread per 16-block of H.
// The token's x block is quantized under the gate and up input scales of each
// of its pairs' experts and stored to that pair's sorted row (pairs with
// pair_row < 0 are skipped); a scale equal (bitwise) to the one just used
// reuses its codes, so a token whose pairs share their input scales is
// quantized once.  The codes are the same function of (x block, scale) as in
// k_quant_x_a4_rows.
__global__ void __launch_bounds__(256) k_quant_x_a4_tokens(FfnArgs a, const int32_t* __restrict__ pair_row,
                                                           const int32_t* __restrict__ ids) {
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_g[kMaxTopK][2];
  const int t = blockIdx.x, k = a.k, nb = a.H / 16;
  const uint4* xrow = reinterpret_cast<const uint4*>(a.x + (size_t)t * a.H);
  const int b0 = threadIdx.x;
  uint4 u0 = make_uint4(0u, 0u, 0u, 0u), u1 = u0;
  if (b0 < nb) {   // this thread's first block is on its way while the pairs are staged
    u0 = xrow[2 * b0];
    u1 = xrow[2 * b0 + 1];
  }
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const size_t p = (size_t)t * k + j;
    const int r = pair_row[p], e = ids[p];
    const bool ok = r >= 0 && e >= 0 && e < a.E;
    s_row[j] = ok ? r : -1;
    s_g[j][0] = ok ? a.gu_inscale[2 * e] : 0.0f;
    s_g[j][1] = ok ? a.gu_inscale[2 * e + 1] : 0.0f;
  }
  __syncthreads();
  for (int b = b0; b < nb; b += blockDim.x) {
    if (b != b0) {
      u0 = xrow[2 * b];
      u1 = xrow[2 * b + 1];
    }
    float v[16];
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
    uint32_t last_g = 0u, lo = 0u, hi = 0u, sc = 0u;
    bool have = false;
    for (int j = 0; j < k; ++j) {
      const int r = s_row[j];
      if (r < 0) continue;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float g = s_g[j][m];
        if (!have || __float_as_uint(g) != last_g) {
          sc = nvfp4_quant16(v, g, lo, hi);
          last_g = __float_as_uint(g);
          have = true;
        }
        const size_t row = (size_t)r * 2 + m;
        *reinterpret_cast<uint2*>(const_cast<uint8_t*>(a.xq_codes) + row * (a.H / 2) + (size_t)b * 8) =
            make_uint2(lo, hi);
        static_cast<uint8_t*>(const_cast<void*>(a.xq_scales))[row * nb + b] = (uint8_t)sc;
      }
    }
  }
}

size_t expert_ffn_workspace(moe_act_mode mode, int T, int k, int H, int I) {
  return ffn_layout(mode, T, k, H, I).total;
}

FfnArgs make_ffn_args(const moe_nvfp4_experts& w, moe_act_mode mode, const uint16_t* x, int T,
                      int k, const int32_t* offsets, const int32_t* sorted_pairs, float* y_pairs,
                      void* ws) {
  const FfnLayout L = ffn_layout(mode, T, k, w.H, w.I);
  uint8_t* base = static_cast<uint8_t*>(ws);
  FfnArgs a;
  a.gu_codes = w.gu_codes;
  a.gu_scales = w.gu_scales;
  a.dn_codes = w.dn_codes;
  a.dn_scales = w.dn_scales;
  a.gu_wscale = w.gu_wscale;
  a.dn_wscale = w.dn_wscale;
  a.gu_inscale = w.gu_inscale;
  a.dn_inscale = w.dn_inscale;
  a.E = w.E;
  a.H = w.H;
  a.I = w.I;
  a.T = T;
  a.k = k;
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.x = x;
  const bool x16 = mode == MOE_A16 || (int)mode == kModeQ4;   // 16-bit activations, nothing quantized
  a.xq_codes = x16 ? nullptr : base + L.xq_codes;
  a.xq_scales = x16 ? nullptr : base + L.xq_scales;
  a.h_codes = base + L.h_codes;
  a.h_scales = x16 ? nullptr : base + L.h_scales;
  a.y = y_pairs;
  a.tiled = w.layout == MOE_LAYOUT_TILED ? 1 : 0;
  return a;
}

moe_status launch_expert_ffn(const moe_nvfp4_experts& w, moe_act_mode mode, const uint16_t* x,
                             int T, int k, const int32_t* offsets, const int32_t* sorted_pairs,
                             float* y_pairs, void* ws, int stage_mask, hipStream_t s,
                             const int32_t* pair_row, const int32_t* ids) {
  const FfnLayout L = ffn_layout(mode, T, k, w.H, w.I);
  uint8_t* base = static_cast<uint8_t*>(ws);
  const FfnArgs a = make_ffn_args(w, mode, x, T, k, offsets, sorted_pairs, y_pairs, ws);
  const int P = T * k;
  const int slots = P < w.E ? P : w.E;

  if (mode == MOE_A8 && (stage_mask & 1)) {
    moe_status st = act_quant_fp8(x, MOE_DT_BF16, T, w.H, base + L.xq_codes,
                                  reinterpret_cast<float*>(base + L.xq_scales), s);
    if (st != MOE_OK) return st;
  } else if (mode == MOE_A4 && (stage_mask & 1)) {
    if (pair_row && ids) {
      const int nb = w.H / 16;
      hipLaunchKernelGGL(k_quant_x_a4_tokens, dim3(T), dim3(nb < 256 ? (nb + 63) / 64 * 64 : 256), 0, s, a,
                         pair_row, ids);
    } else {
      const int64_t n = (int64_t)P * 2 * (w.H / 16);
      hipLaunchKernelGGL(k_quant_x_a4_rows, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    }
    moe_status st = check_launch("nvfp4_expert_ffn (x quantization)");
    if (st != MOE_OK) return st;
  }
  if ((int)mode != kModeQ4 && T > kNarrowMaxT && w.H % 128 == 0 && w.I % 128 == 0)
    return launch_ffn_wide(a, mode, stage_mask, base + L.plan, s);
  return launch_ffn_narrow(a, mode, slots, stage_mask, s);
}

}  // namespace moe

extern "C" size_t nvfp4_expert_ffn_workspace_bytes(moe_act_mode mode, int T, int k, int H, int I) {
  if (T < 1 || k < 1 || H < 32 || I < 32) return 0;
  if (mode != MOE_A16 && mode != MOE_A8 && mode != MOE_A4) return 0;
  return moe::expert_ffn_workspace(mode, T, k, H, I);
}

namespace moe {
moe_status check_experts(const char* name, const moe_nvfp4_experts* w, moe_act_mode mode) {
  MOE_REQUIRE(w, MOE_E_ARG, "%s: null expert set", name);
  MOE_REQUIRE(mode == MOE_A16 || mode == MOE_A8 || mode == MOE_A4, MOE_E_ARG, "%s: bad mode %d",
              name, (int)mode);
  MOE_REQUIRE(w->fmt == MOE_FMT_NVFP4 || w->fmt == MOE_FMT_Q4G64, MOE_E_ARG, "%s: bad weight format %d", name,
              (int)w->fmt);
  MOE_REQUIRE(w->layout == MOE_LAYOUT_CANONICAL || w->layout == MOE_LAYOUT_TILED, MOE_E_ARG, "%s: bad layout %d",
              name, (int)w->layout);
  MOE_REQUIRE(w->layout == MOE_LAYOUT_CANONICAL || (w->fmt == MOE_FMT_NVFP4 && w->H % 128 == 0 && w->I % 128 == 0),
              MOE_E_SHAPE, "%s: the tiled layout is for NVFP4 experts with H and I multiples of 128 (H=%d I=%d)",
              name, w->H, w->I);
  if (w->fmt == MOE_FMT_Q4G64) {
    MOE_REQUIRE(mode == MOE_A16, MOE_E_UNSUPPORTED, "%s: q4_g64_fp16 experts take 16-bit activations only", name);
    MOE_REQUIRE(w->gu_codes && w->gu_scales && w->dn_codes && w->dn_scales, MOE_E_ARG, "%s: null expert array",
                name);
    MOE_REQUIRE(w->E >= 1 && w->E <= kMaxExperts && dim_ok(w->H) && dim_ok(w->I) && w->H % 64 == 0 &&
                    w->I % 64 == 0,
                MOE_E_SHAPE, "%s: bad q4_g64_fp16 expert shape E=%d H=%d I=%d", name, w->E, w->H, w->I);
    MOE_REQUIRE(aligned(w->gu_codes, 16) && aligned(w->gu_scales, 16) && aligned(w->dn_codes, 16) &&
                    aligned(w->dn_scales, 16),
                MOE_E_ALIGN, "%s: misaligned expert array", name);
    return MOE_OK;
  }
  MOE_REQUIRE(w->gu_codes && w->gu_scales && w->dn_codes && w->dn_scales && w->gu_wscale &&
                  w->dn_wscale,
              MOE_E_ARG, "%s: null expert array", name);
  MOE_REQUIRE(mode != MOE_A4 || (w->gu_inscale && w->dn_inscale), MOE_E_ARG,
              "%s: 4-bit mode needs gu_inscale and dn_inscale", name);
  MOE_REQUIRE(w->E >= 1 && w->E <= kMaxExperts && dim_ok(w->H) && dim_ok(w->I), MOE_E_SHAPE,
              "%s: bad expert shape E=%d H=%d I=%d", name, w->E, w->H, w->I);
  MOE_REQUIRE(aligned(w->gu_codes, 16) && aligned(w->gu_scales, 16) && aligned(w->dn_codes, 16) &&
                  aligned(w->dn_scales, 16) && aligned(w->gu_wscale, 4) && aligned(w->dn_wscale, 4) &&
                  (!w->gu_inscale || aligned(w->gu_inscale, 4)) &&
                  (!w->dn_inscale || aligned(w->dn_inscale, 4)),
              MOE_E_ALIGN, "%s: misaligned expert array", name);
  return MOE_OK;
}
}  // namespace moe

static moe_status ffn_entry(const char* name, const moe_nvfp4_experts* w, moe_act_mode mode,
                            int stage_mask, const uint16_t* x, int T, int k,
                            const int32_t* expert_offsets, const int32_t* sorted_pairs,
                            float* y_pairs, void* ws, size_t ws_bytes, hipStream_t s) {
  moe::clear_error();
  moe_status st = moe::check_experts(name, w, mode);
  if (st != MOE_OK) return st;
  MOE_REQUIRE(x && expert_offsets && sorted_pairs && y_pairs && ws, MOE_E_ARG,
              "%s: null pointer argument", name);
  MOE_REQUIRE(T >= 1 && k >= 1 && k <= w->E && (int64_t)T * k <= (1 << 24), MOE_E_SHAPE,
              "%s: bad shape T=%d k=%d", name, T, k);
  MOE_REQUIRE(moe::aligned(x, 16) && moe::aligned(ws, 16) && moe::aligned(y_pairs, 16) &&
                  moe::aligned(expert_offsets, 4) && moe::aligned(sorted_pairs, 4),
              MOE_E_ALIGN, "%s: misaligned pointer", name);
  const size_t need = moe::expert_ffn_workspace(moe::kernel_mode(*w, mode), T, k, w->H, w->I);
  MOE_REQUIRE(ws_bytes >= need, MOE_E_WORKSPACE, "%s: workspace %zu < %zu bytes", name, ws_bytes,
              need);
  return moe::launch_expert_ffn(*w, moe::kernel_mode(*w, mode), x, T, k, expert_offsets, sorted_pairs, y_pairs,
                                ws, stage_mask, s);
}

extern "C" moe_status nvfp4_expert_ffn(const moe_nvfp4_experts* w, moe_act_mode mode,
                                       const uint16_t* x, int T, int k,
                                       const int32_t* expert_offsets, const int32_t* sorted_pairs,
                                       float* y_pairs, void* ws, size_t ws_bytes, hipStream_t s) {
  return ffn_entry("nvfp4_expert_ffn", w, mode, 7, x, T, k, expert_offsets, sorted_pairs, y_pairs,
                   ws, ws_bytes, s);
}

extern "C" moe_status nvfp4_expert_ffn_stage(const moe_nvfp4_experts* w, moe_act_mode mode,
                                             int stage, const uint16_t* x, int T, int k,
                                             const int32_t* expert_offsets,
                                             const int32_t* sorted_pairs, float* y_pairs, void* ws,
                                             size_t ws_bytes, hipStream_t s) {
  if (stage < 0 || stage > 2) {
    moe::set_error("nvfp4_expert_ffn_stage: stage %d not in 0..2", stage);
    return MOE_E_ARG;
  }
  return ffn_entry("nvfp4_expert_ffn_stage", w, mode, 1 << stage, x, T, k, expert_offsets,
                   sorted_pairs, y_pairs, ws, ws_bytes, s);
}

// ------------------------------------------------------------------ debug core
extern "C" size_t moe_debug_nvfp4_matmul_workspace_bytes(int core, int cols) {
  if (cols < 1 || (core != 0 && core != 1)) return 0;
  return core == 1 ? moe::debug_wide_plan_bytes(cols) : 0;
}

extern "C" moe_status moe_debug_nvfp4_matmul(int core, moe_act_mode mode, const uint8_t* codes,
                                             const uint8_t* scales, const float* wscale, int N, int K,
                                             const void* x, const void* x_scales, const float* inscale,
                                             int cols, float* out, void* ws, size_t ws_bytes,
                                             hipStream_t s) {
  const char* name = "moe_debug_nvfp4_matmul";
  moe::clear_error();
  MOE_REQUIRE(core == 0 || core == 1, MOE_E_ARG, "%s: core %d is not 0 (narrow) or 1 (wide)", name, core);
  MOE_REQUIRE(mode == MOE_A16 || mode == MOE_A8 || mode == MOE_A4, MOE_E_ARG, "%s: bad mode %d", name,
              (int)mode);
  MOE_REQUIRE(codes && scales && wscale && x && out, MOE_E_ARG, "%s: null pointer argument", name);
  MOE_REQUIRE(mode == MOE_A16 || x_scales, MOE_E_ARG, "%s: 8/4-bit x needs x_scales", name);
  MOE_REQUIRE(mode != MOE_A4 || inscale, MOE_E_ARG, "%s: 4-bit x needs inscale", name);
  MOE_REQUIRE(N >= 1 && N <= (1 << 20) && moe::dim_ok(K) && cols >= 1 && cols <= (1 << 16), MOE_E_SHAPE,
              "%s: bad shape N=%d K=%d cols=%d", name, N, K, cols);
  MOE_REQUIRE(moe::aligned(codes, 16) && moe::aligned(scales, 16) && moe::aligned(x, 16) &&
                  moe::aligned(out, 16) && moe::aligned(wscale, 4) && (!inscale || moe::aligned(inscale, 4)) &&
                  (!x_scales || moe::aligned(x_scales, 16)),
              MOE_E_ALIGN, "%s: misaligned pointer", name);
  if (core == 1) {
    MOE_REQUIRE(N % 16 == 0 && K % 128 == 0, MOE_E_SHAPE, "%s: the wide core needs N %% 16 == 0, K %% 128 == 0",
                name);
    MOE_REQUIRE(ws && moe::aligned(ws, 16) && ws_bytes >= moe::debug_wide_plan_bytes(cols), MOE_E_WORKSPACE,
                "%s: workspace %zu < %zu bytes", name, ws_bytes, moe::debug_wide_plan_bytes(cols));
  }
  moe::FfnArgs a{};
  a.dn_codes = codes;
  a.dn_scales = scales;
  a.dn_wscale = wscale;
  a.dn_inscale = inscale;
  a.E = 1;
  a.H = N;
  a.I = K;
  a.T = cols;
  a.k = 1;
  a.h_codes = const_cast<uint8_t*>(static_cast<const uint8_t*>(x));
  a.h_scales = const_cast<void*>(x_scales);
  a.y = out;
  return core == 1 ? moe::launch_debug_wide(a, mode, ws, s) : moe::launch_debug_narrow(a, mode, s);
}

extern "C" moe_status moe_debug_q4g64_matmul(const uint8_t* codes, const uint16_t* scales, int N, int K,
                                             const uint16_t* x, int cols, float* out, hipStream_t s) {
  const char* name = "moe_debug_q4g64_matmul";
  moe::clear_error();
  MOE_REQUIRE(codes && scales && x && out, MOE_E_ARG, "%s: null pointer argument", name);
  MOE_REQUIRE(N >= 1 && N <= (1 << 20) && moe::dim_ok(K) && K % 64 == 0 && cols >= 1 && cols <= (1 << 16),
              MOE_E_SHAPE, "%s: bad shape N=%d K=%d cols=%d", name, N, K, cols);
  MOE_REQUIRE(moe::aligned(codes, 16) && moe::aligned(scales, 16) && moe::aligned(x, 16) && moe::aligned(out, 16),
              MOE_E_ALIGN, "%s: misaligned pointer", name);
  moe::FfnArgs a{};
  a.dn_codes = codes;
  a.dn_scales = reinterpret_cast<const uint8_t*>(scales);
  a.E = 1;
  a.H = N;
  a.I = K;
  a.T = cols;
  a.k = 1;
  a.h_codes = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(x));
  a.y = out;
  return moe::launch_debug_narrow(a, (moe_act_mode)moe::kModeQ4, s);
}
