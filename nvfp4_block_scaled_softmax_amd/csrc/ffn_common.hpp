// Shared pieces of the expert FFN kernels: argument block, workspace layout,
// and the per-chunk dot products of the narrow (few-column) path.
#pragma once
#include "abi_common.hpp"
#include "device_common.hpp"

namespace moe {

struct FfnArgs {
  const uint8_t* gu_codes;
  const uint8_t* gu_scales;
  const uint8_t* dn_codes;
  const uint8_t* dn_scales;
  const float* gu_wscale;
  const float* dn_wscale;
  const float* gu_inscale;
  const float* dn_inscale;
  int E, H, I, T, k;
  const int32_t* offsets;
  const int32_t* sorted_pairs;
  const uint16_t* x;
  const uint8_t* xq_codes;   // A8: [T][H] E4M3; A4: [P][2][H/2] (gate, up)
  const void* xq_scales;     // A8: fp32 [T][H/16]; A4: E4M3 [P][2][H/16]
  uint8_t* h_codes;          // A16: bf16 [P][I]; A8: E4M3 [P][I]; A4: [P][I/2]
  void* h_scales;            // A8: fp32 [P][I/16]; A4: E4M3 [P][I/16]
  float* y;                  // [P][H]
  int tiled;                 // weight scales in the tiled layout (moe_layout)
};

struct FfnLayout {
  size_t xq_codes, xq_scales, h_codes, h_scales, plan, total;
};

inline FfnLayout ffn_layout(moe_act_mode mode, int T, int k, int H, int I) {
  const size_t P = (size_t)T * k;
  FfnLayout L{0, 0, 0, 0, 0, 0};
  size_t o = 0;
  auto seg = [&](size_t bytes) { const size_t at = o; o = round_up(o + bytes, 256); return at; };
  if (mode == MOE_A16 || (int)mode == kModeQ4) {
    L.h_codes = seg(P * I * 2);
    if (mode == MOE_A16 && T > 8) L.plan = seg(((P < (size_t)kMaxExperts ? P : (size_t)kMaxExperts) + P / 32) * 16);
  } else if (mode == MOE_A8) {
    L.xq_codes = seg((size_t)T * H);
    L.xq_scales = seg((size_t)T * (H / 16) * 4);
    L.h_codes = seg(P * I);
    L.h_scales = seg(P * (I / 16) * 4);
    if (T > 8) L.plan = seg(((P < (size_t)kMaxExperts ? P : (size_t)kMaxExperts) + P / 32) * 16);
  } else {
    L.xq_codes = seg(P * 2 * (H / 2));
    L.xq_scales = seg(P * 2 * (H / 16));
    L.h_codes = seg(P * (I / 2));
    L.h_scales = seg(P * (I / 16));
    L.plan = seg(((P < (size_t)kMaxExperts ? P : (size_t)kMaxExperts) + P / 32) * 16);
  }
  L.total = o;
  return L;
}
// (kModeQ4 lays out as MOE_A16: the fp16 intermediate [P][I].)

// ---------------------------------------------------------------------------
// Narrow-path LDS chunk layout: one "chunk" = 32 consecutive K values of one
// column, padded so that 16 lanes reading consecutive chunks with 128-bit LDS
// loads hit distinct banks (strides of 80 and 48 bytes).
//   A16 : [64 B bf16 x]                                     stride 80
//   A8  : [32 B E4M3 codes][8 B fp32 scales s0 s1]            stride 48
//   A4  : [16 B codes m0][16 B codes m1][s0 s1 of m0][s0 s1 of m1]  stride 48
//         (gate/up: m0 gate, m1 up; down: only m0)
template <int MODE>
struct ChunkLds;
template <>
struct ChunkLds<MOE_A16> { static constexpr int kStride = 80; };
template <>
struct ChunkLds<MOE_A8> { static constexpr int kStride = 48; };
template <>
struct ChunkLds<MOE_A4> { static constexpr int kStride = 48; };
// q4_g64_fp16 experts: [64 B fp16 x, paired by nibble (pair_by_nibble)] stride 80
template <>
struct ChunkLds<kModeQ4> { static constexpr int kStride = 80; };

// Pair position of chunk c's two E4M3 scales in a tiled scale row of nc
// chunks: in a full window of 32 chunks, chunk 4i + g (step i, piece g) sits
// at 8g + i; a trailing partial window keeps the canonical order.
__host__ __device__ __forceinline__ int tiled_pair(int c, int nc) {
  const int p = c >> 5, cw = c & 31;
  return (p + 1) * 32 <= nc ? (p << 5) | ((cw & 3) << 3) | (cw >> 2) : c;
}

// Bytes of one row's scales per 32-value chunk, and the scale of chunk c within
// a row's scale bytes: NVFP4 two E4M3 per chunk (tiled_nc: the row's chunk
// count when the scales are in the tiled layout, else 0); q4_g64_fp16 one fp16
// per two chunks.
template <int MODE>
__device__ __forceinline__ uint32_t chunk_scale(const uint8_t* srow, int c, int tiled_nc = 0) {
  if constexpr (MODE == kModeQ4) return ld_stream16(srow + 2 * (c >> 1));
  else return ld_stream16(srow + 2 * (tiled_nc ? tiled_pair(c, tiled_nc) : c));
}
template <int MODE>
__host__ __device__ constexpr int scale_row_bytes(int K) { return MODE == kModeQ4 ? K / 32 : K / 16; }

// Dot product of one 16-byte weight chunk (32 E2M1 codes, block scales in the
// two bytes of wsc) with the activation chunk at `c` (LDS), matrix m (A4).
// Returns sum_blocks (block dot) * scale product; the per-matrix factors are
// applied by the caller.
template <int MODE>
__device__ __forceinline__ float chunk_dot(const uint4 w, uint32_t wsc, const uint8_t* c, int m);

template <>
__device__ __forceinline__ float chunk_dot<MOE_A16>(const uint4 w, uint32_t wsc, const uint8_t* c,
                                                    int) {
  const uint4* xc = reinterpret_cast<const uint4*>(c);
  const uint4 x0 = xc[0], x1 = xc[1], x2 = xc[2], x3 = xc[3];
  float b0 = 0.0f, b1 = 0.0f;
#define DOT8(ACC, WW, XX)                                                                        \
  ACC = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<0>(WW), bitcast<bf16x2>(XX.x), ACC, false); \
  ACC = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<1>(WW), bitcast<bf16x2>(XX.y), ACC, false); \
  ACC = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<2>(WW), bitcast<bf16x2>(XX.z), ACC, false); \
  ACC = __builtin_amdgcn_fdot2_f32_bf16(e2m1x2_to_bf16<3>(WW), bitcast<bf16x2>(XX.w), ACC, false);
  DOT8(b0, w.x, x0)
  DOT8(b0, w.y, x1)
  DOT8(b1, w.z, x2)
  DOT8(b1, w.w, x3)
#undef DOT8
  return b0 * e4m3_to_f32(wsc & 0xFFu) + b1 * e4m3_to_f32((wsc >> 8) & 0xFFu);
}

template <>
__device__ __forceinline__ float chunk_dot<MOE_A8>(const uint4 w, uint32_t wsc, const uint8_t* c,
                                                   int) {
  const uint4* xc = reinterpret_cast<const uint4*>(c);
  const uint4 xa = xc[0], xb = xc[1];
  const float2 sx = *reinterpret_cast<const float2*>(c + 32);
  float b0 = 0.0f, b1 = 0.0f;
  // weight dword q holds elements 8q..8q+7; x dword d holds elements 4d..4d+3
#define DOT4(ACC, WW, SELA, SELB, XD)                                                              \
  ACC = __builtin_amdgcn_fdot2(e2m1x2_to_f16<SELA>(WW), e4m3x2_to_f16<false>(XD), ACC, false);     \
  ACC = __builtin_amdgcn_fdot2(e2m1x2_to_f16<SELB>(WW), e4m3x2_to_f16<true>(XD), ACC, false);
  DOT4(b0, w.x, 0, 1, xa.x)
  DOT4(b0, w.x, 2, 3, xa.y)
  DOT4(b0, w.y, 0, 1, xa.z)
  DOT4(b0, w.y, 2, 3, xa.w)
  DOT4(b1, w.z, 0, 1, xb.x)
  DOT4(b1, w.z, 2, 3, xb.y)
  DOT4(b1, w.w, 0, 1, xb.z)
  DOT4(b1, w.w, 2, 3, xb.w)
#undef DOT4
  return b0 * (e4m3_to_f32(wsc & 0xFFu) * sx.x) + b1 * (e4m3_to_f32((wsc >> 8) & 0xFFu) * sx.y);
}

template <>
__device__ __forceinline__ float chunk_dot<MOE_A4>(const uint4 w, uint32_t wsc, const uint8_t* c,
                                                   int m) {
  const uint4 xq = *reinterpret_cast<const uint4*>(c + 16 * m);
  const uint32_t xs = *reinterpret_cast<const uint16_t*>(c + 32 + 2 * m);
  // products of E2M1 values are multiples of 1/4 and each block sum is at most
  // 16 * 36 in magnitude: every partial sum below is exact in fp32.
  float b0 = 0.0f, b1 = 0.0f;
#define DOT8(ACC, WW, XX)                                                                   \
  ACC = __builtin_amdgcn_fdot2(e2m1x2_to_f16<0>(WW), e2m1x2_to_f16<0>(XX), ACC, false);     \
  ACC = __builtin_amdgcn_fdot2(e2m1x2_to_f16<1>(WW), e2m1x2_to_f16<1>(XX), ACC, false);     \
  ACC = __builtin_amdgcn_fdot2(e2m1x2_to_f16<2>(WW), e2m1x2_to_f16<2>(XX), ACC, false);     \
  ACC = __builtin_amdgcn_fdot2(e2m1x2_to_f16<3>(WW), e2m1x2_to_f16<3>(XX), ACC, false);
  DOT8(b0, w.x, xq.x)
  DOT8(b0, w.y, xq.y)
  DOT8(b1, w.z, xq.z)
  DOT8(b1, w.w, xq.w)
#undef DOT8
  const float s0 = e4m3_to_f32(wsc & 0xFFu) * e4m3_to_f32(xs & 0xFFu);      // exact
  const float s1 = e4m3_to_f32((wsc >> 8) & 0xFFu) * e4m3_to_f32(xs >> 8);  // exact
  return b0 * s0 + b1 * s1;
}

template <>
__device__ __forceinline__ float chunk_dot<kModeQ4>(const uint4 w, uint32_t wsc, const uint8_t* c, int) {
  // q4_g64_fp16: 32 int4 codes (one fp16 scale: a chunk is half a group of 64)
  // against 32 fp16 x; products of integers -8..7 and fp16 values are exact.
  const uint4* xc = reinterpret_cast<const uint4*>(c);
  const uint32_t wd[4] = {w.x ^ 0x88888888u, w.y ^ 0x88888888u, w.z ^ 0x88888888u, w.w ^ 0x88888888u};
  float acc = 0.0f;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint4 xv = xc[d];
    acc = __builtin_amdgcn_fdot2(q4_expand_pair<0>(wd[d]), bitcast<f16x2>(xv.x), acc, false);
    acc = __builtin_amdgcn_fdot2(q4_expand_pair<1>(wd[d]), bitcast<f16x2>(xv.y), acc, false);
    acc = __builtin_amdgcn_fdot2(q4_expand_pair<2>(wd[d]), bitcast<f16x2>(xv.z), acc, false);
    acc = __builtin_amdgcn_fdot2(q4_expand_pair<3>(wd[d]), bitcast<f16x2>(xv.w), acc, false);
  }
  return acc * (float)bitcast<_Float16>((uint16_t)(wsc & 0xFFFFu));
}

// Binary search: the expert whose segment [offsets[e], offsets[e+1]) holds row r.
__device__ __forceinline__ int expert_of_row(const int32_t* offsets, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

moe_status launch_ffn_narrow(const FfnArgs& a, moe_act_mode mode, int slots, int stage_mask,
                             hipStream_t s);
// The argument block of an nvfp4_expert_ffn call (workspace pointers included).
FfnArgs make_ffn_args(const moe_nvfp4_experts& w, moe_act_mode mode, const uint16_t* x, int T,
                      int k, const int32_t* offsets, const int32_t* sorted_pairs, float* y_pairs,
                      void* ws);
// The wide (MFMA) path of calls above kNarrowMaxT tokens, for each activation mode.
moe_status launch_ffn_wide(const FfnArgs& a, moe_act_mode mode, int stage_mask, void* plan_ws, hipStream_t s);
// Entries of the wide path's work plan for P sorted rows of E experts.
int wide_plan_entries(int P, int E);
// The product cores alone (moe_debug_nvfp4_matmul), on an argument block whose
// expert 0 down matrix is the N x K operand (H = N, I = K) and whose
// intermediate slots (h_codes, h_scales) hold the T columns.
moe_status launch_debug_narrow(const FfnArgs& a, moe_act_mode mode, hipStream_t s);
moe_status launch_debug_wide(const FfnArgs& a, moe_act_mode mode, void* plan_ws, hipStream_t s);
size_t debug_wide_plan_bytes(int cols);

// Calls with more than this many tokens take the MFMA path (4-bit mode).
constexpr int kNarrowMaxT = 8;

}  // namespace moe
