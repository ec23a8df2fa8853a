// The shared expert's tiles as device functions, shared by its stand-alone
// kernels (shared.hip) and the fused decode kernel (decode.hip).
//
// The shared expert (page "Qwen3.8-Flash-Next NVIDIA NVFP4 for Infernix
// (bit-exact)", section "What is bit-exact and what is quantized": shared
// experts and gates are BF16 dense projections) is one SwiGLU expert that
// every token runs, with BF16 matrices, scaled per token by sigmoid(x . gate).
// Its tiles are bandwidth-bound GEMVs like the routed experts' narrow tiles,
// but on bf16 weights: 16-byte loads of 8 weights meet bf16 activations from
// LDS in v_dot2_f32_bf16 (products exact in fp32, fp32 sums).
//
//   gate/up tile: 4 h rows, one per wave; lanes 0-31 read the gate row, lanes
//                 32-63 the matching up row, each lane CPL 16-byte chunks of it
//                 (chunk kl + 32 j), all issued before any use.
//   down tile:    64 output rows, 16 per wave; 16 lanes per row, 4 rows per
//                 lane group, CPL chunks per lane; each tile also computes the
//                 gate's sigmoid for its tokens.
// Tokens are taken in groups of kShTok with the weights held in registers.
#pragma once
#include "ffn_narrow.hpp"

namespace moe {

constexpr int kShGuRows = 4;                  // h rows per gate/up tile (one per wave)
constexpr int kShDnRows = 64;                 // output rows per down tile
constexpr int kShTok = 8;                     // tokens per pass
constexpr int kShMaxIs = 1024;                // the down tile holds Is/8/16 chunks per lane in registers

struct SharedArgs {
  const uint16_t* gu;     // [2Is][H] bf16: gate rows, then up rows
  const uint16_t* dn;     // [H][Is] bf16
  const uint16_t* gate;   // [H] bf16
  const uint16_t* x;      // [T][H] bf16
  int H, Is, T;
  uint16_t* h;            // [T][Is] bf16: the intermediate
  float* y;               // [T][H] fp32: sigmoid(x . gate) * (h . Wd^T)
  int tg;                 // tokens per pass of the gate/up tile (<= kShTok; x of tg tokens fits its LDS)
};

// The argument block of a shared expert call (shared.hip).
SharedArgs make_shared_args(const moe_shared_expert& sw, const uint16_t* x, int T, void* h_ws, float* y);

// Tokens per gate/up pass: x of that many tokens (H bf16 each) in kShLdsX bytes.
constexpr int kShLdsX = 48 * 1024;
__host__ __device__ constexpr int shared_tok_group(int H) { return kShLdsX / (2 * H) < kShTok ? kShLdsX / (2 * H) : kShTok; }

__device__ __forceinline__ float dot8_bf16(const uint4 w, const uint4 x, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.x), bitcast<bf16x2>(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.y), bitcast<bf16x2>(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.z), bitcast<bf16x2>(x.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.w), bitcast<bf16x2>(x.w), acc, false);
  return acc;
}

// Chunks per lane of the gate/up tile for a row of H bf16 (H / 8 chunks over 32 lanes).
__host__ __device__ constexpr int shared_gu_cpl(int H) { return (H / 8 + 31) / 32; }
// Chunks per lane of the down tile for a row of Is bf16 (Is / 8 chunks over 16 lanes).
__host__ __device__ constexpr int shared_dn_cpl(int Is) { return (Is / 8 + 15) / 16; }

// ------------------------------------------------------------------ gate/up
// Tile rb: h rows 4 rb .. 4 rb + 3 for every token.  h goes to a.h (bf16, with
// device-coherent stores when COH) and, with htag, also as epoch-tagged words
// htag[t * Is/2 + i/2] = (bf16 h_i | h_{i+1} << 16) << 32 | epoch.
template <int CPL, bool COH>
__device__ __forceinline__ void shared_gateup_tile(const SharedArgs& a, int rb, uint8_t* lds,
                                                   uint64_t* htag = nullptr, uint32_t epoch = 0u) {
  __shared__ uint16_t hb[kShTok][kShGuRows];
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int half = lane >> 5, kl = lane & 31;
  const int H = a.H, Is = a.Is, NCH = H / 8;
  const int i = rb * kShGuRows + wave;
  const uint4* row = reinterpret_cast<const uint4*>(a.gu + ((size_t)half * Is + i) * H);
  uint4 wv[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) wv[j] = row[min(kl + 32 * j, NCH - 1)];   // clamped: past NCH unused
  __builtin_amdgcn_sched_barrier(0);
  uint4* xs = reinterpret_cast<uint4*>(lds);
  for (int t0 = 0; t0 < a.T; t0 += a.tg) {
    const int nt = min(a.tg, a.T - t0);
    __syncthreads();   // the previous group's reads of xs are done
    batched_copy<kTileThreads, kStageBatch>(
        nt * NCH, [&](int q) { return reinterpret_cast<const uint4*>(a.x + (size_t)t0 * H)[q]; },
        [&](int q, uint4 v) { xs[q] = v; });
    __syncthreads();
    float acc[kShTok];
#pragma unroll
    for (int t = 0; t < kShTok; ++t) acc[t] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = kl + 32 * j;
      if (c < NCH) {
#pragma unroll
        for (int t = 0; t < kShTok; ++t)
          if (t < nt) acc[t] = dot8_bf16(wv[j], xs[t * NCH + c], acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < kShTok; ++t) {
      const float v = lane_group_sum<32>(acc[t]);   // lanes 0-31: gate sum, 32-63: up sum
      const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
      const float u = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
      if (lane == 0 && t < nt) hb[t][wave] = (uint16_t)f32_to_bf16(swiglu(g, u));
    }
    __syncthreads();
    // two h values per thread: rows 4 rb + 2 p, + 1 of token t0 + t
    if (threadIdx.x < nt * (kShGuRows / 2)) {
      const int t = threadIdx.x / (kShGuRows / 2), p = threadIdx.x % (kShGuRows / 2);
      const uint32_t w2 = (uint32_t)hb[t][2 * p] | ((uint32_t)hb[t][2 * p + 1] << 16);
      const size_t at = (size_t)(t0 + t) * Is + rb * kShGuRows + 2 * p;
      if (htag)
        __hip_atomic_store(&htag[at / 2], (uint64_t)w2 << 32 | epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      hst32<COH>(a.h, 2 * at, w2);
    }
  }
}

// ------------------------------------------------------------------ down
// Tile rb: output rows 64 rb .. 64 rb + 63.  The gate's sigmoid for each token
// is computed here, after the weight loads are out and before wait() (which
// returns once h may be read).  h comes from a.h (device-coherent loads when
// COH), or, with htag, from the tagged words, each polled until it carries
// epoch (a bounded wait on abort_word).  y goes to a.y and, with ytag, also as
// tagged words ytag[t * H + o] = (fp32 bits << 32) | epoch.
template <int CPL, bool COH, typename Wait>
__device__ __forceinline__ void shared_down_tile(const SharedArgs& a, int rb, uint8_t* lds, Wait&& wait,
                                                 const uint64_t* htag = nullptr, uint32_t epoch = 0u,
                                                 uint32_t* abort_word = nullptr, uint64_t* ytag = nullptr) {
  __shared__ float sig[kShTok * 8];
  __shared__ float outb[kShTok][kShDnRows];
  constexpr int LPR = 16, RP = 4;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int slot = lane / LPR, kl = lane % LPR;
  const int H = a.H, Is = a.Is, NCH = Is / 8;
  const int o0 = rb * kShDnRows;
  uint4 wv[RP][CPL];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int orow = min(o0 + wave * 16 + slot * RP + r, H - 1);   // rows past H: computed, never stored
    const uint4* row = reinterpret_cast<const uint4*>(a.dn + (size_t)orow * Is);
#pragma unroll
    for (int j = 0; j < CPL; ++j) wv[r][j] = row[min(kl + LPR * j, NCH - 1)];
  }
  __builtin_amdgcn_sched_barrier(0);
  // sigmoid(x_t . gate), one token per wave at a time (T <= 64 here: kShTok * 8)
  const int nsig = min(a.T, kShTok * 8);
  for (int t = wave; t < nsig; t += kTileWaves) {
    const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)t * H);
    const uint4* gr = reinterpret_cast<const uint4*>(a.gate);
    float acc = 0.0f;
    for (int c = lane; c < H / 8; c += kWave) acc = dot8_bf16(gr[c], xr[c], acc);
    const float z = wave_sum(acc);
    if (lane == 0) sig[t] = __fdiv_rn(1.0f, 1.0f + expf(-z));
  }
  wait();
  uint4* hs = reinterpret_cast<uint4*>(lds);
  for (int t0 = 0; t0 < a.T; t0 += kShTok) {
    const int nt = min(kShTok, a.T - t0);
    if (t0 > 0 && t0 % (kShTok * 8) == 0) {   // more sigmoids (T > 64: the stand-alone kernel)
      __syncthreads();
      for (int t = wave; t < min(kShTok * 8, a.T - t0); t += kTileWaves) {
        const uint4* xr = reinterpret_cast<const uint4*>(a.x + (size_t)(t0 + t) * H);
        const uint4* gr = reinterpret_cast<const uint4*>(a.gate);
        float acc = 0.0f;
        for (int c = lane; c < H / 8; c += kWave) acc = dot8_bf16(gr[c], xr[c], acc);
        const float z = wave_sum(acc);
        if (lane == 0) sig[t] = __fdiv_rn(1.0f, 1.0f + expf(-z));
      }
    }
    __syncthreads();   // the previous group's reads of hs are done; sig is written
    if (htag) {
      Patience pat;
      bool gave_up = false;
      for (int q = threadIdx.x; q < nt * (Is / 2); q += kTileThreads) {
        const uint64_t* wp = htag + (size_t)t0 * (Is / 2) + q;
        uint64_t v = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while ((uint32_t)v != epoch && !gave_up) {
          if (pat.expired(abort_word)) {
            gave_up = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          v = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        reinterpret_cast<uint32_t*>(lds)[q] = (uint32_t)(v >> 32);
      }
    } else {
      batched_copy<kTileThreads, kStageBatch>(
          nt * NCH, [&](int q) { return hld128<COH>(a.h, 2 * (size_t)t0 * Is + 16 * (size_t)q); },
          [&](int q, uint4 v) { hs[q] = v; });
    }
    __syncthreads();
    float acc[RP][kShTok];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int t = 0; t < kShTok; ++t) acc[r][t] = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = kl + LPR * j;
      if (c < NCH) {
#pragma unroll
        for (int t = 0; t < kShTok; ++t) {
          if (t < nt) {
            const uint4 hv = hs[t * NCH + c];
#pragma unroll
            for (int r = 0; r < RP; ++r) acc[r][t] = dot8_bf16(wv[r][j], hv, acc[r][t]);
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int t = 0; t < kShTok; ++t) {
        const float v = lane_group_sum<LPR>(acc[r][t]);
        if (kl == 0 && t < nt) outb[t][wave * 16 + slot * RP + r] = v * sig[(t0 + t) % (kShTok * 8)];
      }
    __syncthreads();
    for (int q = threadIdx.x; q < nt * kShDnRows; q += kTileThreads) {
      const int t = q / kShDnRows, o = q % kShDnRows;
      if (o0 + o < H) {
        const size_t at = (size_t)(t0 + t) * H + o0 + o;
        const uint32_t bits = __builtin_bit_cast(uint32_t, outb[t][o]);
        if (ytag) __hip_atomic_store(&ytag[at], (uint64_t)bits << 32 | epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hst32<COH>(a.y, 4 * at, bits);
      }
    }
  }
}

}  // namespace moe
