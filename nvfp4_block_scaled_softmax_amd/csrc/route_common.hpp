// Router pieces shared by the per-stage kernels and the fused decode routing
// kernel: the few-token logits of one expert per wave, and the per-token top-k.
#pragma once
#include "abi_common.hpp"
#include "device_common.hpp"

namespace moe {

constexpr int kNarrowT = 8;

// Logits of expert e (this wave) for all T <= 8 tokens.  Every thread of the
// workgroup calls it (x is staged into xs by all of them); waves with e >= E
// only help with the staging.
template <int NT, bool COH = false>
__device__ __forceinline__ void router_logits_wave(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias, int T, int H,
                                                   int E, int e, uint4* xs,
                                                   float* __restrict__ logits) {
  const int nch = H / 8;
  const int lane = lane_id();
  // this lane's chunks of the router row go out first (H <= 4096: <= 8 chunks),
  // so their HBM latency overlaps the staging of x
  constexpr int kMaxChunks = kMaxDim / 8 / kWave;
  uint4 wv[kMaxChunks];
  const uint4* wrow = reinterpret_cast<const uint4*>(wr + (size_t)(e < E ? e : 0) * H);
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) wv[j] = wrow[min(lane + kWave * j, nch - 1)];   // clamped; unused past nch
  __builtin_amdgcn_sched_barrier(0);
  batched_copy<NT, 2>(   // NT = threads of the workgroup
      T * nch, [&](int i) { return reinterpret_cast<const uint4*>(x)[i]; },
      [&](int i, uint4 v) { xs[i] = v; });
  __syncthreads();
  if (e >= E) return;
  float acc[kNarrowT];
#pragma unroll
  for (int t = 0; t < kNarrowT; ++t) acc[t] = 0.0f;
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) {
    const int c = lane + kWave * j;
    if (c >= nch) break;
    const uint4 w = wv[j];
#pragma unroll
    for (int t = 0; t < kNarrowT; ++t) {
      if (t < T) {
        const uint4 xv = xs[t * nch + c];
        float a = acc[t];
        a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.x), bitcast<bf16x2>(xv.x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.y), bitcast<bf16x2>(xv.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.z), bitcast<bf16x2>(xv.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(w.w), bitcast<bf16x2>(xv.w), a, false);
        acc[t] = a;
      }
    }
  }
  const float b = bias ? bias[e] : 0.0f;
#pragma unroll
  for (int t = 0; t < kNarrowT; ++t) {
    if (t < T) {
      const float v = group_sum<kWave>(acc[t]);
      if (lane == 0) hst32<COH>(logits, 4 * ((size_t)t * E + e), __builtin_bit_cast(uint32_t, v + b));
    }
  }
}

// One wave per token.  Lane L holds the S contiguous experts L*S .. L*S+S-1, so
// among lanes tied on the maximum the lowest lane holds the lowest index.
// Each round: every lane's best free slot (strict >, so a lane keeps its lowest
// index among equal values), the wave maximum, the lowest lane holding it;
// that expert is marked taken.  No branches depend on the data.
// With lds_ids, the chosen experts also go to LDS (same [t][k] layout), for a
// caller that works on them within the workgroup.
template <int S, bool COH = false>
__device__ __forceinline__ void topk_wave(const float* __restrict__ logits, int t, int E, int k,
                                          int32_t* __restrict__ ids, float* __restrict__ w,
                                          int* lds_ids = nullptr) {
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;
  const float ninf = -__builtin_huge_valf();
  float v[S];
  uint32_t taken = 0u;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int e = lane * S + i;
    const float x = __builtin_bit_cast(float, hld32<COH>(row, 4 * (size_t)(e < E ? e : E - 1)));   // masked below
    v[i] = e < E ? x : ninf;
    taken |= (e < E ? 0u : 1u) << i;
  }
  float sel_v = 0.0f, first_v = 0.0f;
  int sel_i = 0;
  for (int j = 0; j < k; ++j) {
    float bv = ninf;
    int bs = S;                                   // no free slot
#pragma unroll
    for (int i = S - 1; i >= 0; --i) {            // descending: ties end on the lowest slot
      const bool better = !((taken >> i) & 1u) && v[i] >= bv;
      bv = better ? v[i] : bv;
      bs = better ? i : bs;
    }
    const float m = wave_max(bs < S ? bv : ninf);
    const unsigned long long hit = __ballot(bs < S && bv == m);
    const int win_lane = __ffsll((long long)hit) - 1;
    const int win_slot = __builtin_amdgcn_readlane(bs, win_lane);
    const int win = win_lane * S + win_slot;
    if (lane == win_lane) taken |= 1u << win_slot;
    if (j == 0) first_v = m;
    sel_v = lane == j ? m : sel_v;
    sel_i = lane == j ? win : sel_i;
  }
  // renormalised softmax over the chosen logits: exp(l_j - l_max) / sum
  const float ex = lane < k ? expf(sel_v - first_v) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    hst32<COH>(ids, 4 * ((size_t)t * k + lane), (uint32_t)sel_i);
    hst32<COH>(w, 4 * ((size_t)t * k + lane), __builtin_bit_cast(uint32_t, __fdiv_rn(ex, sum)));
    if (lds_ids) lds_ids[t * k + lane] = sel_i;
  }
}

}  // namespace moe
