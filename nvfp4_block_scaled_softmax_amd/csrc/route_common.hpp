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
//
// With TAG, a logit is not stored as a float but published as one 64-bit word
// tagged[t * E + e] = (logit bits << 32) | epoch, written as one atomic store, so
// that a reader polling the words knows when every logit of a call is there.
// XB: x chunks each thread keeps in flight while staging (all of them in one
// round trip when T * H / 8 <= NT * XB).
template <int NT, bool COH = false, bool TAG = false, int XB = 2>
__device__ __forceinline__ void router_logits_wave(const uint16_t* __restrict__ x,
                                                   const uint16_t* __restrict__ wr,
                                                   const float* __restrict__ bias, int T, int H,
                                                   int E, int e, uint4* xs,
                                                   float* __restrict__ logits,
                                                   uint64_t* __restrict__ tagged = nullptr,
                                                   uint32_t epoch = 0u) {
  const int nch = H / 8;
  const int lane = lane_id();
  // this lane's chunks of the router row go out first (H <= 4096: <= 8 chunks),
  // so their HBM latency overlaps the staging of x
  constexpr int kMaxChunks = kMaxDim / 8 / kWave;
  uint4 wv[kMaxChunks];
  const uint4* wrow = reinterpret_cast<const uint4*>(wr + (size_t)(e < E ? e : 0) * H);
#pragma unroll
  for (int j = 0; j < kMaxChunks; ++j) wv[j] = ld_stream128(wrow + min(lane + kWave * j, nch - 1));   // clamped; unused past nch
  __builtin_amdgcn_sched_barrier(0);
  batched_copy<NT, XB>(   // NT = threads of the workgroup
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
  // every token's row sum at once (DPP steps and four lane reads, no LDS
  // round trips), so the T reductions overlap instead of running in turn
  float red[kNarrowT];
#pragma unroll
  for (int t = 0; t < kNarrowT; ++t) red[t] = t < T ? wave_sum(acc[t]) : 0.0f;
#pragma unroll
  for (int t = 0; t < kNarrowT; ++t) {
    if (t < T) {
      const float v = red[t];
      if constexpr (TAG) {
        if (lane == 0)
          __hip_atomic_store(&tagged[(size_t)t * E + e],
                             (uint64_t)__builtin_bit_cast(uint32_t, v + b) << 32 | epoch,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        if (lane == 0) hst32<COH>(logits, 4 * ((size_t)t * E + e), __builtin_bit_cast(uint32_t, v + b));
      }
    }
  }
}

// Order-preserving int keys of finite floats (-0 taken as +0): a > b as floats
// exactly when key(a) > key(b), equal floats give equal keys.
__device__ __forceinline__ int order_key(float f) {
  const int b = __float_as_int(f + 0.0f);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

template <int CTRL>
__device__ __forceinline__ int dpp_i32(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

// Wave maximum of int keys: DPP steps within rows of 16, then the four rows'
// maxima on the scalar unit.
__device__ __forceinline__ int wave_max_key(int v) {
  v = max(v, dpp_i32<kDppXor1>(v));
  v = max(v, dpp_i32<kDppXor2>(v));
  v = max(v, dpp_i32<kDppHalfMirror>(v));
  v = max(v, dpp_i32<kDppMirror>(v));
  const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}

// One wave per token.  Lane L holds the S contiguous experts L*S .. L*S+S-1
// (their order keys in key[], kNoKey past E) and first sorts them by (value
// descending, index ascending), as 64-bit composites (order key << 32 |
// S-1-slot).  Each round then takes the wave maximum of the lanes' heads; among
// lanes tied on it the lowest holds the lowest index, so the lowest such lane
// wins, and it moves its next expert to the head.  The round's critical path is
// one wave reduction; no branches depend on the data.
//
// With lds_ids / lds_w, the chosen experts / weights also go to LDS (same
// [t][k] layout), for a caller that works on them within the workgroup; with
// ids and w null they go to LDS only.
constexpr int kNoKey = (int)0x80000000;   // below every key of a finite value

// Candidate selection before the rounds.  Let L be the k-th largest of the 64
// lanes' maxima: at least k keys are >= L, so every one of the k largest keys
// is >= L (the candidates), and any key larger than a candidate is itself a
// candidate: a candidate's rank among the candidates (by key descending, then
// index ascending) is its rank among all keys.  L comes from a most-significant-
// bit-first search over ballots (per bit: one vector compare, a scalar count),
// on the top 16 bits only (any L no larger than that maximum will do);
// the candidates go to LDS one per lane, each counts the candidates above it,
// and the k smallest counts are the selection in order.  More than kTopkCand
// candidates (many equal keys) take the rounds below instead; both give the
// same selection.
constexpr int kTopkCand = kWave;
struct TopkScratch {
  unsigned long long cand[kTopkCand];      // the candidates, then the selection in rank order
};

// Orders this wave's LDS writes before its later LDS reads by other lanes (LDS
// requests of one wave are served in issue order; the compiler must not move
// the accesses across).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
}

// The chosen experts' weights (lane j < k holds the j-th choice): renormalised
// softmax over the chosen logits, exp(l_j - l_max) / sum, and the stores.
template <bool COH>
__device__ __forceinline__ void topk_weights(int t, int k, int sel_k, int sel_i, int first_k,
                                             int32_t* __restrict__ ids, float* __restrict__ w, int* lds_ids,
                                             float* lds_w) {
  const int lane = lane_id();
  const float ex = lane < k ? expf(key_value(sel_k) - key_value(first_k)) : 0.0f;
  const float sum = wave_sum(ex);
  if (lane < k) {
    const float wt = __fdiv_rn(ex, sum);
    if (ids) hst32<COH>(ids, 4 * ((size_t)t * k + lane), (uint32_t)sel_i);
    if (w) hst32<COH>(w, 4 * ((size_t)t * k + lane), __builtin_bit_cast(uint32_t, wt));
    if (lds_ids) lds_ids[t * k + lane] = sel_i;
    if (lds_w) lds_w[t * k + lane] = wt;
  }
}

// Exclusive prefix over the wave's lanes of c (0 <= c < 2^BITS) and its total,
// from one ballot per bit of c and lane-mask counts: no memory round trips.
template <int BITS>
__device__ __forceinline__ int wave_prefix(int c, int& total) {
  int pre = 0;
  total = 0;
#pragma unroll
  for (int b = 0; b < BITS; ++b) {
    const unsigned long long m = __ballot((c >> b) & 1);
    pre += (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u)) << b;
    total += __popcll(m) << b;
  }
  return pre;
}

// Returns false (nothing written) when there are more than kTopkCand candidates.
template <int S>
__device__ __forceinline__ bool topk_by_rank(const int* key, int k, TopkScratch* sc, int& sel_k, int& sel_i,
                                             int& first_k) {
  static_assert(S <= 31, "a lane's candidate count must fit five bits");
  const int lane = lane_id();
  unsigned u[S];   // the keys as unsigned order keys
  unsigned m = 0u;
#pragma unroll
  for (int i = 0; i < S; ++i) {
    u[i] = (unsigned)key[i] ^ 0x80000000u;
    m = max(m, u[i]);
  }
  // L: the largest value, its low 16 bits zero, that at least k of the lanes'
  // maxima reach (no larger than the k-th largest maximum, which is all the
  // candidate set needs; the low bits would cost a search step each and admit
  // only a few candidates fewer)
  unsigned L = 0u;
#pragma unroll
  for (int b = 31; b >= 16; --b) {
    const unsigned c = L | (1u << b);
    if (__popcll(__ballot(m >= c)) >= (unsigned)k) L = c;
  }
  int c = 0;
#pragma unroll
  for (int i = 0; i < S; ++i) c += u[i] >= L;
  int total;
  int pos = wave_prefix<S < 16 ? 4 : 5>(c, total);
  if (total > kTopkCand) return false;
  // the candidates as ordered 64-bit words (larger key, then lower index,
  // first), padded with zeros (below every candidate) to a multiple of 8
#pragma unroll
  for (int i = 0; i < S; ++i)
    if (u[i] >= L) sc->cand[pos++] = (unsigned long long)u[i] << 32 | (0xFFFFFFFFu - (unsigned)(lane * S + i));
  const int padded = (total + 7) & ~7;
  if (lane >= total && lane < padded) sc->cand[lane] = 0ull;
  wave_lds_sync();
  const unsigned long long mine = lane < total ? sc->cand[lane] : 0ull;
  int r = 0;
  for (int q0 = 0; q0 < padded; q0 += 8) {
    unsigned long long v[8];
#pragma unroll
    for (int q = 0; q < 8; q += 2) {   // four reads in flight together
      const ulonglong2 p = *reinterpret_cast<const ulonglong2*>(&sc->cand[q0 + q]);
      v[q] = p.x;
      v[q + 1] = p.y;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) r += v[q] > mine;
  }
  wave_lds_sync();   // every lane has read the candidates
  if (lane < total && r < k) sc->cand[r] = mine;
  wave_lds_sync();
  const unsigned long long sel = sc->cand[lane < k ? lane : 0];
  sel_k = (int)((unsigned)(sel >> 32) ^ 0x80000000u);
  sel_i = (int)(0xFFFFFFFFu - (unsigned)sel);
  first_k = __builtin_amdgcn_readfirstlane(sel_k);
  wave_lds_sync();   // the next token of this wave writes the scratch again
  return true;
}

template <int S, bool COH = false>
__device__ __forceinline__ void topk_keys(const int* key, int t, int k, int32_t* __restrict__ ids,
                                          float* __restrict__ w, int* lds_ids = nullptr,
                                          float* lds_w = nullptr, TopkScratch* sc = nullptr) {
  const int lane = lane_id();
  int sel_k = 0, sel_i = 0, first_k = 0;
  if (!(sc && topk_by_rank<S>(key, k, sc, sel_k, sel_i, first_k))) {
  long long c[S];
#pragma unroll
  for (int i = 0; i < S; ++i)
    c[i] = (long long)((unsigned long long)(unsigned)key[i] << 32 | (unsigned)(S - 1 - i));
  // odd-even transposition sort, descending (composites are distinct)
#pragma unroll
  for (int r = 0; r < S; ++r) {
#pragma unroll
    for (int i = r & 1; i + 1 < S; i += 2) {
      const long long a = c[i], b = c[i + 1];
      const bool sw = b > a;
      c[i] = sw ? b : a;
      c[i + 1] = sw ? a : b;
    }
  }
  for (int j = 0; j < k; ++j) {
    const int hk = (int)(c[0] >> 32);
    const int m = wave_max_key(hk);
    const unsigned long long hit = __ballot(hk == m);
    const int wl = __ffsll((long long)hit) - 1;
    const int slot = S - 1 - __builtin_amdgcn_readlane((int)(unsigned)c[0], wl);
    if (lane == wl) {
#pragma unroll
      for (int i = 0; i + 1 < S; ++i) c[i] = c[i + 1];
      c[S - 1] = (long long)((unsigned long long)(unsigned)kNoKey << 32);
    }
    if (j == 0) first_k = m;
    sel_k = lane == j ? m : sel_k;
    sel_i = lane == j ? wl * S + slot : sel_i;
  }
  }
  topk_weights<COH>(t, k, sel_k, sel_i, first_k, ids, w, lds_ids, lds_w);
}

// topk_keys over token t's row of fp32 logits [T][E] in memory.
template <int S, bool COH = false>
__device__ __forceinline__ void topk_wave(const float* __restrict__ logits, int t, int E, int k,
                                          int32_t* __restrict__ ids, float* __restrict__ w,
                                          int* lds_ids = nullptr, TopkScratch* sc = nullptr) {
  const int lane = lane_id();
  const float* row = logits + (size_t)t * E;
  int key[S];
#pragma unroll
  for (int i = 0; i < S; ++i) {
    const int e = lane * S + i;
    const float x = __builtin_bit_cast(float, hld32<COH>(row, 4 * (size_t)(e < E ? e : E - 1)));   // masked below
    key[i] = e < E ? order_key(x) : kNoKey;
  }
  topk_keys<S, COH>(key, t, k, ids, w, lds_ids, nullptr, sc);
}

}  // namespace moe
