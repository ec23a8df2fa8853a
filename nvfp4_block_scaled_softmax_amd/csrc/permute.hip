// Token-to-expert permutation: a stable counting sort of the pairs p = t*k + j
// by expert id, built from wave ballot / prefix primitives.
//
// One workgroup of 8 waves:
//  1. histogram in LDS (integer atomics: the counts do not depend on order);
//  2. exclusive scan over the experts (wave prefix + per-wave totals);
//  3. pairs in chunks of 512, in order.  In each wave the lanes holding the same
//     expert find each other with a ballot loop (one iteration per distinct
//     expert); a lane's rank is the count of same-expert lanes below it.  The
//     per-wave group sizes go to LDS so that each lane adds the counts of the
//     same expert in the lower waves of the chunk; the running base of every
//     expert then advances by the chunk's count.  Ranks therefore follow p,
//     which makes the order within an expert's segment ascending in p.
#include "abi_common.hpp"
#include "device_common.hpp"

namespace moe {

constexpr int kPermWaves = 8;
constexpr int kPermThreads = kPermWaves * kWave;

__global__ void __launch_bounds__(kPermThreads) k_permute(const int32_t* __restrict__ ids, int P,
                                                          int E, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_row) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  __shared__ int wave_tot[kPermWaves];
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  for (int e = tid; e < E; e += kPermThreads) {
    cnt[e] = 0;
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  for (int p = tid; p < P; p += kPermThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  // exclusive scan of cnt over E <= 1024 entries: thread tid owns experts 2tid, 2tid+1
  {
    const int e0 = 2 * tid;
    const int c0 = e0 < E ? cnt[e0] : 0;
    const int c1 = e0 + 1 < E ? cnt[e0 + 1] : 0;
    const int own = c0 + c1;
    int incl = own;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    const int excl = before + incl - own;
    if (e0 < E) base[e0] = excl;
    if (e0 + 1 < E) base[e0 + 1] = excl + c0;
    __syncthreads();
    for (int e = tid; e < E; e += kPermThreads) offsets[e] = base[e];
    if (tid == kPermThreads - 1) {
      int total = 0;
      for (int w = 0; w < kPermWaves; ++w) total += wave_tot[w];
      offsets[E] = total;
    }
  }
  __syncthreads();
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < P; c0 += kPermThreads) {
    const int p = c0 + tid;
    int e = -1;
    if (p < P) {
      e = ids[p];
      if (e < 0 || e >= E) e = -1;
    }
    // same-expert groups within the wave
    unsigned long long mine = 0ull;
    unsigned long long todo = __ballot(e >= 0);
    while (todo) {
      const int leader = __ffsll((long long)todo) - 1;
      const int le = __shfl(e, leader, kWave);
      const unsigned long long m = __ballot(e == le);
      if (e == le) mine = m;
      todo &= ~m;
    }
    const int rank = __popcll(mine & lt_mask);
    const bool leader = e >= 0 && rank == 0;
    if (leader) wcnt[wave][e] = __popcll(mine);
    __syncthreads();
    if (e >= 0) {
      int lower = 0;
      for (int w = 0; w < wave; ++w) lower += wcnt[w][e];
      const int row = base[e] + lower + rank;
      sorted_pairs[row] = p;
      pair_row[p] = row;
    } else if (p < P) {
      pair_row[p] = -1;
    }
    __syncthreads();
    if (leader) {
      atomicAdd(&base[e], __popcll(mine));
      wcnt[wave][e] = 0;
    }
    __syncthreads();
  }
}

moe_status launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_row, hipStream_t s) {
  hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), 0, s, ids, T * k, E, offsets,
                     sorted_pairs, pair_row);
  return check_launch("moe_permute");
}

}  // namespace moe

extern "C" moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E,
                                  int32_t* expert_offsets, int32_t* sorted_pairs,
                                  int32_t* pair_row, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(topk_ids && expert_offsets && sorted_pairs && pair_row, MOE_E_ARG,
              "moe_permute: null pointer argument");
  MOE_REQUIRE(T >= 1 && k >= 1 && E >= 1 && E <= moe::kMaxExperts && k <= E &&
                  (int64_t)T * k <= (1 << 30),
              MOE_E_SHAPE, "moe_permute: bad shape T=%d k=%d E=%d", T, k, E);
  MOE_REQUIRE(moe::aligned(topk_ids, 4) && moe::aligned(expert_offsets, 4) &&
                  moe::aligned(sorted_pairs, 4) && moe::aligned(pair_row, 4),
              MOE_E_ALIGN, "moe_permute: misaligned pointer");
  return moe::launch_permute(topk_ids, T, k, E, expert_offsets, sorted_pairs, pair_row, s);
}
