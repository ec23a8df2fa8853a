// Pieces of the stable counting sort shared by the permutation kernels and the
// fused decode routing kernel: the expert scan and the ballot-ranked scatter.
#pragma once
#include "abi_common.hpp"
#include "device_common.hpp"

namespace moe {

constexpr int kPermWaves = 8;
constexpr int kPermThreads = kPermWaves * kWave;

// Stable scatter of pairs [p0, p1) given each expert's first row in base[]
// (LDS): chunks of 512 in order; within a chunk the ballot groups and the
// per-wave counts rank the pairs; base advances by the chunk's counts.
__device__ __forceinline__ void scatter_range(const int32_t* __restrict__ ids, int p0, int p1, int E,
                                              int* base, int (*wcnt)[kMaxExperts],
                                              int32_t* __restrict__ sorted_pairs,
                                              int32_t* __restrict__ pair_row) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const unsigned long long lt_mask = (1ull << lane) - 1ull;
  for (int c0 = p0; c0 < p1; c0 += kPermThreads) {
    const int p = c0 + tid;
    int e = -1;
    if (p < p1) {
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
    } else if (p < p1) {
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

// Exclusive scan of cnt[0..E) into base[] (LDS, E <= 1024, 512 threads: two
// experts each); returns the total to every thread.
__device__ __forceinline__ int scan_experts(const int* cnt, int* base, int E, int* wave_tot) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
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
  int before = 0, total = 0;
  for (int w = 0; w < kPermWaves; ++w) {
    if (w < wave) before += wave_tot[w];
    total += wave_tot[w];
  }
  const int excl = before + incl - own;
  if (e0 < E) base[e0] = excl;
  if (e0 + 1 < E) base[e0 + 1] = excl + c0;
  __syncthreads();
  return total;
}

}  // namespace moe
