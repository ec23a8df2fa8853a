// Token-to-expert permutation: a stable counting sort of the pairs p = t*k + j
// by expert id, built from wave ballot / prefix primitives.
//
// Up to 2048 pairs (decode, verification) one workgroup does everything; more
// pairs (prefill) split into blocks of 1024 with three kernels: per-block expert
// counts, one workgroup that turns them into expert offsets and per-block
// bases (a scan over the blocks per expert, then over the experts), and a
// per-block scatter that ranks its pairs as below, starting from its bases.
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

__global__ void __launch_bounds__(kPermThreads) k_permute(const int32_t* __restrict__ ids, int P,
                                                          int E, int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ sorted_pairs,
                                                          int32_t* __restrict__ pair_row) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  __shared__ int wave_tot[kPermWaves];
  const int tid = threadIdx.x;
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
  const int total = scan_experts(cnt, base, E, wave_tot);
  for (int e = tid; e < E; e += kPermThreads) offsets[e] = base[e];
  if (tid == 0) offsets[E] = total;
  scatter_range(ids, 0, P, E, base, wcnt, sorted_pairs, pair_row);
}

// Multi-block path.  bc[b][e]: pairs of expert e in block b, turned in place
// into the first row of block b's expert-e pairs.
constexpr int kPermBlock = 1024;     // pairs per block
constexpr int kPermOneBlock = 2048;  // up to this many pairs: one workgroup

__global__ void __launch_bounds__(kPermThreads) k_permute_count(const int32_t* __restrict__ ids,
                                                                int P, int E,
                                                                int32_t* __restrict__ bc) {
  __shared__ int cnt[kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) cnt[e] = 0;
  __syncthreads();
  const int p0 = blockIdx.x * kPermBlock, p1 = min(P, p0 + kPermBlock);
  for (int p = p0 + tid; p < p1; p += kPermThreads) {
    const int e = ids[p];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kPermThreads) bc[(size_t)blockIdx.x * E + e] = cnt[e];
}

__global__ void __launch_bounds__(kPermThreads) k_permute_bases(int nblk, int E,
                                                                int32_t* __restrict__ bc,
                                                                int32_t* __restrict__ offsets) {
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int wave_tot[kPermWaves];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) {   // per expert: exclusive scan over blocks
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const int c = bc[(size_t)b * E + e];
      bc[(size_t)b * E + e] = run;
      run += c;
    }
    cnt[e] = run;
  }
  __syncthreads();
  const int total = scan_experts(cnt, base, E, wave_tot);
  for (int e = tid; e < E; e += kPermThreads) {
    offsets[e] = base[e];
    for (int b = 0; b < nblk; ++b) bc[(size_t)b * E + e] += base[e];
  }
  if (tid == 0) offsets[E] = total;
}

__global__ void __launch_bounds__(kPermThreads) k_permute_scatter(const int32_t* __restrict__ ids,
                                                                  int P, int E,
                                                                  const int32_t* __restrict__ bc,
                                                                  int32_t* __restrict__ sorted_pairs,
                                                                  int32_t* __restrict__ pair_row) {
  __shared__ int base[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kPermThreads) {
    base[e] = bc[(size_t)blockIdx.x * E + e];
#pragma unroll
    for (int w = 0; w < kPermWaves; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  const int p0 = blockIdx.x * kPermBlock;
  scatter_range(ids, p0, min(P, p0 + kPermBlock), E, base, wcnt, sorted_pairs, pair_row);
}

size_t permute_workspace(int P, int E) {
  return P > kPermOneBlock ? (size_t)((P + kPermBlock - 1) / kPermBlock) * E * 4 : 0;
}

moe_status launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_row, void* ws, hipStream_t s) {
  const int P = T * k;
  if (P <= kPermOneBlock) {
    hipLaunchKernelGGL(k_permute, dim3(1), dim3(kPermThreads), 0, s, ids, P, E, offsets,
                       sorted_pairs, pair_row);
    return check_launch("moe_permute");
  }
  const int nblk = (P + kPermBlock - 1) / kPermBlock;
  int32_t* bc = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(k_permute_count, dim3(nblk), dim3(kPermThreads), 0, s, ids, P, E, bc);
  moe_status st = check_launch("moe_permute (count)");
  if (st != MOE_OK) return st;
  hipLaunchKernelGGL(k_permute_bases, dim3(1), dim3(kPermThreads), 0, s, nblk, E, bc, offsets);
  if ((st = check_launch("moe_permute (bases)")) != MOE_OK) return st;
  hipLaunchKernelGGL(k_permute_scatter, dim3(nblk), dim3(kPermThreads), 0, s, ids, P, E, bc,
                     sorted_pairs, pair_row);
  return check_launch("moe_permute (scatter)");
}

}  // namespace moe

extern "C" size_t moe_permute_workspace_bytes(int T, int k, int E) {
  if (T < 1 || k < 1 || E < 1 || E > moe::kMaxExperts || (int64_t)T * k > (1 << 30)) return 0;
  return moe::permute_workspace(T * k, E);
}

extern "C" moe_status moe_permute(const int32_t* topk_ids, int T, int k, int E,
                                  int32_t* expert_offsets, int32_t* sorted_pairs,
                                  int32_t* pair_row, void* ws, size_t ws_bytes, hipStream_t s) {
  moe::clear_error();
  MOE_REQUIRE(topk_ids && expert_offsets && sorted_pairs && pair_row, MOE_E_ARG,
              "moe_permute: null pointer argument");
  MOE_REQUIRE(T >= 1 && k >= 1 && E >= 1 && E <= moe::kMaxExperts && k <= E &&
                  (int64_t)T * k <= (1 << 30),
              MOE_E_SHAPE, "moe_permute: bad shape T=%d k=%d E=%d", T, k, E);
  MOE_REQUIRE(moe::aligned(topk_ids, 4) && moe::aligned(expert_offsets, 4) &&
                  moe::aligned(sorted_pairs, 4) && moe::aligned(pair_row, 4) &&
                  moe::aligned(ws, 4),
              MOE_E_ALIGN, "moe_permute: misaligned pointer");
  const size_t need = moe::permute_workspace(T * k, E);
  MOE_REQUIRE(ws_bytes >= need && (need == 0 || ws), MOE_E_WORKSPACE,
              "moe_permute: workspace %zu < %zu bytes", ws_bytes, need);
  return moe::launch_permute(topk_ids, T, k, E, expert_offsets, sorted_pairs, pair_row, ws, s);
}
