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
#include "permute_common.hpp"

namespace moe {

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
