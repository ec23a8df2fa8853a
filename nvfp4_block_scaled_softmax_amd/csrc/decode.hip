// Fused decode layer (T <= 8 tokens): the routed-expert layer in one launch
// (16-bit activations, up to 64 pairs: k_layer_decode, below) or two:
//
//   A  k_route_decode:   router logits (one wave per expert row); the last
//                        workgroup to finish runs top-k, the stable
//                        permutation and the list of active experts.
//   B  k_experts_decode: gate/up + SwiGLU tiles, down tiles and the combine.
//                        A down tile issues its weight loads at once and then
//                        waits for its expert's gate/up tiles, so the down
//                        weights stream while gate/up computes; the last down
//                        tile of each output-row block sums the token's expert
//                        outputs (and the residual) for those rows.
//
// The arithmetic is the per-stage kernels' own (shared device functions), so
// the fused layer is bit-identical to moe_route_topk + moe_permute +
// nvfp4_expert_ffn + moe_combine.
//
// Ordering between workgroups.  Gate/up tiles have lower workgroup indices
// than down tiles, and waits are only on lower-indexed workgroups, except a
// combining tile's wait for the other down tiles of its row block, which
// themselves wait only on gate/up tiles.  Workgroups are dispatched in index
// order (round-robin over the XCDs, in order within each), so every workgroup
// waited for is resident, done, or gets a slot from a workgroup that finishes
// without waiting: the waits cannot starve.  (A ticket from one shared atomic
// counter would not need that order, but 800 workgroups serialised on one
// counter cost more than the whole expert pass.)  HIP does not promise that
// dispatch order, so every wait is bounded (Patience: a deadline, and an abort
// word that the first wait to give up sets, which ends every other wait of the
// launch at its next check); the call then completes with the combine writing
// NaN where it gave up, and the abort word (the `timeouts` counter of the state
// block) stays non-zero for moe_layer_status to report.
//
// The data handed between workgroups (logits, h, y, the plan) crosses XCDs,
// whose L2s are not coherent with each other: it is written and read with
// device-coherent (sc1) accesses that pass the XCD-local caches.  In the two
// launches a producer waits for its stores to complete before its workgroup
// bumps a counter, and consumers poll the counter with relaxed device-scope
// loads.  In the single launch the values themselves carry the call's epoch
// (one 64-bit atomic store per value: logits, plan words, h pairs, y), and
// consumers poll the values, with no store-completion wait and no counter.  No
// L2 write-back or invalidate is needed.
//
// The counters and tagged words live in a state block at the start of the
// layer workspace.  It must be zero before the first call; every call leaves
// the counters at zero (A's last workgroup clears B's, the single launch's tail
// clears them before it publishes), and tagged words need no reset: a stale
// word carries another call's epoch.
#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <tuple>

#include "combine_common.hpp"
#include "ffn_narrow.hpp"
#include "permute_common.hpp"
#include "route_common.hpp"
#include "shared_common.hpp"

namespace moe {

constexpr int kDecMaxSlots = 512;     // active experts of a call: at most T * k <= 8 * 64
constexpr int kDecMaxRowBlocks = kMaxDim / kDnRows;
constexpr int kSmallP = 64;           // up to this many pairs the routing tail ranks them directly
// Arrival counters of a captured call: one per 128-byte line, workgroup i
// counting on line i % kArrivalLines, so that ~2000 adds at the start of a
// launch do not queue on one address.
constexpr int kArrivalLines = 64;
// The single launch runs a block's shared expert too when its intermediate is
// at most this wide (its down tile holds Is / 128 chunks per lane in registers).
constexpr int kFusedShIs = 512;

// Each counter sits on its own 128-byte line: many workgroups poll or bump them
// at once, and counters sharing a line would queue behind each other.
struct alignas(128) Counter {
  uint32_t v;
  uint32_t pad[31];
};

struct DecodeState {
  Counter route_done;                  // A: workgroups finished
  Counter timeouts;                    // waits that gave up: the abort word (stays 0)
  Counter dev_epoch;                   // single launch under graph capture: the low 31 bits of
                                       // the call's epoch, advanced by the call itself
  Counter arrivals[kArrivalLines];     // single launch under graph capture: workgroups of the
                                       // call that have read dev_epoch, spread over lines by
                                       // workgroup index (reset by the call)
  Counter outs_epoch;                  // single launch: epoch of the call whose routing outputs
                                       // (ids, weights, sorted pairs, pair rows) are complete
  int32_t n_active;                    // active experts (written by A)
  Counter gu_done[kDecMaxSlots];       // B: gate/up tiles finished, per active expert
  Counter dn_done[kDecMaxRowBlocks];   // B: down tiles finished, per output-row block
  int4 plan[kDecMaxSlots];             // active expert: (expert, first sorted row, rows, 0)
  // single-launch layer: every slot's plan packed with the call's epoch (see
  // pack_pub); one copy polled by gate/up tiles, one by down tiles
  uint64_t pub[2][kDecMaxSlots];
  // single-launch layer: the router logits of the call, each tagged with its
  // epoch ((logit bits << 32) | epoch), [T][E]; the routing tail polls them
  uint64_t logit_tag[kNarrowT * kMaxExperts];
  // single-launch layer: the down outputs y of the call, tagged the same way,
  // [sorted row][H]; each row block's combining tile polls them
  uint64_t y_tag[kSmallP * kMaxDim];
  // single-launch layer: the intermediate h, two bf16 values per tagged word,
  // [sorted row][I/2]; the down tiles poll them
  uint64_t h_tag[kSmallP * kMaxDim / 2];
  // single-launch block: the shared expert's intermediate [T][Is/2] (two bf16
  // per word) and its gated output [T][H], tagged the same way
  uint64_t sh_h_tag[kNarrowT * kFusedShIs / 2];
  uint64_t sh_y_tag[kNarrowT * kMaxDim];
};

size_t decode_state_bytes() { return sizeof(DecodeState); }

// A published plan entry in one 64-bit word (read and written as one atomic
// access): bits 0-31 the call's epoch, 32-42 the expert (kNoExpert: the slot
// is past the active count), 43-50 the mask of its tokens (an expert's sorted
// rows are its tokens in ascending order, so the mask gives the rows and their
// tokens), 51-56 the active count - 1, 57-62 its first sorted row.  Holds for
// E <= 1024, T <= 8 and up to kSmallP pairs.
constexpr uint32_t kNoExpert = 0x7FF;
__device__ __forceinline__ uint64_t pack_pub(uint32_t epoch, uint32_t e, uint32_t tmask, uint32_t row0,
                                             uint32_t n_active) {
  return (uint64_t)epoch | ((uint64_t)e << 32) | ((uint64_t)tmask << 43) | ((uint64_t)(n_active - 1) << 51) |
         ((uint64_t)row0 << 57);
}

// One slot of the expert half: its expert (< 0: no work), first sorted row,
// rows, the call's active experts, the mask of its tokens (-1: read them from
// sorted_pairs), and the epoch a combine waits for in outs_epoch (0: none).
struct SlotPlan {
  int e, row0, rows, n_active, tmask;
  uint32_t outs_epoch;
};
size_t decode_timeouts_offset() { return offsetof(DecodeState, timeouts); }

__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Thread 0 waits (bounded, see Patience) until *p >= want; the data behind the
// count is then read with device-coherent loads.
__device__ __forceinline__ void wait_at_least(const uint32_t* p, uint32_t want, uint32_t* abort_word) {
  if (threadIdx.x == 0) {
    Patience pat;
    while (ld_relaxed(p) < want && !pat.expired(abort_word)) __builtin_amdgcn_s_sleep(8);
  }
  __syncthreads();
}

// The stable permutation of P <= kSmallP pairs (of T <= 8 tokens) whose experts
// are in pid (LDS), by all NT threads: a pair's sorted row is (#pairs with a
// smaller expert) + (#earlier pairs with its expert).  Wave 0 holds one pair per
// lane and compares through lane reads (no memory round trips); splan gets the
// active experts in ascending order (expert, first row, rows, mask of their
// tokens), *s_n their count, which is returned.  The sorted pairs and pair rows
// go to memory (device-coherently with COH: read back in the same launch), or,
// with null pointers, to LDS only (lds_sorted / lds_prow).  The expert offsets
// are small_offsets' part.
template <bool COH>
__device__ int rank_small(const int* pid, int4* splan, int* s_n, int P, int k,
                          int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_row,
                          int* lds_sorted = nullptr, int* lds_prow = nullptr) {
  const int tid = threadIdx.x, lane = lane_id();
  if (tid < kWave) {
    const bool mine = lane < P;
    const int e = mine ? pid[lane] : 0x7FFFFFFF;
    // every lane reads the pairs' experts four at a time (one broadcast LDS
    // read; entries past P are masked by the uniform index test)
    int lt = 0, eq_before = 0, n_eq = 0, tmask = 0, first_lt = 0;
    if (P == k) {   // one token: its experts are distinct, a pair's row is its expert's rank
      for (int q0 = 0; q0 < P; q0 += 4) {
        const int4 f = *reinterpret_cast<const int4*>(pid + q0);
        lt += (f.x < e) + (q0 + 1 < P && f.y < e) + (q0 + 2 < P && f.z < e) + (q0 + 3 < P && f.w < e);
      }
      n_eq = 1;
      tmask = 1;
      first_lt = lt;
    } else {
      for (int q0 = 0, tq = 0, jq = 0; q0 < P; q0 += 4) {   // pair q is token tq's jq-th
        const int4 f4 = *reinterpret_cast<const int4*>(pid + q0);
        const int fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q0 + u;
          if (q < P) {
            const bool eq = fv[u] == e;
            lt += fv[u] < e;
            eq_before += eq && q < lane;
            n_eq += eq;
            tmask |= (int)eq << tq;
            if (++jq == k) {
              jq = 0;
              ++tq;
            }
          }
        }
      }
      // distinct experts below e: the pairs that are their expert's first
      const unsigned long long first = __ballot(mine && eq_before == 0);
      for (int q0 = 0; q0 < P; q0 += 4) {
        const int4 f4 = *reinterpret_cast<const int4*>(pid + q0);
        const int fv[4] = {f4.x, f4.y, f4.z, f4.w};
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (((first >> (q0 + u)) & 1ull) != 0ull) first_lt += fv[u] < e;
      }
    }
    const unsigned long long firsts = __ballot(mine && eq_before == 0);   // (the whole wave takes part)
    if (mine) {
      const int row = lt + eq_before;
      if (sorted_pairs) {
        hst32<COH>(sorted_pairs, 4 * (size_t)row, (uint32_t)lane);
        hst32<COH>(pair_row, 4 * (size_t)lane, (uint32_t)row);
      } else {
        lds_sorted[row] = lane;
        lds_prow[lane] = row;
      }
      if (eq_before == 0) splan[first_lt] = make_int4(e, lt, n_eq, tmask);
    }
    if (lane == 0) *s_n = __popcll(firsts);
  }
  __syncthreads();
  return *s_n;
}

// offsets[x] for x = 0..E from the n active experts in splan (ascending): the
// first row of the first active expert >= x (binary search), or P past the last.
template <int NT>
__device__ void small_offsets(const int4* splan, int n, int P, int E, int32_t* __restrict__ offsets) {
  for (int x = threadIdx.x; x <= E; x += NT) {
    int lo = 0, hi = n;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (splan[mid].x < x) lo = mid + 1;
      else hi = mid;
    }
    offsets[x] = lo < n ? splan[lo].y : P;
  }
}

// ------------------------------------------------------------------ A: routing
// 8 waves, one expert row each.  Dynamic LDS: x of the T tokens.  8-bit mode
// (xq_codes not null): the workgroups also quantize x per token for the expert
// half, from the x they hold in LDS, in the arithmetic of act_quant_fp8 (E4M3
// codes [T][H], fp32 scales [T][H/16]); the expert kernel, a later launch,
// reads them.
template <int S>
__global__ void __launch_bounds__(kPermThreads)
    k_route_decode(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                   const float* __restrict__ bias, int T, int H, int E, int k,
                   float* __restrict__ logits, int32_t* __restrict__ ids, float* __restrict__ tw,
                   int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pairs,
                   int32_t* __restrict__ pair_row, DecodeState* __restrict__ st,
                   uint8_t* __restrict__ xq_codes, float* __restrict__ xq_scales) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int cnt[kMaxExperts];
  __shared__ int base[kMaxExperts];
  __shared__ int rank[kMaxExperts];
  __shared__ int wcnt[kPermWaves][kMaxExperts];
  __shared__ int wave_tot[kPermWaves];
  // every pair's expert (T * k <= 8 * 64), 16-byte aligned: rank_small reads it
  // four at a time; the generic permutation reads it too, not the ids stored
  // to memory an instant before
  __shared__ __align__(16) int pid[kNarrowT * kMaxTopK];
  __shared__ int s_n;
  __shared__ int4 splan[kSmallP];
  __shared__ int s_last;
  __shared__ TopkScratch s_topk[kPermWaves];
  const int tid = threadIdx.x, wave = tid / kWave;
  router_logits_wave<kPermThreads, true, false, 8>(x, wr, bias, T, H, E, blockIdx.x * kPermWaves + wave,
                           reinterpret_cast<uint4*>(smem), logits);
  if (xq_codes) {   // (x of every token is in smem, staged by the call above)
    const int nb = H / 16;
    const uint16_t* xs = reinterpret_cast<const uint16_t*>(smem);
    for (int i = blockIdx.x * kPermThreads + tid; i < T * nb; i += gridDim.x * kPermThreads) {
      const uint4 u0 = *reinterpret_cast<const uint4*>(xs + (size_t)i * 16);
      const uint4 u1 = *reinterpret_cast<const uint4*>(xs + (size_t)i * 16 + 8);
      const uint32_t wv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
      float v[16];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = bf16_to_f32(wv[j] & 0xFFFFu);
        v[2 * j + 1] = bf16_to_f32(wv[j] >> 16);
      }
      uint32_t w4[4];
      const float sc = fp8_quant16(v, w4);
      *reinterpret_cast<uint4*>(xq_codes + (size_t)i * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
      xq_scales[i] = sc;
    }
  }
  wait_vmem();   // this wave's logits have reached the device-coherent level
  __syncthreads();
  if (tid == 0) {
    const uint32_t done =
        __hip_atomic_fetch_add(&st->route_done.v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = done == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  // ---- the last workgroup: every expert's logits are visible
  const int P = T * k;
  for (int t = wave; t < T; t += kPermWaves)
    topk_wave<S, true>(logits, t, E, k, ids, tw, pid, &s_topk[wave]);
  __syncthreads();   // pid is written
  if (P <= kSmallP) {
    const int n_act = rank_small<false>(pid, splan, &s_n, P, k, sorted_pairs, pair_row);
    small_offsets<kPermThreads>(splan, n_act, P, E, offsets);
    for (int i = tid; i < n_act; i += kPermThreads) st->plan[i] = splan[i];
    if (tid == 0) st->n_active = n_act;
  } else {
    for (int e = tid; e < E; e += kPermThreads) {
      cnt[e] = 0;
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) wcnt[w][e] = 0;
    }
    __syncthreads();
    for (int p = tid; p < P; p += kPermThreads) atomicAdd(&cnt[pid[p]], 1);
    __syncthreads();
    const int total = scan_experts(cnt, base, E, wave_tot);
    for (int e = tid; e < E; e += kPermThreads) offsets[e] = base[e];
    if (tid == 0) offsets[E] = total;
    // active experts in ascending order: a second scan, over the 0/1 flags
    for (int e = tid; e < E; e += kPermThreads) rank[e] = cnt[e] > 0;
    __syncthreads();
    const int n_active = scan_experts(rank, rank, E, wave_tot);
    for (int e = tid; e < E; e += kPermThreads)
      if (cnt[e] > 0) st->plan[rank[e]] = make_int4(e, base[e], cnt[e], 0);
    if (tid == 0) st->n_active = n_active;
    scatter_range(pid, 0, P, E, base, wcnt, sorted_pairs, pair_row);
  }
  // B's counters start at zero: the previous call's B has finished (it ran
  // before this kernel on the stream); clear what it may have counted, and the
  // single-launch entries (epoch 0 matches no call)
  for (int i = tid; i < 2 * kDecMaxSlots; i += kPermThreads) st->pub[i / kDecMaxSlots][i % kDecMaxSlots] = 0u;
  for (int i = tid; i < kDecMaxSlots; i += kPermThreads) st->gu_done[i].v = 0u;
  for (int i = tid; i < kDecMaxRowBlocks; i += kPermThreads) st->dn_done[i].v = 0u;
  if (tid == 0) __hip_atomic_store(&st->route_done.v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------ B: experts
// Modes whose intermediate the single launch hands over as tagged words.
template <int MODE>
constexpr bool kTagH = MODE == MOE_A16 || MODE == MOE_A8;

// The expert tiles of one call, wg counted from the first expert workgroup:
// [0, G) gate/up tile (slot, rb) = (wg / nrb_gu, wg % nrb_gu); [G, G + D) down
// tile of (slot, rb) likewise with nrb_dn.  plan_of(slot, role) gives the
// slot's SlotPlan, expert < 0 for a slot past the active count (its tiles exit
// at once).  FUSED: the single launch, where the 8-bit x is not in the
// workspace yet (the routing workgroups write it meanwhile), so the gate/up
// tiles quantize it themselves while they wait for the plan.
template <int MODE, int GL, int GC, int DL, int DC, bool FUSED = false, typename PlanOf>
__device__ __forceinline__ void expert_tiles(const FfnArgs& a, DecodeState* __restrict__ st, int wg,
                                             uint32_t dn_hold, int max_slots, int cols_gu, int cols_dn,
                                             const int32_t* __restrict__ pair_row,
                                             const float* __restrict__ tw,
                                             const uint16_t* __restrict__ residual,
                                             uint16_t* __restrict__ out, uint8_t* lds,
                                             const float* __restrict__ shared_y, PlanOf&& plan_of,
                                             const uint64_t* __restrict__ shared_ytag = nullptr) {
  __shared__ int s_flag;
  __shared__ int s_prow[kDecMaxSlots];            // the combine's pair rows, weights and residual,
  __shared__ float s_tw[kDecMaxSlots];            // loaded while the tile waits for gate/up
  __shared__ __align__(8) uint16_t s_res[kNarrowT][kDnRows];
  const int tid = threadIdx.x;
  const int nrb_gu = a.I / kGuRows, nrb_dn = (a.H + kDnRows - 1) / kDnRows;
  const int G = max_slots * nrb_gu;
  if (wg < G) {
    const int slot = wg / nrb_gu, rb = wg % nrb_gu;
    // x of every token fits the tile's LDS (16/8-bit modes): it is staged while
    // the plan is awaited, so no x load trails the weight loads
    const bool xs = MODE != MOE_A4 && a.T <= cols_gu;   // (always so in the single launch)
    if (xs) {
      if constexpr (FUSED && MODE == MOE_A8) stage_gateup_quant_a8(a, lds);
      else stage_gateup_cols<MODE, true>(a, 0, 0, 0, a.T, nullptr, lds);
      __syncthreads();
    }
    const SlotPlan pl = plan_of(slot, 0);
    if (pl.e < 0) return;
    if (kTagH<MODE> && pl.outs_epoch != 0u) {   // single launch: h goes out as tagged words
      if (FUSED && MODE == MOE_A8) {
        gateup_tile<MODE, GL, GC, true, false, true>(a, pl.e, pl.row0, pl.rows, rb, cols_gu, lds, pl.tmask,
                                                     st->h_tag, pl.outs_epoch);
      } else if (xs) {
        gateup_tile<MODE, GL, GC, true, false, true>(a, pl.e, pl.row0, pl.rows, rb, cols_gu, lds, pl.tmask,
                                                     st->h_tag, pl.outs_epoch);
      } else {
        gateup_tile<MODE, GL, GC, true>(a, pl.e, pl.row0, pl.rows, rb, cols_gu, lds, pl.tmask, st->h_tag,
                                        pl.outs_epoch);
      }
      return;
    }
    if constexpr (MODE != MOE_A4) {
      if (xs) gateup_tile<MODE, GL, GC, true, false, true>(a, pl.e, pl.row0, pl.rows, rb, cols_gu, lds, pl.tmask);
      else gateup_tile<MODE, GL, GC, true>(a, pl.e, pl.row0, pl.rows, rb, cols_gu, lds, pl.tmask);
    } else {
      gateup_tile<MODE, GL, GC, true, true>(a, pl.e, pl.row0, pl.rows, rb, cols_gu, lds, pl.tmask);
    }
    wait_vmem();   // this wave's h has reached the device-coherent level
    __syncthreads();
    if (tid == 0)
      __hip_atomic_fetch_add(&st->gu_done[slot].v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    const int d = wg - G, slot = d / nrb_dn, rb = d % nrb_dn;
    const SlotPlan pl = plan_of(slot, 1);
    if (pl.e < 0) return;
    if (dn_hold != 0u) {   // let the gate/up weights stream first (see launch_one3)
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      const uint64_t hold = (uint64_t)dn_hold * (uint64_t)pl.n_active;
      while (__builtin_amdgcn_s_memrealtime() - t0 < hold) __builtin_amdgcn_s_sleep(1);
    }
    down_tile<MODE, DL, DC, true>(a, pl.e, pl.row0, pl.rows, rb, cols_dn, lds, [&] {
      // (the weight loads are out) what a combine of this row block needs, in
      // case this tile turns out to be the block's last; in the single launch
      // the routing outputs are complete once outs_epoch holds the call's epoch
      if (pl.outs_epoch != 0u) {
        if (tid == 0) {
          Patience pat;
          while (ld_relaxed(&st->outs_epoch.v) != pl.outs_epoch && !pat.expired(&st->timeouts.v))
            __builtin_amdgcn_s_sleep(2);
        }
        __syncthreads();
      }
      const int P = a.T * a.k;
      for (int i = tid; i < P; i += kTileThreads) {
        s_prow[i] = (int)hld32<true>(pair_row, 4 * (size_t)i);
        s_tw[i] = __builtin_bit_cast(float, hld32<true>(tw, 4 * (size_t)i));
      }
      for (int i = tid; i < a.T * kDnRows; i += kTileThreads) {
        const int t = i / kDnRows, o = rb * kDnRows + i % kDnRows;
        s_res[t][i % kDnRows] = residual && o < a.H ? residual[(size_t)t * a.H + o] : (uint16_t)0;
      }
      if (!(kTagH<MODE> && pl.outs_epoch != 0u))   // (single launch: h words are polled instead)
        wait_at_least(&st->gu_done[slot].v, (uint32_t)nrb_gu, &st->timeouts.v);
    }, pl.outs_epoch != 0u ? st->y_tag : nullptr, pl.outs_epoch,
       kTagH<MODE> && pl.outs_epoch != 0u ? st->h_tag : nullptr, &st->timeouts.v);
    if (pl.outs_epoch != 0u) {
      // single launch: the tile of slot 0 (always active) combines its row block
      // by polling the tagged outputs of every pair's row; the others are done
      if (slot != 0) return;
      const uint32_t epoch = pl.outs_epoch;
      for (int i = tid; i < a.T * kDnRows; i += kTileThreads) {
        const int t = i / kDnRows, ol = i % kDnRows, o = rb * kDnRows + ol;
        if (o >= a.H) continue;
        float acc = 0.0f;
        // the abort word travels with every poll (no round trip of its own): an
        // output whose inputs were given up on, here or by a producer, is NaN
        uint32_t aborted = 0u;
        Patience pat;
        uint64_t sv = (uint64_t)epoch;   // the shared expert's output word (fused block), value 0 until read
        for (int j0 = 0; j0 < a.k; j0 += 16) {   // as combine_acc4: j ascending, one fma each
          uint64_t v[16];
          while (true) {
            bool ready = true;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const int j = j0 + u, r = j < a.k ? s_prow[t * a.k + j] : -1;
              v[u] = r >= 0 ? __hip_atomic_load(&st->y_tag[(size_t)r * a.H + o], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)
                            : (uint64_t)epoch;   // value 0
              ready = ready && (uint32_t)v[u] == epoch;
            }
            if (shared_ytag && j0 == 0) {   // polled with the first group
              sv = __hip_atomic_load(&shared_ytag[(size_t)t * a.H + o], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              ready = ready && (uint32_t)sv == epoch;
            }
            aborted |= ld_relaxed(&st->timeouts.v);
            if (ready) break;
            if (pat.expired(&st->timeouts.v)) {
              aborted = 1u;
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
#pragma unroll
          for (int u = 0; u < 16; ++u)
            if (j0 + u < a.k)
              acc = __builtin_fmaf(s_tw[t * a.k + j0 + u], __builtin_bit_cast(float, (uint32_t)(v[u] >> 32)), acc);
        }
        if (shared_ytag) acc += __builtin_bit_cast(float, (uint32_t)(sv >> 32));   // as add_shared4
        else if (shared_y) acc += shared_y[(size_t)t * a.H + o];                  // (one element)
        uint32_t ob = f32_to_bf16(acc);   // as combine_round4, one element
        if (residual) ob = f32_to_bf16(bf16_to_f32(s_res[t][ol]) + bf16_to_f32(ob));
        out[(size_t)t * a.H + o] = aborted != 0u ? kBf16NaN : (uint16_t)ob;
      }
      return;
    }
    wait_vmem();   // this wave's y has reached the device-coherent level
    __syncthreads();
    if (tid == 0) {
      // the abort word is read beside the counter bump (no round trip of its own)
      const uint32_t ab = ld_relaxed(&st->timeouts.v);
      const uint32_t c =
          __hip_atomic_fetch_add(&st->dn_done[rb].v, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_flag = c == (uint32_t)pl.n_active - 1 ? (ab != 0u ? 2 : 1) : 0;
    }
    __syncthreads();
    if (s_flag == 2) {   // a wait of this call gave up: the block's outputs are NaN
      for (int i = tid; i < a.T * kDnRows; i += kTileThreads) {
        const int t = i / kDnRows, o = rb * kDnRows + i % kDnRows;
        if (o < a.H) out[(size_t)t * a.H + o] = kBf16NaN;
      }
    } else if (s_flag) {   // every expert's rows of this block are in: combine them
      const int n4 = kDnRows / 4, c0 = rb * n4;
      for (int i = tid; i < a.T * n4; i += kTileThreads) {
        const int t = i / n4, c = c0 + i % n4;
        if (4 * c < a.H) {
          float4 acc = combine_acc4(
              [&](int r) {
                return __builtin_bit_cast(float4, hld128<true>(a.y, 4 * ((size_t)r * a.H) + 16 * (size_t)c));
              },
              s_prow, s_tw, t, a.k);
          add_shared4(acc, shared_y, t, a.H, c);
          const uint2 rr = *reinterpret_cast<const uint2*>(&s_res[t][4 * (c - c0)]);
          *reinterpret_cast<uint2*>(out + (size_t)t * a.H + (size_t)c * 4) =
              combine_round4(acc, residual != nullptr, rr);
        }
      }
    }
  }
}

// The expert half on its own: the routing kernel has finished, so the plan is
// read with plain loads.
// Four workgroups per CU (at most 128 VGPRs) where the tiles fit without
// spilling: a call at T = 8 has thousands of tiles, so occupancy sets how many
// rounds they take (4-bit mode: 129 VGPRs unbounded, 3 per CU).  The LDS side
// of the same bound: launch_b stages at most kExpertGuCols columns.
constexpr int kExpertGuCols = 4;
template <int MODE, int GL, int GC, int DL, int DC>
__global__ void __launch_bounds__(kTileThreads, MODE == kModeQ4 ? 1 : 4)
    k_experts_decode(FfnArgs a, DecodeState* __restrict__ st, int max_slots, int cols_gu,
                     int cols_dn, const int32_t* __restrict__ pair_row,
                     const float* __restrict__ tw, const uint16_t* __restrict__ residual,
                     uint16_t* __restrict__ out, const float* __restrict__ shared_y) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int n_active = st->n_active;
  expert_tiles<MODE, GL, GC, DL, DC>(
      a, st, blockIdx.x, 0u, max_slots, cols_gu, cols_dn, pair_row, tw, residual, out, lds, shared_y,
      [&](int slot, int) {
        if (slot >= n_active) return SlotPlan{-1, 0, 0, 0, -1, 0u};
        const int4 pl = st->plan[slot];
        return SlotPlan{pl.x, pl.y, pl.z, n_active, -1, 0u};
      });
}

// ------------------------------------------------------------------ A + B in one launch
// Up to kSmallP pairs: workgroups [0, R) compute the router logits (one expert
// per wave), each published as a word stamped with this call's epoch (a number
// not reused, never 0: from the host, or under graph capture from the device,
// see below); the last routing workgroup polls them and runs top-k and
// the permutation; the expert tiles follow.  It publishes each slot's plan
// entry stamped with the epoch; expert tiles poll their slot's entry until the
// stamp matches.  An entry and its stamp are one 64-bit word, written and
// polled as one atomic access; every entry is rewritten each call.  Gate/up
// tiles publish h, and down tiles y, the same way, so each consumer polls the
// values it needs (slot 0's down tile of each output-row block combines).
//
// The tail keeps top-k, weights and the permutation in LDS until the entries
// are out: a workgroup barrier waits for the wave's outstanding stores, so a
// device-coherent store before any barrier of the tail would put its round trip
// on the critical path.  An entry is all a gate/up tile needs (it carries the
// expert's tokens); the routing outputs (ids, weights, sorted pairs, pair rows,
// offsets) are stored after the entries, and outs_epoch announces them once
// complete, which a down tile checks before it reads pair rows and weights for
// the combine.  The counters of the expert half are cleared by the tail's first
// wave before it polls the logits, and it waits for those stores there (while
// the other workgroups' logits are on their way), so they are complete before
// any entry goes out.
// Four workgroups per CU must fit for the whole grid of a one-token call to be
// resident at once: at most 128 VGPRs (four waves per SIMD), which the shapes
// up to H = 3072 and E = 512 meet without spilling; wider ones are left to the
// compiler's choice.
template <int S, int MODE, int GL, int GC, int DL, int DC, bool SH>
__global__ void __launch_bounds__(kTileThreads, (GC <= 3 && S <= 8) ? 4 : 1)
    k_layer_decode(const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr,
                   const float* __restrict__ bias, float* __restrict__ logits,
                   int32_t* __restrict__ ids, float* __restrict__ tw, FfnArgs a,
                   DecodeState* __restrict__ st, int max_slots, int cols_gu, int cols_dn,
                   int32_t* __restrict__ pair_row, const uint16_t* __restrict__ residual,
                   uint16_t* __restrict__ out, uint32_t epoch_arg, uint32_t dn_hold,
                   const float* __restrict__ shared_y, SharedArgs sa, int sgu, int sdn) {
  extern __shared__ __align__(16) uint8_t lds[];
  // epoch_arg 0 (a call recorded into a graph, where an epoch baked into the
  // launch would repeat on every replay): the epoch is 2^31 | dev_epoch (never 0
  // and never a host epoch, whose top bit is clear).  Every workgroup reads it
  // first and then counts itself in `arrivals` (an add whose result nobody waits
  // for); once all have arrived, the routing tail advances dev_epoch for the
  // next call and resets the count.  No workgroup reads dev_epoch after its
  // start, so every workgroup of the call holds the same epoch, and the next call
  // (a later kernel on the stream) sees the advanced one: the captured layer is
  // one graph node.
  uint32_t epoch = epoch_arg;
  if (epoch_arg == 0u) {
    const uint32_t v = __hip_atomic_load(&st->dev_epoch.v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) {
      wait_vmem();   // the read has returned before the arrival is counted
      __hip_atomic_fetch_add(&st->arrivals[blockIdx.x % kArrivalLines].v, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    epoch = 0x80000000u | (v & 0x7FFFFFFFu);
  }
  __shared__ __align__(16) int pid[kSmallP];   // 16-byte aligned: rank_small reads it four at a time
  __shared__ int s_n;
  __shared__ int4 splan[kSmallP];
  __shared__ SlotPlan s_pl;
  __shared__ float s_tw[kSmallP];
  __shared__ int s_sorted[kSmallP], s_prow[kSmallP];
  __shared__ TopkScratch s_topk[kTileWaves];
  const int tid = threadIdx.x, wave = tid / kWave;
  const int T = a.T, H = a.H, E = a.E, k = a.k, P = T * k;
  const int R = (E + kTileWaves - 1) / kTileWaves;
  const int wg = blockIdx.x;
  if (wg < R) {
    router_logits_wave<kTileThreads, true, true>(x, wr, bias, T, H, E, wg * kTileWaves + wave,
                                                 reinterpret_cast<uint4*>(lds), logits,
                                                 st->logit_tag, epoch);
    if constexpr (MODE == MOE_A8) {
      // x quantized per token into the workspace (the gate/up tiles quantize
      // their own copy in LDS; this one is for the caller), from the x that
      // router_logits_wave staged in LDS, after the logits are out
      const int nb = H / 16;
      const uint16_t* xl = reinterpret_cast<const uint16_t*>(lds);
      uint8_t* xc = const_cast<uint8_t*>(a.xq_codes);
      float* xsc = static_cast<float*>(const_cast<void*>(a.xq_scales));
      for (int i = wg * kTileThreads + tid; i < T * nb; i += R * kTileThreads) {
        const uint4 u0 = *reinterpret_cast<const uint4*>(xl + (size_t)i * 16);
        const uint4 u1 = *reinterpret_cast<const uint4*>(xl + (size_t)i * 16 + 8);
        const uint32_t wv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
        float v[16];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          v[2 * j] = bf16_to_f32(wv[j] & 0xFFFFu);
          v[2 * j + 1] = bf16_to_f32(wv[j] >> 16);
        }
        uint32_t w4[4];
        const float sc = fp8_quant16(v, w4);
        *reinterpret_cast<uint4*>(xc + (size_t)i * 16) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
        xsc[i] = sc;
      }
    }
    if (wg != R - 1) return;   // the last routing workgroup runs the tail
    if (wave == 0) {   // the expert half's counters (left by the previous call) back to zero
      const int nrb_dn = (H + kDnRows - 1) / kDnRows;
      for (int i = lane_id(); i < max_slots; i += kWave)
        __hip_atomic_store(&st->gu_done[i].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (int i = lane_id(); i < nrb_dn; i += kWave)
        __hip_atomic_store(&st->dn_done[i].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      wait_vmem();
    }
    // one wave per token polls the token's E tagged logits until every one
    // carries this call's epoch (the words are this call's only once they
    // match), then selects from the values it holds
    for (int t = wave; t < T; t += kTileWaves) {
      const uint64_t* row = st->logit_tag + (size_t)t * E;
      const int lane = lane_id();
      uint64_t v[S];
      Patience pat;
      while (true) {
        bool mine = true;
#pragma unroll
        for (int i = 0; i < S; ++i) {
          const int e = lane * S + i;
          v[i] = e < E ? __hip_atomic_load(&row[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : (uint64_t)epoch;
          mine = mine && (uint32_t)v[i] == epoch;
        }
        if (__all(mine)) break;
        // every lane polls in step, so the wave gives up as one (stale logits
        // still give valid expert ids: each key's slot is its expert)
        if (pat.expired(&st->timeouts.v)) break;
        __builtin_amdgcn_s_sleep(2);
      }
      int key[S];
#pragma unroll
      for (int i = 0; i < S; ++i)
        key[i] = lane * S + i < E ? order_key(__builtin_bit_cast(float, (uint32_t)(v[i] >> 32))) : kNoKey;
      topk_keys<S, true>(key, t, k, nullptr, nullptr, pid, s_tw, &s_topk[wave]);
    }
    __syncthreads();
    const int n_act = rank_small<true>(pid, splan, &s_n, P, k, nullptr, nullptr, s_sorted, s_prow);
    // every entry, also those this call does not poll, so that each holds the
    // previous call's epoch at most
    for (int i = tid; i < 2 * kDecMaxSlots; i += kTileThreads) {
      const int slot = i % kDecMaxSlots;
      const int4 pl = slot < n_act ? splan[slot] : make_int4((int)kNoExpert, 0, 0, 0);
      __hip_atomic_store(&st->pub[i / kDecMaxSlots][slot],
                         pack_pub(epoch, (uint32_t)pl.x, (uint32_t)pl.w, (uint32_t)pl.y, (uint32_t)n_act),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the routing outputs, after the entries
    for (int i = tid; i < P; i += kTileThreads) {
      hst32<true>(ids, 4 * (size_t)i, (uint32_t)pid[i]);
      hst32<true>(tw, 4 * (size_t)i, __builtin_bit_cast(uint32_t, s_tw[i]));
      hst32<true>(const_cast<int32_t*>(a.sorted_pairs), 4 * (size_t)i, (uint32_t)s_sorted[i]);
      hst32<true>(pair_row, 4 * (size_t)i, (uint32_t)s_prow[i]);
    }
    small_offsets<kTileThreads>(splan, n_act, P, E, const_cast<int32_t*>(a.offsets));
    wait_vmem();
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&st->outs_epoch.v, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (epoch_arg == 0u && wave == 0) {   // the next captured call's epoch, once every workgroup holds this one
      const int lane = lane_id();
      Patience pat;
      while (true) {
        const uint32_t n = lane < kArrivalLines ? ld_relaxed(&st->arrivals[lane].v) : 0u;
        const uint32_t total = (uint32_t)wave_sum((float)n);   // exact: counts below 2^24
        if (total >= gridDim.x || pat.expired(&st->timeouts.v)) break;
        __builtin_amdgcn_s_sleep(8);
      }
      if (lane < kArrivalLines)
        __hip_atomic_store(&st->arrivals[lane].v, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0)
        __hip_atomic_store(&st->dev_epoch.v, (epoch + 1u) & 0x7FFFFFFFu, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    return;
  }
  // a block's shared expert (sgu + sdn workgroups, none for a plain layer): it
  // needs no routing, so its weights stream while the call is routed; h and y
  // go out as tagged words, the combine polls y
  if constexpr (SH) {   // (a separate instantiation: a plain layer's kernel carries none of this)
    if (wg < R + sgu) {
      shared_gateup_tile<4 * GC, true>(sa, wg - R, lds, st->sh_h_tag, epoch);
      return;
    }
    if (wg < R + sgu + sdn) {
      shared_down_tile<kFusedShIs / 128, true>(sa, wg - R - sgu, lds, NoHook{}, st->sh_h_tag, epoch,
                                               &st->timeouts.v, st->sh_y_tag);
      return;
    }
  }
  expert_tiles<MODE, GL, GC, DL, DC, true>(
      a, st, wg - R - (SH ? sgu + sdn : 0), dn_hold, max_slots, cols_gu, cols_dn, pair_row, tw, residual, out, lds,
      shared_y,
      [&](int slot, int role) {
        if (tid == 0) {
          const uint64_t* e = &st->pub[role][slot];
          Patience pat;
          uint64_t v;
          while (true) {
            v = __hip_atomic_load(e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)v == epoch || pat.expired(&st->timeouts.v)) break;
            __builtin_amdgcn_s_sleep(4);
          }
          const uint32_t ex = (uint32_t)(v >> 32) & 0x7FFu;
          if ((uint32_t)v != epoch) {
            s_pl = SlotPlan{-1, 0, 0, 0, -1, 0u};   // gave up on this tile
          } else {
            const int tmask = (int)((v >> 43) & 0xFFu);
            s_pl = ex == kNoExpert ? SlotPlan{-1, 0, 0, 0, -1, 0u}
                                   : SlotPlan{(int)ex, (int)((v >> 57) & 0x3Fu), (int)__popc((unsigned)tmask),
                                              (int)((v >> 51) & 0x3Fu) + 1, tmask, epoch};
          }
        }
        __syncthreads();
        return s_pl;
      }, SH ? st->sh_y_tag : nullptr);
}

// ------------------------------------------------------------------ launch
// Workgroups of `kernel` (kTileThreads threads, `lds` bytes of dynamic LDS) that
// are resident at once on the current device, cached per (device, kernel, LDS);
// 0 when the runtime does not say.
static int resident_groups(const void* kernel, size_t lds) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_tuple(dev, kernel, lds);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int per_cu = 0, cus = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, kTileThreads, lds) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return 0;
  return cache[key] = per_cu * cus;
}

// Hold-back of the down tiles' weight loads in the single launch, per active
// expert, in ticks of the 100 MHz real-time counter: 300 ns, the time to stream
// one expert's gate/up weights (1.77 MB at H=3072, I=512) at the ~6 TB/s the
// expert loads reach.  When every workgroup of the call is resident at once,
// gate/up and down tiles see the plan together and their loads would share the
// bandwidth, while gate/up is on the critical path and the down weights are
// needed only after it (measured at T=1: 23.8 -> 23.15 us per call).  When the
// grid is not resident at once, down tiles start late anyway and holding them
// back only delays them (measured at T=2: +3.5 us), so there is no hold-back.
constexpr uint32_t kDnHoldTicksPerExpert = 30;

template <int S>
static void launch_a(const uint16_t* x, const uint16_t* wr, const float* bias, int T, int H, int E,
                     int k, float* logits, int32_t* ids, float* tw, int32_t* offsets,
                     int32_t* sorted, int32_t* prow, DecodeState* st, uint8_t* xq_codes, float* xq_scales,
                     hipStream_t s) {
  hipLaunchKernelGGL(k_route_decode<S>, dim3((E + kPermWaves - 1) / kPermWaves), dim3(kPermThreads),
                     (size_t)T * H * 2, s, x, wr, bias, T, H, E, k, logits, ids, tw, offsets,
                     sorted, prow, st, xq_codes, xq_scales);
}

// (lanes per row, chunks per lane) of the narrow tiles for a reduction of NC
// 32-wide chunks, as the per-stage kernels choose them; the fused kernel is
// built for gate/up with 33..128 chunks and down with 5..32 chunks.
static int gu_config(int nc) { return nc <= 32 ? -1 : nc <= 64 ? 2 : nc <= 96 ? 3 : nc <= 128 ? 4 : -1; }
static int dn_config(int nc) { return nc <= 4 ? -1 : nc <= 8 ? 8 : nc <= 16 ? 16 : nc <= 32 ? 32 : -1; }

bool decode_fusable(int T, int H, int I) {
  return T <= kNarrowT && gu_config(H / 32) > 0 && dn_config(I / 32) > 0;
}

static bool single_launch(moe_act_mode mode, int T, int k) {
  return (mode == MOE_A16 || mode == MOE_A8) && T * k <= kSmallP;
}

int decode_launches(moe_act_mode mode, int T, int k, int H, int I) {
  if (T < 1 || k < 1 || !decode_fusable(T, H, I)) return 0;
  return single_launch(mode, T, k) ? 1 : 2;
}

template <int MODE, int GC, int DL>
static void launch_b3(const FfnArgs& a, DecodeState* st, int max_slots, int cols_gu, int cols_dn,
                      const int32_t* prow, const float* tw, const uint16_t* residual,
                      uint16_t* out, const float* shared_y, hipStream_t s) {
  const int grid = max_slots * (a.I / kGuRows + (a.H + kDnRows - 1) / kDnRows);
  const size_t lds_gu = (size_t)cols_gu * (a.H / 32) * ChunkLds<MODE>::kStride;
  const size_t lds_dn = (size_t)cols_dn * (a.I / 32) * ChunkLds<MODE>::kStride;
  hipLaunchKernelGGL((k_experts_decode<MODE, 32, GC, DL, 1>), dim3(grid), dim3(kTileThreads),
                     lds_gu > lds_dn ? lds_gu : lds_dn, s, a, st, max_slots, cols_gu, cols_dn, prow,
                     tw, residual, out, shared_y);
}

template <int MODE, int GC>
static void launch_b2(const FfnArgs& a, int dl, DecodeState* st, int max_slots, int cols_gu,
                      int cols_dn, const int32_t* prow, const float* tw, const uint16_t* residual,
                      uint16_t* out, const float* shy, hipStream_t s) {
  if (dl == 8) launch_b3<MODE, GC, 8>(a, st, max_slots, cols_gu, cols_dn, prow, tw, residual, out, shy, s);
  else if (dl == 16) launch_b3<MODE, GC, 16>(a, st, max_slots, cols_gu, cols_dn, prow, tw, residual, out, shy, s);
  else launch_b3<MODE, GC, 32>(a, st, max_slots, cols_gu, cols_dn, prow, tw, residual, out, shy, s);
}

template <int MODE>
static void launch_b(const FfnArgs& a, DecodeState* st, int max_slots, const int32_t* prow,
                     const float* tw, const uint16_t* residual, uint16_t* out, const float* shy,
                     hipStream_t s) {
  // column groups as the per-stage kernels size them, gate/up at most 4: the
  // dynamic LDS is sized for the widest slot, but a slot of a call with up to
  // 8 tokens mostly holds 1 or 2 of them, and 8 columns of x (37 KB in the
  // 4-bit mode at H = 3072) left room for only 3 workgroups per CU; with 4 the
  // tiles run 4 per CU and a wider slot loops over its columns (W4A4 at T = 8:
  // 84.4 -> 77.4 us per call)
  const int per_col_gu = (a.H / 32) * ChunkLds<MODE>::kStride;
  const int per_col_dn = (a.I / 32) * ChunkLds<MODE>::kStride;
  const int cols_gu = max(1, min(min(kExpertGuCols, a.T), kLdsBudget / per_col_gu));
  const int cols_dn = max(1, min(min(8, a.T), kLdsBudget / per_col_dn));
  const int gc = gu_config(a.H / 32), dl = dn_config(a.I / 32);
  if (gc == 2) launch_b2<MODE, 2>(a, dl, st, max_slots, cols_gu, cols_dn, prow, tw, residual, out, shy, s);
  else if (gc == 3) launch_b2<MODE, 3>(a, dl, st, max_slots, cols_gu, cols_dn, prow, tw, residual, out, shy, s);
  else launch_b2<MODE, 4>(a, dl, st, max_slots, cols_gu, cols_dn, prow, tw, residual, out, shy, s);
}

// ---- the single-launch layer (16- and 8-bit activations, up to kSmallP pairs)
// sa: a block's shared expert run by the same launch (decode_fuses_shared: 16-bit
// mode only), or null.
template <int MODE, int S, int GC, int DL>
static void launch_one3(const FfnArgs& a, const uint16_t* x, const uint16_t* wr, const float* bias,
                        float* logits, int32_t* ids, float* tw, int32_t* prow, DecodeState* st,
                        const uint16_t* residual, uint16_t* out, uint64_t epoch, const float* shy,
                        const SharedArgs* sa, hipStream_t s) {
  const int P = a.T * a.k, max_slots = P < a.E ? P : a.E;
  const int cols = max(1, min(min(8, a.T), kLdsBudget / ((a.H / 32) * ChunkLds<MODE>::kStride)));
  const int cols_dn = max(1, min(min(8, a.T), kLdsBudget / ((a.I / 32) * ChunkLds<MODE>::kStride)));
  const int R = (a.E + kTileWaves - 1) / kTileWaves;
  const int sgu = sa ? sa->Is / kShGuRows : 0, sdn = sa ? (a.H + kShDnRows - 1) / kShDnRows : 0;
  const int grid = R + sgu + sdn + max_slots * (a.I / kGuRows + (a.H + kDnRows - 1) / kDnRows);
  size_t lds = (size_t)a.T * a.H * 2;
  lds = std::max(lds, (size_t)cols * (a.H / 32) * ChunkLds<MODE>::kStride);
  lds = std::max(lds, (size_t)cols_dn * (a.I / 32) * ChunkLds<MODE>::kStride);
  if (sa) lds = std::max(lds, (size_t)a.T * sa->Is * 2);   // the shared down tile's h
  const SharedArgs sarg = sa ? *sa : SharedArgs{};
  auto go = [&](auto kernel) {
    const int cap = resident_groups(reinterpret_cast<const void*>(kernel), lds);
    const uint32_t dn_hold = cap > 0 && grid <= cap ? kDnHoldTicksPerExpert : 0u;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(kTileThreads), lds, s, x, wr, bias, logits, ids, tw, a, st,
                       max_slots, cols, cols_dn, prow, residual, out, (uint32_t)epoch, dn_hold, shy, sarg, sgu,
                       sdn);
  };
  if constexpr (MODE == MOE_A16) {
    if (sa) go(&k_layer_decode<S, MODE, 32, GC, DL, 1, true>);
    else go(&k_layer_decode<S, MODE, 32, GC, DL, 1, false>);
  } else {
    go(&k_layer_decode<S, MODE, 32, GC, DL, 1, false>);
  }
}

template <int MODE, int S, int GC>
static void launch_one2(int dl, const FfnArgs& a, const uint16_t* x, const uint16_t* wr,
                        const float* bias, float* logits, int32_t* ids, float* tw, int32_t* prow,
                        DecodeState* st, const uint16_t* residual, uint16_t* out, uint64_t epoch,
                        const float* shy, const SharedArgs* sa, hipStream_t s) {
  if (dl == 8) launch_one3<MODE, S, GC, 8>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else if (dl == 16) launch_one3<MODE, S, GC, 16>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else launch_one3<MODE, S, GC, 32>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
}

template <int MODE, int S>
static void launch_one(const FfnArgs& a, const uint16_t* x, const uint16_t* wr, const float* bias,
                       float* logits, int32_t* ids, float* tw, int32_t* prow, DecodeState* st,
                       const uint16_t* residual, uint16_t* out, uint64_t epoch, const float* shy,
                       const SharedArgs* sa, hipStream_t s) {
  const int gc = gu_config(a.H / 32), dl = dn_config(a.I / 32);
  if (gc == 2) launch_one2<MODE, S, 2>(dl, a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else if (gc == 3) launch_one2<MODE, S, 3>(dl, a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else launch_one2<MODE, S, 4>(dl, a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
}

template <int MODE>
static void launch_one_mode(const FfnArgs& a, const uint16_t* x, const uint16_t* wr, const float* bias,
                            float* logits, int32_t* ids, float* tw, int32_t* prow, DecodeState* st,
                            const uint16_t* residual, uint16_t* out, uint64_t epoch, const float* shy,
                            const SharedArgs* sa, hipStream_t s) {
  const int E = a.E;
  if (E <= 64) launch_one<MODE, 1>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else if (E <= 128) launch_one<MODE, 2>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else if (E <= 256) launch_one<MODE, 4>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else if (E <= 512) launch_one<MODE, 8>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
  else launch_one<MODE, 16>(a, x, wr, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
}

bool decode_fuses_shared(moe_act_mode mode, int T, int k, int H, int I, int Is) {
  return mode == MOE_A16 && decode_fusable(T, H, I) && single_launch(mode, T, k) && Is >= 32 &&
         Is <= kFusedShIs && Is % 32 == 0;
}

// Epochs of eager single-launch calls: 31 bits, not reused within 2^31 calls
// of the process, never 0 (the workspace starts at zero); device epochs (graph
// capture) have the top bit set.
static std::atomic<uint64_t> g_epoch{0};

moe_status launch_layer_decode(const moe_nvfp4_experts& w, moe_act_mode mode, int stage_mask,
                               const uint16_t* x, const uint16_t* w_router, const float* bias,
                               int T, int k, const uint16_t* residual, uint16_t* out,
                               int32_t* ids, float* tw, int32_t* offsets, int32_t* sorted,
                               int32_t* prow, float* y, float* logits, void* ffn_ws, void* state,
                               const float* shared_y, hipStream_t s, const moe_shared_expert* fuse_sw,
                               void* sh_h) {
  DecodeState* st = static_cast<DecodeState*>(state);
  const int E = w.E, H = w.H;
  moe_status r;
  if (stage_mask == 3 && single_launch(mode, T, k)) {
    // one launch; under graph capture, where a replay would repeat an epoch baked
    // into the launch, epoch 0 makes the kernel use and advance the workspace's
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return check_launch("moe_layer_forward (capture query)");
    {
      const FfnArgs a = make_ffn_args(w, mode, x, T, k, offsets, sorted, y, ffn_ws);
      SharedArgs sarg;
      const SharedArgs* sa = nullptr;
      if (fuse_sw) {   // (the caller checked decode_fuses_shared)
        sarg = make_shared_args(*fuse_sw, x, T, sh_h, const_cast<float*>(shared_y));
        sa = &sarg;
      }
      uint64_t epoch = 0;   // 0: read the device epoch
      if (cs == hipStreamCaptureStatusNone) {
        do epoch = ++g_epoch & 0x7FFFFFFFu; while (epoch == 0u);   // 0: a never-written entry
      }
      const float* shy = sa ? nullptr : shared_y;   // (fused: the combine polls the launch's own)
      if (mode == MOE_A8)
        launch_one_mode<MOE_A8>(a, x, w_router, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
      else
        launch_one_mode<MOE_A16>(a, x, w_router, bias, logits, ids, tw, prow, st, residual, out, epoch, shy, sa, s);
      return check_launch("moe_layer_forward (decode layer)");
    }
  }
  if (stage_mask & 1) {   // routing (8-bit mode: with x quantized per token; 4-bit x is quantized in the gate/up tiles)
    const FfnArgs q = make_ffn_args(w, mode, x, T, k, offsets, sorted, y, ffn_ws);
    uint8_t* xqc = mode == MOE_A8 ? const_cast<uint8_t*>(q.xq_codes) : nullptr;
    float* xqs = mode == MOE_A8 ? static_cast<float*>(const_cast<void*>(q.xq_scales)) : nullptr;
    if (E <= 64) launch_a<1>(x, w_router, bias, T, H, E, k, logits, ids, tw, offsets, sorted, prow, st, xqc, xqs, s);
    else if (E <= 128) launch_a<2>(x, w_router, bias, T, H, E, k, logits, ids, tw, offsets, sorted, prow, st, xqc, xqs, s);
    else if (E <= 256) launch_a<4>(x, w_router, bias, T, H, E, k, logits, ids, tw, offsets, sorted, prow, st, xqc, xqs, s);
    else if (E <= 512) launch_a<8>(x, w_router, bias, T, H, E, k, logits, ids, tw, offsets, sorted, prow, st, xqc, xqs, s);
    else launch_a<16>(x, w_router, bias, T, H, E, k, logits, ids, tw, offsets, sorted, prow, st, xqc, xqs, s);
    r = check_launch("moe_layer_forward (decode routing)");
    if (r != MOE_OK) return r;
  }
  if (stage_mask & 2) {   // experts and combine
    const FfnArgs a = make_ffn_args(w, mode, x, T, k, offsets, sorted, y, ffn_ws);
    const int P = T * k, max_slots = P < E ? P : E;
    switch ((int)mode) {   // (kModeQ4 is the library's internal mode of q4_g64_fp16 experts)
      case MOE_A16: launch_b<MOE_A16>(a, st, max_slots, prow, tw, residual, out, shared_y, s); break;
      case MOE_A8: launch_b<MOE_A8>(a, st, max_slots, prow, tw, residual, out, shared_y, s); break;
      case kModeQ4: launch_b<kModeQ4>(a, st, max_slots, prow, tw, residual, out, shared_y, s); break;
      default: launch_b<MOE_A4>(a, st, max_slots, prow, tw, residual, out, shared_y, s); break;
    }
    return check_launch("moe_layer_forward (decode experts)");
  }
  return MOE_OK;
}

}  // namespace moe
