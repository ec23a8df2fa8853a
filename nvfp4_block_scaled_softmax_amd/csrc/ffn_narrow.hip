// Narrow expert path: each expert's few token columns against its NVFP4 rows.
//
// Prior art (page "Infernix releases", release 2026.10.11, "Highlights"):
// calls of up to eight columns run on one-column expert kernels that expand
// FP4 in one instruction and keep the products exact; the down pass is
// chained on gate/up.  Here, for gfx950:
//   * the weight stream is read with 128-bit loads (32 E2M1 codes per lane),
//     the two E4M3 block scales of that chunk with one 16-bit load, all of a
//     lane's chunks issued before any is used;
//   * codes expand with v_cvt_scalef32_pk_{bf16,f16}_fp4 and meet the
//     activations in v_dot2 instructions (bf16 x for 16-bit mode, E4M3 or
//     E2M1 codes for 8/4-bit mode, where the 16-element block sums are exact);
//   * activations sit in LDS in a bank-conflict-free padded layout; a lane
//     reads only the chunks it owns;
//   * gate and up rows of the same h index live in the two halves of a wave,
//     so SwiGLU and the intermediate's rounding/quantization happen in the
//     gate/up kernel's epilogue; down follows on the same stream.
// A workgroup serves one active expert (found from the offsets on the device,
// so nothing returns to the host) and a tile of rows; it loops over the
// expert's columns in LDS-sized groups, its weights staying in registers.
#include "ffn_narrow.hpp"

namespace moe {

// ------------------------------------------------------------------ kernels
// grid (I / 16, active-expert slots) and (ceil(H / 64), slots): a workgroup
// finds its active expert from the offsets, then runs one tile.
__device__ __forceinline__ bool slot_expert(const FfnArgs& a, int* s_info) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  if (wave == 0) {
    const int e = find_active_expert(a.offsets, a.E, blockIdx.y);
    if (lane == 0) {
      s_info[0] = e;
      s_info[1] = e >= 0 ? a.offsets[e] : 0;
      s_info[2] = e >= 0 ? a.offsets[e + 1] - a.offsets[e] : 0;
    }
  }
  __syncthreads();
  return s_info[0] >= 0;
}

template <int MODE, int LPR, int CPL>
__global__ void __launch_bounds__(kTileThreads) k_gateup_narrow(FfnArgs a, int max_cols) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_info[3];
  if (!slot_expert(a, s_info)) return;
  gateup_tile<MODE, LPR, CPL>(a, s_info[0], s_info[1], s_info[2], blockIdx.x, max_cols, lds);
}

template <int MODE, int LPR, int CPL>
__global__ void __launch_bounds__(kTileThreads) k_down_narrow(FfnArgs a, int max_cols) {
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int s_info[3];
  if (!slot_expert(a, s_info)) return;
  down_tile<MODE, LPR, CPL, false>(a, s_info[0], s_info[1], s_info[2], blockIdx.x, max_cols, lds,
                                   NoHook{});
}

// The product core alone (moe_debug_nvfp4_matmul): the down tile over one
// matrix of N = a.H rows and K = a.I, its T columns from the intermediate's
// workspace slots (h_codes / h_scales), no plan and no SwiGLU.
template <int MODE, int LPR, int CPL>
__global__ void __launch_bounds__(kTileThreads) k_debug_narrow(FfnArgs a, int max_cols) {
  extern __shared__ __align__(16) uint8_t lds[];
  down_tile<MODE, LPR, CPL, false>(a, 0, 0, a.T, blockIdx.x, max_cols, lds, NoHook{});
}

// ------------------------------------------------------------------ launch
template <int MODE, int LPR, int CPL>
static void launch_gu(const FfnArgs& a, int slots, int max_cols, hipStream_t s) {
  const size_t lds = (size_t)max_cols * (a.H / 32) * ChunkLds<MODE>::kStride;
  hipLaunchKernelGGL((k_gateup_narrow<MODE, LPR, CPL>), dim3(a.I / kGuRows, slots), dim3(kTileThreads), lds,
                     s, a, max_cols);
}
template <int MODE, int LPR, int CPL>
static void launch_dn(const FfnArgs& a, int slots, int max_cols, hipStream_t s) {
  const size_t lds = (size_t)max_cols * (a.I / 32) * ChunkLds<MODE>::kStride;
  hipLaunchKernelGGL((k_down_narrow<MODE, LPR, CPL>), dim3((a.H + kDnRows - 1) / kDnRows, slots),
                     dim3(kTileThreads), lds, s, a, max_cols);
}

// Lanes per row and chunks per lane for a reduction length K (K % 32 == 0, K <= 4096).
template <int MODE, bool GU>
static void dispatch(const FfnArgs& a, int K, int slots, int max_cols, hipStream_t s) {
  const int NC = K / 32;
#define GO(LPR, CPL) \
  (GU ? launch_gu<MODE, LPR, CPL>(a, slots, max_cols, s) : launch_dn<MODE, LPR, CPL>(a, slots, max_cols, s))
  if (NC <= 4) GO(4, 1);
  else if (NC <= 8) GO(8, 1);
  else if (NC <= 16) GO(16, 1);
  else if (NC <= 32) GO(32, 1);
  else if (NC <= 64) GO(32, 2);
  else if (NC <= 96) GO(32, 3);
  else GO(32, 4);
#undef GO
}

template <int MODE>
static moe_status run(const FfnArgs& a, int slots, int stage_mask, hipStream_t s) {
  const int per_col_gu = (a.H / 32) * ChunkLds<MODE>::kStride;
  const int per_col_dn = (a.I / 32) * ChunkLds<MODE>::kStride;
  // an expert has at most T columns; LDS is sized for what a call can need
  const int cols_gu = max(1, min(min(8, a.T), kLdsBudget / per_col_gu));
  const int cols_dn = max(1, min(min(8, a.T), kLdsBudget / per_col_dn));
  if (stage_mask & 2) {
    dispatch<MODE, true>(a, a.H, slots, cols_gu, s);
    moe_status st = check_launch("nvfp4_expert_ffn (gate/up)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 4) {
    dispatch<MODE, false>(a, a.I, slots, cols_dn, s);
    return check_launch("nvfp4_expert_ffn (down)");
  }
  return MOE_OK;
}

template <int MODE, int LPR, int CPL>
static void launch_dbg(const FfnArgs& a, int max_cols, hipStream_t s) {
  const size_t lds = (size_t)max_cols * (a.I / 32) * ChunkLds<MODE>::kStride;
  hipLaunchKernelGGL((k_debug_narrow<MODE, LPR, CPL>), dim3((a.H + kDnRows - 1) / kDnRows), dim3(kTileThreads),
                     lds, s, a, max_cols);
}

template <int MODE>
static moe_status run_debug(const FfnArgs& a, hipStream_t s) {
  const int per_col = (a.I / 32) * ChunkLds<MODE>::kStride;
  const int cols = max(1, min(min(8, a.T), kLdsBudget / per_col));
  const int NC = a.I / 32;
  // the lanes-per-row / chunks-per-lane choice of the per-stage kernels
  if (NC <= 4) launch_dbg<MODE, 4, 1>(a, cols, s);
  else if (NC <= 8) launch_dbg<MODE, 8, 1>(a, cols, s);
  else if (NC <= 16) launch_dbg<MODE, 16, 1>(a, cols, s);
  else if (NC <= 32) launch_dbg<MODE, 32, 1>(a, cols, s);
  else if (NC <= 64) launch_dbg<MODE, 32, 2>(a, cols, s);
  else if (NC <= 96) launch_dbg<MODE, 32, 3>(a, cols, s);
  else launch_dbg<MODE, 32, 4>(a, cols, s);
  return check_launch("moe_debug_nvfp4_matmul (narrow)");
}

moe_status launch_debug_narrow(const FfnArgs& a, moe_act_mode mode, hipStream_t s) {
  switch ((int)mode) {
    case MOE_A16: return run_debug<MOE_A16>(a, s);
    case MOE_A8: return run_debug<MOE_A8>(a, s);
    case kModeQ4: return run_debug<kModeQ4>(a, s);
    default: return run_debug<MOE_A4>(a, s);
  }
}

moe_status launch_ffn_narrow(const FfnArgs& a, moe_act_mode mode, int slots, int stage_mask,
                             hipStream_t s) {
  switch ((int)mode) {
    case MOE_A16: return run<MOE_A16>(a, slots, stage_mask, s);
    case MOE_A8: return run<MOE_A8>(a, slots, stage_mask, s);
    case kModeQ4: return run<kModeQ4>(a, slots, stage_mask, s);
    default: return run<MOE_A4>(a, slots, stage_mask, s);
  }
}

}  // namespace moe
