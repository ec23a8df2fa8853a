// Wide expert path (4-bit activations): the grouped GEMM of a prefill chunk on
// the gfx950 matrix cores.
//
// Prior art (page "Inferno", section "Performance"; page "Infernix", section
// "Activation precision"): NVFP4 prefill runs on FP4 tensor-core MMA.  CDNA4's
// block-scaled FP4 MFMA applies one power-of-two scale per 32 elements, while
// NVFP4 carries an E4M3 scale per 16, so that instruction cannot take these
// operands without rounding them.  Instead both operands are expanded exactly
// to f16: an E2M1 value times an E4M3 scale has at most 6 significant bits and
// lies in [2^-10, 2688], which f16 holds exactly; products are exact in fp32 and
// v_mfma_f32_16x16x32_f16 accumulates them in fp32.  The layer is HBM-bound at
// these shapes (3.56 n_e FLOP per weight byte, n_e <= a few hundred), so the
// f16 matrix rate is ample.
//
// Tiles.  A workgroup (4 waves) serves one expert and 64 rows: gate/up takes
// 64 h rows (wave w: gate rows and up rows i0+16w .. +15, both accumulated, so
// SwiGLU and the 4-bit quantization of h happen in registers; 16 rows are one
// quantization block); down takes 64 output rows.  Tokens: up to 64 per pass
// (4 MFMA column tiles), more passes for hotter experts.  K steps of 128: each
// lane loads 16 bytes of codes (32 weights) and one 16-bit pair of E4M3 scales
// per row tile; the activations of the step are expanded to f16 once into LDS
// (row stride 272 B: 16 lanes reading 16 B at consecutive tokens hit distinct
// banks) and shared by the 4 waves.  The next step's weights and activation
// codes are in flight while the current step computes; several workgroups per
// CU (35 KB of LDS each) cover the rest of the latency.
#include <type_traits>

#include "ffn_common.hpp"

namespace moe {

constexpr int kXcds = 8;             // XCDs of the chip, each with its own L2
constexpr int kWideWaves = 4;
constexpr int kWideRows = 16 * kWideWaves;   // rows per workgroup
constexpr int kWideTok = 64;                 // tokens per pass
constexpr int kWideTiles = kWideTok / 16;
constexpr int kKStep = 128;                  // K per step
constexpr int kRowStride = kKStep * 2 + 16;  // bytes per token row of the f16 tile

// 8 E2M1 codes (one dword) times an E4M3 scale, as the f16x8 MFMA operand.
__device__ __forceinline__ f16x8 expand8(uint32_t codes, f16x2 s2) {
  const f16x2 a = e2m1x2_to_f16<0>(codes) * s2;
  const f16x2 b = e2m1x2_to_f16<1>(codes) * s2;
  const f16x2 c = e2m1x2_to_f16<2>(codes) * s2;
  const f16x2 d = e2m1x2_to_f16<3>(codes) * s2;
  return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Both E4M3 bytes of a 16-bit scale pair as f16 splats: .x = first, .y = second.
__device__ __forceinline__ void scale_pair(uint32_t sc, f16x2& s0, f16x2& s1) {
  const f16x2 p = e4m3x2_to_f16<false>(sc);   // bytes 0, 1 of sc
  s0 = f16x2{p.x, p.x};
  s1 = f16x2{p.y, p.y};
}

// Expand 32 activation codes + 2 scales into 32 f16 at dst (64 bytes of LDS).
__device__ __forceinline__ void stage32(uint8_t* dst, uint4 c, uint32_t sc) {
  f16x2 s0, s1;
  scale_pair(sc, s0, s1);
  const f16x8 v0 = expand8(c.x, s0), v1 = expand8(c.y, s0);
  const f16x8 v2 = expand8(c.z, s1), v3 = expand8(c.w, s1);
  uint4* d = reinterpret_cast<uint4*>(dst);
  d[0] = bitcast<uint4>(v0);
  d[1] = bitcast<uint4>(v1);
  d[2] = bitcast<uint4>(v2);
  d[3] = bitcast<uint4>(v3);
}

// Codes of one value under a decided NVFP4 block (d = dec(s) * g): as nvfp4_quant16.
__device__ __forceinline__ uint32_t e2m1_under(float v, float d) {
  return d > 0.0f ? f32_to_e2m1(__fdiv_rn(v, d)) : 0u;
}


// One K step of one 16-row weight tile, per lane: 32 codes (16 B) and their two
// E4M3 scales.  The same shape carries one token's 32 activation codes.
struct Frag {
  uint4 c;
  uint16_t s;   // widened where used, so no instruction touches it before then
};

// A stream of 32-wide pieces along K, read with buffer loads: the resources
// (base and size of a wave's region, in SGPRs) are wave-uniform, the lane's own
// byte offsets into its row are fixed, and the step's offset is a scalar, so a
// load costs no vector address arithmetic.  K is a multiple of 128 on this
// path, so every step's pieces lie inside their rows (loads past the last step
// re-read it); 0x00020000 is the raw-buffer format word of the gfx9 family.
struct Stream {
  __amdgpu_buffer_rsrc_t codes, scales;
  int vc, vs;   // this lane's byte offsets: codes, scales
};

__device__ __forceinline__ Stream make_stream(const uint8_t* codes, const uint8_t* scales, int rows,
                                              int K, int row, int piece) {
  Stream t;
  t.codes = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(codes), (short)0, rows * (K / 2),
                                              0x00020000);
  t.scales = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(scales), (short)0,
                                               rows * (K / 16), 0x00020000);
  t.vc = row * (K / 2) + 16 * piece;
  t.vs = row * (K / 16) + 2 * piece;
  return t;
}

__device__ __forceinline__ void load_frag(Frag& f, const Stream& t, int st) {
  f.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t.codes, t.vc, st * 64, 0));
  f.s = __builtin_amdgcn_raw_buffer_load_b16(t.scales, t.vs, st * 8, 0);
}

// The work plan: active experts, most tokens first (so the longest workgroups
// start first), each with its first sorted row and token count.  One
// workgroup, one thread per expert; the order is by the unique key
// (count, -index): count descending, ties by ascending index, counts clamped to
// 2^20 (the order stays a permutation).  Each wave broadcasts 64 keys at a time
// from one register with readlane, so the O(E^2) comparison costs a scalar read
// and a compare per pair.
__global__ void __launch_bounds__(1024) k_wide_plan(const int32_t* __restrict__ offsets, int E,
                                                    int4* __restrict__ plan) {
  __shared__ uint32_t key[kMaxExperts];
  const int e = threadIdx.x;
  const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
  const uint32_t mine = e < E ? ((uint32_t)min(c, (1 << 20) - 1) << 11) | (uint32_t)(2047 - e) : 0u;
  key[e] = mine;
  __syncthreads();
  const int nwave = (E + kWave - 1) / kWave;
  if (e >= nwave * kWave) return;   // whole waves past E
  int rank = 0;
  for (int w = 0; w < nwave; ++w) {
    const uint32_t v = key[w * kWave + lane_id()];    // 0 past E: never above a real key
#pragma unroll
    for (int j = 0; j < kWave; ++j) rank += (uint32_t)__builtin_amdgcn_readlane((int)v, j) > mine;
  }
  // empty experts sort last; their entries are marked unused
  if (e < E) plan[rank] = c > 0 ? make_int4(e, offsets[e], c, 0) : make_int4(-1, 0, 0, 0);
}

struct Job {
  int e, row0, ne, rb;
};

// Workgroup -> (row block, plan entry), XCD-aware.  Workgroups are handed to the
// 8 XCDs round-robin by linear index, and each XCD has its own L2.  All row
// blocks of one plan entry share that expert's activations, so they are given
// to one XCD: XCD x runs entries x, x+8, x+16, ... (heaviest first), each entry's
// nrb row blocks back to back.  The grid is padded to whole groups of 8 entries;
// padding workgroups get entry -1.
__device__ __forceinline__ Job wide_job(const int4* plan, int nrb, int slots) {
  const int L = blockIdx.x;
  const int x = L % kXcds, j = L / kXcds;
  const int slot = (j / nrb) * kXcds + x;
  Job jb{-1, 0, 0, j % nrb};
  if (slot < slots) {
    const int4 p = plan[slot];
    jb.e = p.x;
    jb.row0 = p.y;
    jb.ne = p.z;
  }
  return jb;
}

// ------------------------------------------------------------------ main loop
// NM weight matrices (gate/up: 2, down: 1) against the activations of up to 64
// tokens of one expert, K = the reduction length.  Wave w takes 16 rows of
// matrix w / 4; its 4 accumulator tiles are the 64 token columns.
//
// Pipeline: a lane's weight and activation fragments for step s + kDepth are
// issued at step s into one of kDepth + 1 register sets; the step loop is
// unrolled by kDepth + 1 so that every set keeps its registers (no copies,
// which would force a wait on the load).  The activation fragments of step s
// are expanded to f16 into one of two LDS buffers; one barrier per step
// separates that write from the MFMAs that read it, and the buffer written at
// step s was last read at step s - 2, before the barrier of step s - 1.
constexpr int kDepth = 2;
constexpr int kSets = kDepth + 1;

template <int NM>
struct WideLds {
  static constexpr int kBuf = NM * kWideTok * kRowStride;   // one buffer: [NM][token][k] f16
  __align__(16) uint8_t bt[2 * kBuf];
};

template <int NM, int NT>
__device__ __forceinline__ void wide_mainloop_t(const Stream& ws, const Stream& xs, int K,
                                                uint8_t* bt, f32x4 (&acc)[kWideTiles]) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int m = wave / 4;
  // staging item of this thread: (matrix sm, token sn, 32-wide piece sq)
  const int sm = threadIdx.x / (kWideTok * 4), sn = (threadIdx.x / 4) % kWideTok, sq = threadIdx.x % 4;
  const int nsteps = K / kKStep;
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  Frag w[kSets], x[kSets];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) {
    load_frag(w[d], ws, min(d, nsteps - 1));
    load_frag(x[d], xs, min(d, nsteps - 1));
  }
  // One step with the fragments of register set U.  Loads past the last step
  // re-read the last piece (in cache, never used), so the steady-state body has
  // no branch around a load: the wait counters then see a fixed issue order.
  auto step = [&](int st, auto U) {
    constexpr int u = decltype(U)::value;
    constexpr int nx = (u + kDepth) % kSets;
    const int ld = min(st + kDepth, nsteps - 1);
    load_frag(x[nx], xs, ld);
    load_frag(w[nx], ws, ld);
    uint8_t* buf = bt + (st & 1) * WideLds<NM>::kBuf;
    stage32(buf + (sm * kWideTok + sn) * kRowStride + 64 * sq, x[u].c, x[u].s);
    __syncthreads();
    f16x2 s0v, s1v;
    scale_pair(w[u].s, s0v, s1v);
    const uint32_t ww[4] = {w[u].c.x, w[u].c.y, w[u].c.z, w[u].c.w};
    f16x8 av[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) av[j] = expand8(ww[j], j < 2 ? s0v : s1v);
    const uint8_t* bm = buf + m * kWideTok * kRowStride;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int off = (t * 16 + r) * kRowStride + 64 * g + 16 * j;
        const f16x8 bv = bitcast<f16x8>(*reinterpret_cast<const uint4*>(bm + off));
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[j], bv, acc[t], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep each tile's B loads with its MFMAs
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  static_assert(kSets == 3, "the unrolled body below names three register sets");
  int s0 = 0;
  for (; s0 + kSets <= nsteps; s0 += kSets) {
    step(s0, I0{});
    step(s0 + 1, I1{});
    step(s0 + 2, I2{});
  }
  if (s0 < nsteps) step(s0, I0{});
  if (s0 + 1 < nsteps) step(s0 + 1, I1{});
}

// The main loop specialised on the number of 16-token column tiles in use, so
// the steady-state body is straight-line code.
template <int NM>
__device__ __forceinline__ void wide_mainloop(const Stream& ws, const Stream& xs, int K, int ntt,
                                              uint8_t* bt, f32x4 (&acc)[kWideTiles]) {
  switch (ntt) {
    case 1: wide_mainloop_t<NM, 1>(ws, xs, K, bt, acc); break;
    case 2: wide_mainloop_t<NM, 2>(ws, xs, K, bt, acc); break;
    case 3: wide_mainloop_t<NM, 3>(ws, xs, K, bt, acc); break;
    default: wide_mainloop_t<NM, 4>(ws, xs, K, bt, acc); break;
  }
}

// ------------------------------------------------------------------ gate/up + SwiGLU + h
// Workgroup: one expert, 64 h rows; waves 0-3 the gate rows i0+16w .. +15, waves
// 4-7 the matching up rows.  After the K loop the gate waves hand g through
// LDS to the up waves, which form h, quantize it and store it.  Rows of a
// ragged last row block and token slots past the expert's count read clamped
// (valid) addresses; their results are never stored.
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4, 4))) k_gateup_wide_a4(FfnArgs a, const int4* __restrict__ plan,
                                                        int slots) {
  __shared__ WideLds<2> lds;
  const Job job = wide_job(plan, (a.I + kWideRows - 1) / kWideRows, slots);
  if (job.e < 0) return;
  const int e = job.e, row0 = job.row0, ne = job.ne;
  const int H = a.H, I = a.I;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int m = wave >> 2;                                  // 0 gate, 1 up
  const int i0 = job.rb * kWideRows + (wave & 3) * 16;      // this wave's h rows
  const bool on = i0 < I;
  const size_t row16 = (size_t)e * 2 * I + (size_t)m * I + (on ? i0 : I - 16);   // wave's first row
  const Stream ws = make_stream(a.gu_codes + row16 * (H / 2), a.gu_scales + row16 * (H / 16), 16, H,
                                r, g);
  const float fm = a.gu_wscale[2 * e + m] * a.gu_inscale[2 * e + m];
  const int sm = threadIdx.x / (kWideTok * 4), sn = (threadIdx.x / 4) % kWideTok, sq = threadIdx.x % 4;
  float* gbuf = reinterpret_cast<float*>(lds.bt);           // [64 h rows][64 tokens] after the K loop

  for (int p0 = 0; p0 < ne; p0 += kWideTok) {
    const int np = min(kWideTok, ne - p0);
    const int ntt = (np + 15) / 16;
    const size_t xr0 = (size_t)(row0 + p0) * 2;             // the pass's first activation row
    const Stream xs = make_stream(a.xq_codes + xr0 * (H / 2),
                                  static_cast<const uint8_t*>(a.xq_scales) + xr0 * (H / 16), 2 * np, H,
                                  min(sn, np - 1) * 2 + sm, sq);
    f32x4 acc[kWideTiles];
    wide_mainloop<2>(ws, xs, H, ntt, lds.bt, acc);
    __syncthreads();                       // every wave is done with the LDS tiles
    if (m == 0 && on) {
#pragma unroll
      for (int t = 0; t < kWideTiles; ++t)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          gbuf[((wave & 3) * 16 + 4 * g + q) * kWideTok + t * 16 + r] = acc[t][q] * fm;
    }
    __syncthreads();
    if (m == 1 && on) {
      const float gdn = a.dn_inscale[e];
#pragma unroll
      for (int t = 0; t < kWideTiles; ++t) {
        if (t >= ntt) continue;
        float h[4];
        float am = 0.0f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gv = gbuf[((wave & 3) * 16 + 4 * g + q) * kWideTok + t * 16 + r];
          h[q] = swiglu(gv, acc[t][q] * fm);
          am = __builtin_fmaxf(am, __builtin_fabsf(h[q]));
        }
        am = __builtin_fmaxf(am, __shfl_xor(am, 16, kWave));
        am = __builtin_fmaxf(am, __shfl_xor(am, 32, kWave));
        const uint32_t sc = f32_to_e4m3(__fdiv_rn(__fdiv_rn(am, 6.0f), gdn));
        const float d = __fmul_rn(e4m3_to_f32(sc), gdn);
        uint32_t nib = 0u;
#pragma unroll
        for (int q = 0; q < 4; ++q) nib |= e2m1_under(h[q], d) << (4 * q);
        const int n = t * 16 + r;
        if (n < np) {
          const size_t row = (size_t)(row0 + p0 + n);
          *reinterpret_cast<uint16_t*>(a.h_codes + row * (I / 2) + i0 / 2 + 2 * g) = (uint16_t)nib;
          if (g == 0) static_cast<uint8_t*>(a.h_scales)[row * (I / 16) + i0 / 16] = (uint8_t)sc;
        }
      }
    }
    __syncthreads();                       // gbuf is read before the next pass stages
  }
}

// ------------------------------------------------------------------ down
// Workgroup: one expert, 64 output rows (wave w: rows o0+16w .. +15).
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) k_down_wide_a4(FfnArgs a, const int4* __restrict__ plan,
                                                      int slots) {
  __shared__ WideLds<1> lds;
  const Job job = wide_job(plan, (a.H + kWideRows - 1) / kWideRows, slots);
  if (job.e < 0) return;
  const int e = job.e, row0 = job.row0, ne = job.ne;
  const int H = a.H, I = a.I;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int o0 = job.rb * kWideRows + wave * 16;           // this wave's output rows
  const bool on = o0 < H;
  const size_t row16 = (size_t)e * H + (on ? o0 : H - 16);   // wave's first row
  const Stream ws = make_stream(a.dn_codes + row16 * (I / 2), a.dn_scales + row16 * (I / 16), 16, I,
                                r, g);
  const float f = a.dn_wscale[e] * a.dn_inscale[e];
  const int sn = threadIdx.x / 4, sq = threadIdx.x % 4;

  for (int p0 = 0; p0 < ne; p0 += kWideTok) {
    const int np = min(kWideTok, ne - p0);
    const int ntt = (np + 15) / 16;
    const size_t hr0 = (size_t)(row0 + p0);
    const Stream xs = make_stream(a.h_codes + hr0 * (I / 2),
                                  static_cast<const uint8_t*>(a.h_scales) + hr0 * (I / 16), np, I,
                                  min(sn, np - 1), sq);
    f32x4 acc[kWideTiles];
    wide_mainloop<1>(ws, xs, I, ntt, lds.bt, acc);
    if (on) {
#pragma unroll
      for (int t = 0; t < kWideTiles; ++t) {
        const int n = t * 16 + r;
        if (t < ntt && n < np) {
          float4 o = make_float4(acc[t][0] * f, acc[t][1] * f, acc[t][2] * f, acc[t][3] * f);
          *reinterpret_cast<float4*>(a.y + (size_t)(row0 + p0 + n) * H + o0 + 4 * g) = o;
        }
      }
    }
    __syncthreads();                       // LDS buffers are free before the next pass stages
  }
}

// Grid of the XCD-aware mapping: whole groups of 8 plan entries, nrb row blocks each.
static unsigned wide_grid(int slots, int nrb) {
  return (unsigned)(((slots + kXcds - 1) / kXcds) * kXcds * nrb);
}

moe_status launch_ffn_wide_a4(const FfnArgs& a, int slots, int stage_mask, void* plan_ws,
                              hipStream_t s) {
  int4* plan = static_cast<int4*>(plan_ws);
  if (stage_mask & 6) {
    hipLaunchKernelGGL(k_wide_plan, dim3(1), dim3(1024), 0, s, a.offsets, a.E, plan);
    moe_status st = check_launch("nvfp4_expert_ffn (wide plan)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 2) {
    const int nrb = (a.I + kWideRows - 1) / kWideRows;
    hipLaunchKernelGGL(k_gateup_wide_a4, dim3(wide_grid(slots, nrb)), dim3(512), 0, s, a, plan, slots);
    moe_status st = check_launch("nvfp4_expert_ffn (wide gate/up)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 4) {
    const int nrb = (a.H + kWideRows - 1) / kWideRows;
    hipLaunchKernelGGL(k_down_wide_a4, dim3(wide_grid(slots, nrb)), dim3(256), 0, s, a, plan, slots);
    return check_launch("nvfp4_expert_ffn (wide down)");
  }
  return MOE_OK;
}

}  // namespace moe
