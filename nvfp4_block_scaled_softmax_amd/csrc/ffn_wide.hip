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
// Work.  The plan lists chunks of at most 32 tokens of one expert; each
// workgroup computes one chunk against a block of weight rows (gate/up: 64 h
// rows, down: kDownRows output rows), so hot experts spread over many
// workgroups and every workgroup streams its weight rows once.  A wave owns 16
// weight rows (gate/up: waves 0-3 gate rows, 4-7 the matching up rows; down:
// kDownWaves waves of output rows) and up to two 16-token MFMA column tiles.
//
// K loop.  Steps of 128: per step a lane loads 16 bytes of codes (32 values)
// and their two E4M3 scales for its weight row, and the same for its token of
// each column tile, straight into registers (buffer loads: wave-uniform
// resources, fixed lane offsets, a scalar step offset).  Weights and tokens are
// expanded the same way and feed 4 MFMAs per tile.  There is no LDS and no
// barrier in the loop: each wave runs ahead on its own, with the fragments of
// the next two steps in flight.  Gate and up meet in LDS once, after the loop,
// to form SwiGLU, quantize h (16 rows are one block) and store it.
#include <type_traits>

#include "ffn_common.hpp"

namespace moe {

constexpr int kXcds = 8;                     // XCDs of the chip, each with its own L2
constexpr int kWideRows = 64;                // weight rows per gate/up workgroup
// Down: K is only I, so a workgroup's fixed costs (plan, staging the chunk's
// activations, pipeline fill) weigh more; it takes 16 output rows per wave
// over kDownWaves waves to spread them over more weight bytes.
constexpr int kDownWaves = 8;
constexpr int kDownRows = 16 * kDownWaves;
constexpr int kWideTok = 32;                 // tokens per chunk
constexpr int kWideTiles = kWideTok / 16;    // MFMA column tiles per chunk
constexpr int kKStep = 128;                  // K per step

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

// Codes of one value under a decided NVFP4 block (d = dec(s) * g): as nvfp4_quant16.
__device__ __forceinline__ uint32_t e2m1_under(float v, float d) {
  return d > 0.0f ? f32_to_e2m1(__fdiv_rn(v, d)) : 0u;
}

// 32 consecutive K values of one row: 16 bytes of codes, two E4M3 scales.
struct Frag {
  uint4 c;
  uint16_t s;   // widened where used, so no instruction touches it before then
};

// Buffer resource over [base, base + bytes); 0x00020000 is the raw-buffer
// format word of the gfx9 family.  Every offset used below stays inside.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Rows of NVFP4 pieces along K: codes [rows][K/2], scales [rows][K/16].  A lane
// reads piece g (32 values) of step st of its row: code offset row*K/2 + 16g +
// 64st, scale offset row*K/16 + 2g + 8st; the step part is a scalar.
struct Rows {
  __amdgpu_buffer_rsrc_t codes, scales;
};

__device__ __forceinline__ Rows make_rows(const uint8_t* codes, const uint8_t* scales, int rows,
                                          int K) {
  return Rows{rsrc(codes, rows * (K / 2)), rsrc(scales, rows * (K / 16))};
}

// A lane's 32 weight codes of step st (16 bytes of its row).
__device__ __forceinline__ uint4 load_wcodes(const Rows& t, int vc, int st) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t.codes, vc, st * 64, 0));
}

// Weight scales come in windows of 8 steps: row r has 8 scale bytes per step,
// 64 per window; lane (r, g) loads bytes 16g .. 16g+15 of its row's window p
// (steps 8p + 2g and 8p + 2g + 1), one 16-byte load per 8 steps instead of a
// 2-byte load per step.  Past the end of a row the load reads the next row
// (unused); past the wave's region the buffer returns zeros.
__device__ __forceinline__ uint4 load_wscales(const Rows& t, int vs_row, int g, int p) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(t.scales, vs_row + 64 * p + 16 * g, 0, 0));
}

// The two scale bytes of lane (r, g) for step i (0..7) of the window held in
// sw: they sit in lane r + 16 (i / 2), dword 2 (i % 2) + g / 2, half g % 2.
template <int I>
__device__ __forceinline__ uint32_t window_scales(const uint4& sw, int lane) {
  const int src = (lane & 15) + 16 * (I / 2);
  const uint32_t lo = __shfl(I % 2 ? sw.z : sw.x, src, kWave);
  const uint32_t hi = __shfl(I % 2 ? sw.w : sw.y, src, kWave);
  const int g = lane >> 4;
  const uint32_t d = g < 2 ? lo : hi;
  return (g & 1) ? d >> 16 : d & 0xFFFFu;
}

__device__ __forceinline__ void expand_frag(const uint4& c, uint32_t sc, f16x8 (&v)[4]) {
  f16x2 s0, s1;
  scale_pair(sc, s0, s1);
  v[0] = expand8(c.x, s0);
  v[1] = expand8(c.y, s0);
  v[2] = expand8(c.z, s1);
  v[3] = expand8(c.w, s1);
}

// ------------------------------------------------------------------ plan
// The work plan: every active expert's tokens cut into chunks of at most 32, in
// expert order, as (expert, first sorted row, rows).  One workgroup, one thread
// per expert: chunk counts, a block-wide exclusive scan, then each expert
// writes its entries; entries past the total, up to n_entries, are marked unused.
__global__ void __launch_bounds__(1024) k_wide_plan(const int32_t* __restrict__ offsets, int E,
                                                    int n_entries, int4* __restrict__ plan) {
  __shared__ int wsum[1024 / kWave];
  __shared__ int total;
  const int e = threadIdx.x;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int c = e < E ? (offsets[e + 1] - offsets[e] + kWideTok - 1) / kWideTok : 0;
  int incl = c;                                   // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int v = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += v;
  }
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int v = 0; v < wave; ++v) before += wsum[v];
  if (e == (int)blockDim.x - 1) total = before + incl;
  if (c > 0) {
    const int first = before + incl - c;
    const int r0 = offsets[e], n = offsets[e + 1] - r0;
    for (int j = 0; j < c; ++j)
      plan[first + j] = make_int4(e, r0 + j * kWideTok, min(kWideTok, n - j * kWideTok), 0);
  }
  __syncthreads();
  for (int i = total + threadIdx.x; i < n_entries; i += blockDim.x) plan[i] = make_int4(-1, 0, 0, 0);
}

struct Job {
  int e, row0, ne, rb;
};

// Workgroup -> (row block, plan entry), XCD-aware.  Workgroups are handed to the
// 8 XCDs round-robin by linear index, and each XCD has its own L2.  All row
// blocks of one plan entry share its activations, so they are given to one
// XCD: XCD x runs entries x, x+8, x+16, ..., each entry's nrb row blocks back
// to back.  The grid is padded to whole groups of 8 entries; padding
// workgroups get entry -1.
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
// A wave owns 16 weight rows (lane row r = lane % 16, piece g = lane / 16) and
// NT 16-token column tiles.  MFMA j of a step takes K values 32g + 8j .. +7 of
// the step in both operands (a K permutation that A and B share), so the A
// operand is one dword of the lane's weight fragment and the B operand one
// 16-byte LDS read.
//
// Activations: the chunk's tokens are expanded to f16 once per workgroup, 256
// K values at a time, into one of two LDS buffers (row stride 528 B: 16 lanes
// reading 16 B at consecutive tokens hit distinct banks).  One barrier per 256
// K separates a buffer's writes from its reads; the buffer written during
// chunk c (for chunk c + 1) was last read during chunk c - 1, before the
// barrier that ended it.  Raw activation codes are loaded two chunks ahead.
//
// Weights: each wave streams its own rows, three 128-K steps ahead, in four
// register sets; the loop body (two chunks, four steps) names each set at a
// fixed position, so no register copies force a wait on a load.  Loads past
// the end re-read the last step or chunk (in cache, never used), so no branch
// sits around a load and the wait counters see a fixed issue order.
constexpr int kChunkK = 256;                   // K per LDS chunk (two steps)
constexpr int kTokStride = kChunkK * 2 + 16;   // bytes per token row of an LDS chunk
constexpr int kWSets = 4;                      // weight register sets (three steps ahead)
// Loop body: one window of weight scales (8 steps), which is also whole chunk
// pairs (LDS buffers and raw sets alternate per chunk) and whole rounds of the
// weight sets.
constexpr int kBody = 8;
static_assert(kBody % kWSets == 0 && kBody % 4 == 0, "loop body");

// f(integral_constant<int, I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <int NM>
struct WideLds {
  static constexpr int kBuf = NM * kWideTok * kTokStride;   // [NM][token][k] f16
  __align__(16) uint8_t buf[2 * kBuf];
};

// One thread's share of staging: matrix sm, token sn, 32-wide piece sq of a chunk.
struct Stager {
  int sm, sn, sq;
  int vc, vs;       // byte offsets of the thread's token row (codes, scales)
  int K;
  bool on;          // the token belongs to a computed column tile
};

__device__ __forceinline__ void load_chunk(Frag& f, const Rows& x, const Stager& sg, int c) {
  const int kc = min(c * (kChunkK / 2) + 16 * sg.sq, sg.K / 2 - 16);   // clamped into the row
  const int ks = min(c * (kChunkK / 16) + 2 * sg.sq, sg.K / 16 - 2);
  f.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x.codes, sg.vc + kc, 0, 0));
  f.s = __builtin_amdgcn_raw_buffer_load_b16(x.scales, sg.vs + ks, 0, 0);
}

__device__ __forceinline__ void stage_chunk(uint8_t* buf, const Frag& f, const Stager& sg) {
  if (!sg.on) return;
  f16x2 s0, s1;
  scale_pair(f.s, s0, s1);
  uint4* d = reinterpret_cast<uint4*>(buf + (sg.sm * kWideTok + sg.sn) * kTokStride + 64 * sg.sq);
  d[0] = bitcast<uint4>(expand8(f.c.x, s0));
  d[1] = bitcast<uint4>(expand8(f.c.y, s0));
  d[2] = bitcast<uint4>(expand8(f.c.z, s1));
  d[3] = bitcast<uint4>(expand8(f.c.w, s1));
}

// w: the wave's 16 weight rows, lane offsets wc/ws; x: the chunk's activation
// rows; m: the wave's matrix (which LDS plane its B operands come from).
template <int NM, int NT>
__device__ __forceinline__ void wide_mainloop(const Rows& w, int wc, int ws_row, const Rows& x,
                                              const Stager& sg, int m, int K, WideLds<NM>& lds,
                                              f32x4 (&acc)[kWideTiles]) {
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int nsteps = K / kKStep, nchunks = (nsteps + 1) / 2;
  const int nwin = (nsteps + kBody - 1) / kBody;
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 fw[kWSets];
  Frag fx[2];
  load_chunk(fx[0], x, sg, 0);
  load_chunk(fx[1], x, sg, min(1, nchunks - 1));
  uint4 sw = load_wscales(w, ws_row, g, 0), swn;
#pragma unroll
  for (int d = 0; d < kWSets - 1; ++d) fw[d] = load_wcodes(w, wc, min(d, nsteps - 1));
  stage_chunk(lds.buf, fx[0], sg);
  __syncthreads();

  // step s = s0 + u of the body (one scale window): chunk s / 2, LDS buffer and
  // raw set (u / 2) % 2, weight set u % kWSets
  auto step = [&](int s0, auto U) {
    constexpr int u = decltype(U)::value;
    constexpr int cb = (u / 2) % 2;
    const int s = s0 + u;
    if constexpr (u == 0) swn = load_wscales(w, ws_row, g, min(s0 / kBody + 1, nwin - 1));
    if constexpr (u % 2 == 0)   // first step of a chunk: raw codes of the chunk after next
      load_chunk(fx[cb], x, sg, min(s / 2 + 2, nchunks - 1));
    fw[(u + kWSets - 1) % kWSets] = load_wcodes(w, wc, min(s + kWSets - 1, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);   // the loads go out before the compute below
    if (s < nsteps) {
      f16x8 av[4];
      expand_frag(fw[u % kWSets], window_scales<u>(sw, lane), av);
      const uint8_t* bm = lds.buf + cb * WideLds<NM>::kBuf + m * kWideTok * kTokStride +
                          (u % 2) * (kKStep * 2) + 64 * g;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x8 bv =
              bitcast<f16x8>(*reinterpret_cast<const uint4*>(bm + (16 * t + r) * kTokStride + 16 * j));
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[j], bv, acc[t], 0, 0, 0);
        }
      }
    }
    if constexpr (u % 2 == 1) {   // last step of a chunk: stage the next chunk, then sync
      stage_chunk(lds.buf + (cb ^ 1) * WideLds<NM>::kBuf, fx[cb ^ 1], sg);
      __syncthreads();
    }
    if constexpr (u == kBody - 1) sw = swn;   // issued 8 steps ago
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int s0 = 0; s0 < nsteps; s0 += kBody)
    static_for<0, kBody>([&](auto U) { step(s0, U); });
}

// f(integral_constant<int, NT>) with NT = the number of column tiles in use.
template <typename F>
__device__ __forceinline__ void by_tiles(int ntt, F&& f) {
  if (ntt <= 1)
    f(std::integral_constant<int, 1>{});
  else
    f(std::integral_constant<int, 2>{});
}

// Staging share of thread tid for a chunk of np tokens (ntt tiles computed) in
// NM matrices; activation row of (token, matrix) = token * NM + matrix.
template <int NM>
__device__ __forceinline__ Stager make_stager(int np, int ntt, int K) {
  Stager sg;
  sg.sm = threadIdx.x / (kWideTok * 8);
  sg.sn = (threadIdx.x / 8) % kWideTok;
  sg.sq = threadIdx.x % 8;
  const int row = min(sg.sn, np - 1) * NM + min(sg.sm, NM - 1);
  sg.vc = row * (K / 2);
  sg.vs = row * (K / 16);
  sg.K = K;
  sg.on = sg.sn < 16 * ntt && sg.sm < NM;   // threads past NM planes only wait at the barriers
  return sg;
}

// ------------------------------------------------------------------ gate/up + SwiGLU + h
// Workgroup: one chunk, 64 h rows i0 .. i0+63; wave w < 4: gate rows i0+16w ..
// +15, wave w >= 4: the same up rows.  Rows past I (a ragged last row block)
// read clamped rows and store nothing.
__global__ void __launch_bounds__(512) k_gateup_wide_a4(FfnArgs a, const int4* __restrict__ plan,
                                                        int slots) {
  __shared__ WideLds<2> lds;
  __shared__ float gbuf[kWideRows][kWideTok];   // gate * its multipliers, [h row][token]
  const Job job = wide_job(plan, (a.I + kWideRows - 1) / kWideRows, slots);
  if (job.e < 0) return;
  const int e = job.e, row0 = job.row0, np = job.ne;
  const int H = a.H, I = a.I;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int m = wave >> 2;                                  // 0 gate, 1 up
  const int wr = (wave & 3) * 16;                           // wave's rows within the block
  const int i0 = job.rb * kWideRows + wr;                   // this wave's h rows
  const bool on = i0 < I;
  const size_t row16 = (size_t)e * 2 * I + (size_t)m * I + (on ? i0 : I - 16);
  const Rows w = make_rows(a.gu_codes + row16 * (H / 2), a.gu_scales + row16 * (H / 16), 16, H);
  const size_t xr0 = (size_t)row0 * 2;                      // the chunk's first activation row
  const Rows x = make_rows(a.xq_codes + xr0 * (H / 2),
                           static_cast<const uint8_t*>(a.xq_scales) + xr0 * (H / 16), 2 * np, H);
  const int ntt = (np + 15) / 16;
  const Stager sg = make_stager<2>(np, ntt, H);
  f32x4 acc[kWideTiles];
  by_tiles(ntt, [&](auto NT) {
    wide_mainloop<2, decltype(NT)::value>(w, r * (H / 2) + 16 * g, r * (H / 16), x, sg, m,
                                          H, lds, acc);
  });
  const float fm = a.gu_wscale[2 * e + m] * a.gu_inscale[2 * e + m];
  if (m == 0) {
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) gbuf[wr + 4 * g + q][16 * t + r] = acc[t][q] * fm;
  }
  __syncthreads();
  if (m == 0 || !on) return;
  const float gdn = a.dn_inscale[e];
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) {
    if (t >= ntt) continue;
    float h[4];
    float am = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = swiglu(gbuf[wr + 4 * g + q][16 * t + r], acc[t][q] * fm);
      am = __builtin_fmaxf(am, __builtin_fabsf(h[q]));
    }
    am = __builtin_fmaxf(am, __shfl_xor(am, 16, kWave));
    am = __builtin_fmaxf(am, __shfl_xor(am, 32, kWave));
    const uint32_t sc = f32_to_e4m3(__fdiv_rn(__fdiv_rn(am, 6.0f), gdn));
    const float d = __fmul_rn(e4m3_to_f32(sc), gdn);
    uint32_t nib = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) nib |= e2m1_under(h[q], d) << (4 * q);
    const int n = 16 * t + r;
    if (n < np) {
      const size_t row = (size_t)(row0 + n);
      *reinterpret_cast<uint16_t*>(a.h_codes + row * (I / 2) + i0 / 2 + 2 * g) = (uint16_t)nib;
      if (g == 0) static_cast<uint8_t*>(a.h_scales)[row * (I / 16) + i0 / 16] = (uint8_t)sc;
    }
  }
}

// ------------------------------------------------------------------ down
// Workgroup: one chunk, 16 NW output rows (wave w: rows o0 = 16 NW rb + 16w .. +15).
// Waves past the first four only wait at the staging barriers (the chunk's
// activations need 256 staging threads).
template <int NW>
__global__ void __launch_bounds__(NW * kWave) k_down_wide_a4(FfnArgs a, const int4* __restrict__ plan,
                                                            int slots) {
  constexpr int kRows = 16 * NW;   // output rows of the workgroup: 16 per wave
  __shared__ WideLds<1> lds;
  const Job job = wide_job(plan, (a.H + kRows - 1) / kRows, slots);
  if (job.e < 0) return;
  const int e = job.e, row0 = job.row0, np = job.ne;
  const int H = a.H, I = a.I;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int o0 = job.rb * kRows + wave * 16;
  const bool on = o0 < H;
  const size_t row16 = (size_t)e * H + (on ? o0 : H - 16);
  const Rows w = make_rows(a.dn_codes + row16 * (I / 2), a.dn_scales + row16 * (I / 16), 16, I);
  const Rows x = make_rows(a.h_codes + (size_t)row0 * (I / 2),
                           static_cast<const uint8_t*>(a.h_scales) + (size_t)row0 * (I / 16), np, I);
  const int ntt = (np + 15) / 16;
  const Stager sg = make_stager<1>(np, ntt, I);
  f32x4 acc[kWideTiles];
  by_tiles(ntt, [&](auto NT) {
    wide_mainloop<1, decltype(NT)::value>(w, r * (I / 2) + 16 * g, r * (I / 16), x, sg, 0,
                                          I, lds, acc);
  });
  if (!on) return;
  const float f = a.dn_wscale[e] * a.dn_inscale[e];
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) {
    const int n = 16 * t + r;
    if (t < ntt && n < np) {
      const float4 o = make_float4(acc[t][0] * f, acc[t][1] * f, acc[t][2] * f, acc[t][3] * f);
      *reinterpret_cast<float4*>(a.y + (size_t)(row0 + n) * H + o0 + 4 * g) = o;
    }
  }
}

// Plan entries for P sorted rows: at most one partial chunk per active expert
// (active experts <= min(E, P)) plus P / 32 full chunks.
int wide_plan_entries(int P, int E) { return (P < E ? P : E) + P / kWideTok; }

// Grid of the XCD-aware mapping: whole groups of 8 plan entries, nrb row blocks each.
static unsigned wide_grid(int entries, int nrb) {
  return (unsigned)(((entries + kXcds - 1) / kXcds) * kXcds * nrb);
}

// The product core alone (moe_debug_nvfp4_matmul): one matrix of N = a.H rows
// and K = a.I as expert 0's down matrix, its a.T columns cut into chunks of 32.
__global__ void __launch_bounds__(256) k_debug_plan(int cols, int n_entries, int4* __restrict__ plan) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j < n_entries)
    plan[j] = j * kWideTok < cols ? make_int4(0, j * kWideTok, min(kWideTok, cols - j * kWideTok), 0)
                                  : make_int4(-1, 0, 0, 0);
}

size_t debug_wide_plan_bytes(int cols) { return (size_t)((cols + kWideTok - 1) / kWideTok) * sizeof(int4); }

moe_status launch_debug_wide(const FfnArgs& a, void* plan_ws, hipStream_t s) {
  int4* plan = static_cast<int4*>(plan_ws);
  const int n = (a.T + kWideTok - 1) / kWideTok;
  hipLaunchKernelGGL(k_debug_plan, dim3((n + 255) / 256), dim3(256), 0, s, a.T, n, plan);
  moe_status st = check_launch("moe_debug_nvfp4_matmul (plan)");
  if (st != MOE_OK) return st;
  const int nrb = (a.H + kDownRows - 1) / kDownRows;
  hipLaunchKernelGGL(k_down_wide_a4<kDownWaves>, dim3(wide_grid(n, nrb)), dim3(kDownWaves * kWave), 0, s, a,
                     plan, n);
  return check_launch("moe_debug_nvfp4_matmul (wide)");
}

moe_status launch_ffn_wide_a4(const FfnArgs& a, int stage_mask, void* plan_ws, hipStream_t s) {
  int4* plan = static_cast<int4*>(plan_ws);
  const int n = wide_plan_entries(a.T * a.k, a.E);
  if (stage_mask & 6) {
    hipLaunchKernelGGL(k_wide_plan, dim3(1), dim3(1024), 0, s, a.offsets, a.E, n, plan);
    moe_status st = check_launch("nvfp4_expert_ffn (wide plan)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 2) {
    const int nrb = (a.I + kWideRows - 1) / kWideRows;
    hipLaunchKernelGGL(k_gateup_wide_a4, dim3(wide_grid(n, nrb)), dim3(512), 0, s, a, plan, n);
    moe_status st = check_launch("nvfp4_expert_ffn (wide gate/up)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 4) {
    const int nrb = (a.H + kDownRows - 1) / kDownRows;
    hipLaunchKernelGGL(k_down_wide_a4<kDownWaves>, dim3(wide_grid(n, nrb)), dim3(kDownWaves * kWave), 0, s,
                       a, plan, n);
    return check_launch("nvfp4_expert_ffn (wide down)");
  }
  return MOE_OK;
}

}  // namespace moe
