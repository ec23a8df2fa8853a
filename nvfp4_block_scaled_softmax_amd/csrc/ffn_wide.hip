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

// The same as a bf16x8 operand (16-bit activations): E2M1 to fp32, times the
// E4M3 scale in fp32 (exact: at most 6 significant bits), packed to bf16 (exact).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ bf16x8 expand8_bf16(uint32_t codes, float s) {
  const f32x2 a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
  const f32x2 b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
  const f32x2 c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
  const f32x2 d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
  return bf16x8{(__bf16)(a.x * s), (__bf16)(a.y * s), (__bf16)(b.x * s), (__bf16)(b.y * s),
                (__bf16)(c.x * s), (__bf16)(c.y * s), (__bf16)(d.x * s), (__bf16)(d.y * s)};
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

// Buffer resource over [base, base + bytes); 0x00020000 is the raw-buffer
// format word of the gfx9 family.  Every offset used below stays inside.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Rows of NVFP4 pieces along K: codes [rows][K/2], scales [rows][K/16].  A lane
// reads piece g (32 values) of step st of its row: code offset row*K/2 + 16g +
// 64st, scale offset row*K/16 + 2g + 8st; the step part is a scalar.  (As an
// activation source: the rows of the mode's stored activations, see XRows.)
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
// 64 per window; lane (r, g) loads bytes 16g .. 16g+15 of its row's window p,
// one 16-byte load per 8 steps instead of a 2-byte load per step.  Canonical
// layout: those are steps 8p + 2g and 8p + 2g + 1, and each step's pair is
// fetched from the lane that holds it; tiled layout (a full window): they are
// piece g of all 8 steps, the lane's own.  Past the end of a row the load reads the next row
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

// The same in the tiled layout (a full window): lane (r, g) loaded piece g of
// all 8 steps, step I in dword I / 2, half I % 2; no exchange between lanes.
template <int I>
__device__ __forceinline__ uint32_t window_scales_tiled(const uint4& sw) {
  const uint32_t d = I / 2 == 0 ? sw.x : I / 2 == 1 ? sw.y : I / 2 == 2 ? sw.z : sw.w;
  return I % 2 ? d >> 16 : d & 0xFFFFu;
}

// The MFMA operand type of a mode: bf16 for 16-bit activations, f16 otherwise.
template <int MODE>
using WideOp = typename std::conditional<MODE == MOE_A16, bf16x8, f16x8>::type;

template <int MODE>
__device__ __forceinline__ void expand_frag(const uint4& c, uint32_t sc, WideOp<MODE> (&v)[4]) {
  if constexpr (MODE == MOE_A16) {
    const float s0 = e4m3_to_f32(sc & 0xFFu), s1 = e4m3_to_f32((sc >> 8) & 0xFFu);
    v[0] = expand8_bf16(c.x, s0);
    v[1] = expand8_bf16(c.y, s0);
    v[2] = expand8_bf16(c.z, s1);
    v[3] = expand8_bf16(c.w, s1);
  } else {
    f16x2 s0, s1;
    scale_pair(sc, s0, s1);
    v[0] = expand8(c.x, s0);
    v[1] = expand8(c.y, s0);
    v[2] = expand8(c.z, s1);
    v[3] = expand8(c.w, s1);
  }
}

template <int MODE>
__device__ __forceinline__ f32x4 wide_mfma(const WideOp<MODE>& a, const uint4& b, const f32x4& c) {
  if constexpr (MODE == MOE_A16) return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bitcast<bf16x8>(b), c, 0, 0, 0);
  else return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bitcast<f16x8>(b), c, 0, 0, 0);
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
// K values at a time, into one of two LDS buffers (row stride 528 B: lanes
// reading 16 B at consecutive tokens hit distinct banks).  Within a token's row
// the 16-byte slot s sits at s ^ ((s >> 3) & 3) (slot_swz): a staging thread
// writes four consecutive slots 4q .. 4q+3, and eight threads of one token
// would otherwise write them to two bank groups.  One barrier per 256
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

// Physical 16-byte slot of logical slot s (0..31) in a token's LDS row: the
// low two bits are XORed with bits 3-4, a permutation that spreads the slots
// one staging instruction writes (s = 4 sq + q, sq = 0..7) over eight banks
// groups and leaves the slot of a B-operand read (one s across 16 tokens) alone.
__host__ __device__ constexpr int slot_swz(int s) { return s ^ ((s >> 3) & 3); }
// The closed forms stage_chunk and wide_mainloop use: staging slot 4 sq + q at
// 4 sq + (q ^ (sq >> 1)); read slot 16 h + 4 g + j at 16 h + 4 g + (j ^ (2 h + g / 2) % 4).
constexpr bool slot_swz_forms() {
  for (int sq = 0; sq < 8; ++sq)
    for (int q = 0; q < 4; ++q)
      if (slot_swz(4 * sq + q) != 4 * sq + (q ^ ((sq >> 1) & 3))) return false;
  for (int h = 0; h < 2; ++h)
    for (int g = 0; g < 4; ++g)
      for (int j = 0; j < 4; ++j)
        if (slot_swz(16 * h + 4 * g + j) != 16 * h + 4 * g + (j ^ ((2 * h + (g >> 1)) & 3))) return false;
  return true;
}
static_assert(slot_swz_forms(), "slot swizzle closed forms");

template <int NM>
struct WideLds {
  static constexpr int kBuf = NM * kWideTok * kTokStride;   // [NM][token][k] 16-bit values
  __align__(16) uint8_t buf[2 * kBuf];
};

// LDS planes of a chunk's activations: 4-bit gate/up, one per matrix (each
// matrix has its own input scale); 16-bit, the bf16 values; 8-bit, each value
// f32(E4M3 value * its block's fp32 scale) as the sum of two fp16 (hi, lo:
// 22 significant bits), which the main loop multiplies in two MFMAs.
template <int MODE, bool GU>
constexpr int wide_planes() { return MODE == MOE_A16 ? 1 : (MODE == MOE_A8 ? 2 : (GU ? 2 : 1)); }

// One thread's share of staging: plane sm, token sn, 32-wide piece sq of a chunk.
struct Stager {
  int sm, sn, sq;
  int vc, vs;       // byte offsets of the thread's activation row (values or codes, scales)
  int K;
  bool on;          // the token belongs to a computed column tile
};

// The raw activation piece a staging thread loads per chunk.
template <int MODE>
struct XFrag;
template <>
struct XFrag<MOE_A4> {
  uint4 c;
  uint16_t s;   // widened where used, so no instruction touches it before then
};
template <>
struct XFrag<MOE_A16> {
  uint4 v[4];
};
template <>
struct XFrag<MOE_A8> {
  uint4 c[2];
  uint2 s;
};

// Activation rows as buffers: 4-bit codes [rows][K/2] + E4M3 [rows][K/16]; 16-bit
// bf16 [rows][K]; 8-bit E4M3 [rows][K] + fp32 [rows][K/16].
template <int MODE>
__device__ __forceinline__ Rows make_xrows(const void* vals, const void* scales, int rows, int K) {
  if constexpr (MODE == MOE_A16) return Rows{rsrc(vals, rows * K * 2), rsrc(vals, rows * K * 2)};
  else if constexpr (MODE == MOE_A8) return Rows{rsrc(vals, rows * K), rsrc(scales, rows * (K / 16) * 4)};
  else return Rows{rsrc(vals, rows * (K / 2)), rsrc(scales, rows * (K / 16))};
}

template <int MODE>
__device__ __forceinline__ void load_chunk(XFrag<MODE>& f, const Rows& x, const Stager& sg, int c) {
  const int ke = min(c * kChunkK + 32 * sg.sq, sg.K - 32);   // first K value, clamped into the row
  if constexpr (MODE == MOE_A16) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      f.v[q] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x.codes, sg.vc + 2 * ke + 16 * q, 0, 0));
  } else if constexpr (MODE == MOE_A8) {
    f.c[0] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x.codes, sg.vc + ke, 0, 0));
    f.c[1] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x.codes, sg.vc + ke + 16, 0, 0));
    f.s = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(x.scales, sg.vs + 4 * (ke / 16), 0, 0));
  } else {
    f.c = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(x.codes, sg.vc + ke / 2, 0, 0));
    f.s = __builtin_amdgcn_raw_buffer_load_b16(x.scales, sg.vs + ke / 16, 0, 0);
  }
}

// Four E4M3 codes (one dword) times fp32 scale s times the token's power of two
// pw, each product one rounding, split into fp16 hi and lo parts.
__device__ __forceinline__ void fp8x4_hilo(uint32_t w, float s, float pw, uint2& hi, uint2& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const float v = __fmul_rn(__fmul_rn(e4m3_to_f32((w >> (8 * b)) & 0xFFu), s), pw);
    const _Float16 vh = (_Float16)v;
    h[b] = __builtin_bit_cast(uint16_t, vh);
    l[b] = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)vh));   // v - hi is exact in fp32
  }
  hi = make_uint2(h[0] | h[1] << 16, h[2] | h[3] << 16);
  lo = make_uint2(l[0] | l[1] << 16, l[2] | l[3] << 16);
}

template <int MODE>
__device__ __forceinline__ void stage_chunk(uint8_t* buf, const XFrag<MODE>& f, const Stager& sg, float pw) {
  if (!sg.on) return;
  // slots 4 sq + q of the token's row, at slot_swz(4 sq + q) = 4 sq + (q ^ x)
  uint8_t* row = buf + (sg.sm * kWideTok + sg.sn) * kTokStride + 64 * sg.sq;
  const int x = (sg.sq >> 1) & 3;
  auto d = [&](int q) { return reinterpret_cast<uint4*>(row + 16 * (q ^ x)); };
  if constexpr (MODE == MOE_A16) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *d(q) = f.v[q];
  } else if constexpr (MODE == MOE_A8) {
    const float s0 = __uint_as_float(f.s.x), s1 = __uint_as_float(f.s.y);
    const uint32_t w[8] = {f.c[0].x, f.c[0].y, f.c[0].z, f.c[0].w, f.c[1].x, f.c[1].y, f.c[1].z, f.c[1].w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint2 h0, l0, h1, l1;
      fp8x4_hilo(w[2 * q], q < 2 ? s0 : s1, pw, h0, l0);
      fp8x4_hilo(w[2 * q + 1], q < 2 ? s0 : s1, pw, h1, l1);
      *d(q) = make_uint4(h0.x, h0.y, h1.x, h1.y);
      *reinterpret_cast<uint4*>(reinterpret_cast<uint8_t*>(d(q)) + kWideTok * kTokStride) =   // plane 1
          make_uint4(l0.x, l0.y, l1.x, l1.y);
    }
  } else {
    f16x2 s0, s1;
    scale_pair(f.s, s0, s1);
    *d(0) = bitcast<uint4>(expand8(f.c.x, s0));
    *d(1) = bitcast<uint4>(expand8(f.c.y, s0));
    *d(2) = bitcast<uint4>(expand8(f.c.z, s1));
    *d(3) = bitcast<uint4>(expand8(f.c.w, s1));
  }
}

// w: the wave's 16 weight rows, lane offsets wc/ws; x: the chunk's activation
// rows; m: the wave's matrix (4-bit gate/up: which LDS plane its B operands come
// from; the 8-bit mode reads planes 0 and 1 into the same sums).
template <int MODE, int NM, int NT>
__device__ __forceinline__ void wide_mainloop(const Rows& w, int wc, int ws_row, const Rows& x,
                                              const Stager& sg, int m, int K, WideLds<NM>& lds,
                                              f32x4 (&acc)[kWideTiles], float pw, int tiled) {
  const int lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  const int nsteps = K / kKStep, nchunks = (nsteps + 1) / 2;
  const int nwin = (nsteps + kBody - 1) / kBody;
  constexpr int kB = MODE == MOE_A8 ? 2 : 1;   // LDS planes per MFMA operand
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 fw[kWSets];
  XFrag<MODE> fx[2];
  load_chunk<MODE>(fx[0], x, sg, 0);
  load_chunk<MODE>(fx[1], x, sg, min(1, nchunks - 1));
  uint4 sw = load_wscales(w, ws_row, g, 0), swn;
#pragma unroll
  for (int d = 0; d < kWSets - 1; ++d) fw[d] = load_wcodes(w, wc, min(d, nsteps - 1));
  stage_chunk<MODE>(lds.buf, fx[0], sg, pw);
  __syncthreads();

  // step s = s0 + u of the body (one scale window): chunk s / 2, LDS buffer and
  // raw set (u / 2) % 2, weight set u % kWSets
  auto step = [&](int s0, auto U) {
    constexpr int u = decltype(U)::value;
    constexpr int cb = (u / 2) % 2;
    const int s = s0 + u;
    if constexpr (u == 0) swn = load_wscales(w, ws_row, g, min(s0 / kBody + 1, nwin - 1));
    if constexpr (u % 2 == 0)   // first step of a chunk: raw activations of the chunk after next
      load_chunk<MODE>(fx[cb], x, sg, min(s / 2 + 2, nchunks - 1));
    fw[(u + kWSets - 1) % kWSets] = load_wcodes(w, wc, min(s + kWSets - 1, nsteps - 1));
    __builtin_amdgcn_sched_barrier(0);   // the loads go out before the compute below
    if (s < nsteps) {
      WideOp<MODE> av[4];
      // a full window of tiled scales holds this lane's pairs; else fetch them
      const uint32_t sc = tiled && s0 + kBody <= nsteps ? window_scales_tiled<u>(sw) : window_scales<u>(sw, lane);
      expand_frag<MODE>(fw[u % kWSets], sc, av);
      const uint8_t* bm = lds.buf + cb * WideLds<NM>::kBuf + (MODE == MOE_A4 ? m : 0) * kWideTok * kTokStride +
                          (u % 2) * (kKStep * 2) + 64 * g;
      // logical slot 16 (u % 2) + 4 g + j of the row sits at 16 (u % 2) + 4 g + (j ^ xr) (slot_swz)
      const int xr = (2 * (u % 2) + (g >> 1)) & 3;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
          for (int b = 0; b < kB; ++b) {
            const uint4 bv =
                *reinterpret_cast<const uint4*>(bm + (b * kWideTok + 16 * t + r) * kTokStride + 16 * (j ^ xr));
            acc[t] = wide_mfma<MODE>(av[j], bv, acc[t]);
          }
        }
      }
    }
    if constexpr (u % 2 == 1) {   // last step of a chunk: stage the next chunk, then sync
      stage_chunk<MODE>(lds.buf + (cb ^ 1) * WideLds<NM>::kBuf, fx[cb ^ 1], sg, pw);
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

// Staging share of thread tid for a chunk of np tokens (ntt tiles computed).
// 4-bit gate/up: NM planes, activation row (token, matrix) = token * NM + matrix
// of the chunk's rows; otherwise one row per token (plane 0 threads stage it,
// the 8-bit mode into both planes), at row_of(token of the chunk) of the source.
template <int MODE, int NM, typename RowOf>
__device__ __forceinline__ Stager make_stager(int np, int ntt, int K, RowOf&& row_of) {
  Stager sg;
  sg.sm = threadIdx.x / (kWideTok * 8);
  sg.sn = (threadIdx.x / 8) % kWideTok;
  sg.sq = threadIdx.x % 8;
  sg.K = K;
  if constexpr (MODE == MOE_A4) {
    const int row = min(sg.sn, np - 1) * NM + min(sg.sm, NM - 1);
    sg.vc = row * (K / 2);
    sg.vs = row * (K / 16);
    sg.on = sg.sn < 16 * ntt && sg.sm < NM;   // threads past NM planes only wait at the barriers
  } else {
    const int row = row_of(min(sg.sn, np - 1));
    sg.vc = MODE == MOE_A16 ? row * K * 2 : row * K;
    sg.vs = row * (K / 16) * 4;
    sg.sm = 0;
    sg.on = sg.sn < 16 * ntt && threadIdx.x < kWideTok * 8;
  }
  return sg;
}

// 8-bit mode: a power of two per token of the chunk that keeps its activations
// below 2^14 in magnitude (so their fp16 hi parts are finite; 1 for ordinary
// data), from the row's block scales (fp32 [rows][K/16]; amax <= 448 * scale):
// the staging multiplies by pw[n], the epilogue by 1 / pw[n] (both exact).
template <int NWAVES, typename RowOf>
__device__ __forceinline__ void token_pow2(const float* scales, int K, int np, RowOf&& row_of, float* pw) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  for (int n = wave; n < kWideTok; n += NWAVES) {
    float mx = 0.0f;
    if (n < np) {
      const float* rs = scales + (size_t)row_of(n) * (K / 16);
      for (int b = lane; b < K / 16; b += kWave) mx = __builtin_fmaxf(mx, rs[b]);
    }
    mx = wave_max(mx) * 448.0f;
    // 2^(13 - floor(log2 mx)) from the exponent field (mx >= 2^14 is normal and finite here)
    const int ex = (int)((__float_as_uint(mx) >> 23) & 0xFFu) - 127;
    if (lane == 0) pw[n] = mx >= 16384.0f ? __uint_as_float((uint32_t)(13 - ex + 127) << 23) : 1.0f;
  }
}

// ------------------------------------------------------------------ gate/up + SwiGLU + h
// Workgroup: one chunk, 64 h rows i0 .. i0+63; wave w < 4: gate rows i0+16w ..
// +15, wave w >= 4: the same up rows.  Rows past I (a ragged last row block)
// read clamped rows and store nothing.  The intermediate in the mode's
// precision: bf16 (16-bit), E4M3 with an fp32 scale per 16 (8-bit), NVFP4
// under the down matrix's input scale (4-bit); 16 rows of a wave are one block.
template <int MODE>
__global__ void __launch_bounds__(512) k_gateup_wide(FfnArgs a, const int4* __restrict__ plan, int slots) {
  constexpr int NM = wide_planes<MODE, true>();
  __shared__ WideLds<NM> lds;
  __shared__ float gbuf[kWideRows][kWideTok];   // gate * its multipliers, [h row][token]
  __shared__ float s_pw[kWideTok];
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
  const int ntt = (np + 15) / 16;
  // activation rows: 4-bit, the chunk's pair rows (gate, up) of the quantized x;
  // otherwise the tokens' rows of x (bf16 or E4M3 + fp32 scales)
  auto tok_of = [&](int n) { return a.sorted_pairs[row0 + n] / a.k; };
  Rows x;
  if constexpr (MODE == MOE_A4) {
    const size_t xr0 = (size_t)row0 * 2;
    x = make_rows(a.xq_codes + xr0 * (H / 2), static_cast<const uint8_t*>(a.xq_scales) + xr0 * (H / 16), 2 * np, H);
  } else if constexpr (MODE == MOE_A16) {
    x = make_xrows<MODE>(a.x, nullptr, a.T, H);
  } else {
    x = make_xrows<MODE>(a.xq_codes, a.xq_scales, a.T, H);
  }
  const Stager sg = make_stager<MODE, NM>(np, ntt, H, tok_of);
  float pw = 1.0f;
  if constexpr (MODE == MOE_A8) {
    token_pow2<8>(static_cast<const float*>(a.xq_scales), H, np, tok_of, s_pw);
    __syncthreads();
    pw = s_pw[sg.sn];
  }
  f32x4 acc[kWideTiles];
  by_tiles(ntt, [&](auto NT) {
    wide_mainloop<MODE, NM, decltype(NT)::value>(w, r * (H / 2) + 16 * g, r * (H / 16), x, sg, m, H, lds, acc, pw,
                                                 a.tiled);
  });
  const float fm = a.gu_wscale[2 * e + m] * (MODE == MOE_A4 ? a.gu_inscale[2 * e + m] : 1.0f);
  float tok_f[kWideTiles];   // 8-bit mode: undo the token's power of two (exact)
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) tok_f[t] = MODE == MOE_A8 ? 1.0f / s_pw[16 * t + r] : 1.0f;
  if (m == 0) {
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) gbuf[wr + 4 * g + q][16 * t + r] = acc[t][q] * tok_f[t] * fm;
  }
  __syncthreads();
  if (m == 0 || !on) return;
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) {
    if (t >= ntt) continue;
    float h[4];
    float am = 0.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[q] = swiglu(gbuf[wr + 4 * g + q][16 * t + r], acc[t][q] * tok_f[t] * fm);
      am = __builtin_fmaxf(am, __builtin_fabsf(h[q]));
    }
    const int n = 16 * t + r;
    const size_t row = (size_t)(row0 + n);
    if constexpr (MODE == MOE_A16) {
      if (n < np) {
        const uint32_t b0 = f32_to_bf16(h[0]) | f32_to_bf16(h[1]) << 16, b1 = f32_to_bf16(h[2]) | f32_to_bf16(h[3]) << 16;
        *reinterpret_cast<uint2*>(a.h_codes + (row * I + i0 + 4 * g) * 2) = make_uint2(b0, b1);
      }
      continue;
    }
    am = __builtin_fmaxf(am, __shfl_xor(am, 16, kWave));   // the 16 rows' amax (one block)
    am = __builtin_fmaxf(am, __shfl_xor(am, 32, kWave));
    if constexpr (MODE == MOE_A8) {   // as fp8_quant16: s = bamax / 448, codes E4M3(h / s)
      const float sc = __fdiv_rn(am, 448.0f);
      uint32_t cw = 0u;
      if (sc > 0.0f) {
#pragma unroll
        for (int q = 0; q < 4; ++q) cw |= f32_to_e4m3(__fdiv_rn(h[q], sc)) << (8 * q);
      }
      if (n < np) {
        *reinterpret_cast<uint32_t*>(a.h_codes + row * I + i0 + 4 * g) = cw;
        if (g == 0) static_cast<float*>(a.h_scales)[row * (I / 16) + i0 / 16] = sc;
      }
    } else {
      const float gdn = a.dn_inscale[e];
      const uint32_t sc = f32_to_e4m3(__fdiv_rn(__fdiv_rn(am, 6.0f), gdn));
      const float d = __fmul_rn(e4m3_to_f32(sc), gdn);
      uint32_t nib = 0u;
#pragma unroll
      for (int q = 0; q < 4; ++q) nib |= e2m1_under(h[q], d) << (4 * q);
      if (n < np) {
        *reinterpret_cast<uint16_t*>(a.h_codes + row * (I / 2) + i0 / 2 + 2 * g) = (uint16_t)nib;
        if (g == 0) static_cast<uint8_t*>(a.h_scales)[row * (I / 16) + i0 / 16] = (uint8_t)sc;
      }
    }
  }
}

// ------------------------------------------------------------------ down
// Workgroup: one chunk, 16 NW output rows (wave w: rows o0 = 16 NW rb + 16w .. +15).
// Waves past the first four only wait at the staging barriers (the chunk's
// activations need 256 staging threads).
template <int MODE, int NW>
__global__ void __launch_bounds__(NW * kWave) k_down_wide(FfnArgs a, const int4* __restrict__ plan, int slots) {
  constexpr int kRows = 16 * NW;   // output rows of the workgroup: 16 per wave
  constexpr int NM = wide_planes<MODE, false>();
  __shared__ WideLds<NM> lds;
  __shared__ float s_pw[kWideTok];
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
  auto row_of = [&](int n) { return row0 + n; };
  Rows x;
  if constexpr (MODE == MOE_A4)
    x = make_rows(a.h_codes + (size_t)row0 * (I / 2), static_cast<const uint8_t*>(a.h_scales) + (size_t)row0 * (I / 16),
                  np, I);
  else   // the rows of the whole intermediate; the stager offsets select the chunk's
    x = make_xrows<MODE>(a.h_codes, a.h_scales, row0 + np, I);
  const int ntt = (np + 15) / 16;
  const Stager sg = make_stager<MODE, NM>(np, ntt, I, row_of);
  float pw = 1.0f;
  if constexpr (MODE == MOE_A8) {
    token_pow2<NW>(static_cast<const float*>(a.h_scales), I, np, row_of, s_pw);
    __syncthreads();
    pw = s_pw[sg.sn];
  }
  f32x4 acc[kWideTiles];
  by_tiles(ntt, [&](auto NT) {
    wide_mainloop<MODE, NM, decltype(NT)::value>(w, r * (I / 2) + 16 * g, r * (I / 16), x, sg, 0, I, lds, acc, pw,
                                                 a.tiled);
  });
  if (!on) return;
  const float f = a.dn_wscale[e] * (MODE == MOE_A4 ? a.dn_inscale[e] : 1.0f);
#pragma unroll
  for (int t = 0; t < kWideTiles; ++t) {
    const int n = 16 * t + r;
    if (t < ntt && n < np) {
      const float ft = MODE == MOE_A8 ? f / s_pw[n] : f;
      const float4 o = make_float4(acc[t][0] * ft, acc[t][1] * ft, acc[t][2] * ft, acc[t][3] * ft);
      *reinterpret_cast<float4*>(a.y + (size_t)(row0 + n) * H + o0 + 4 * g) = o;
    }
  }
}

// Down with a short K (I <= 512, at most four 128-K steps): the chunk's whole
// intermediate fits the two LDS buffers, so it is staged once and the
// workgroup sweeps PASSES blocks of 16 NW output rows over it (wave w: rows
// o0 = 16 NW (PASSES rb + p) + 16 w .. +15 in pass p), with the next pass's
// weights loaded while the current one computes.  Staging (activation loads,
// expansion, a barrier) is the fixed cost of a down workgroup at this K; the
// sweep spreads it over PASSES times the weight rows.  Each output row is
// computed as in k_down_wide: the same fragments, MFMA order and epilogue.
template <int MODE, int NW, int PASSES>
__global__ void __launch_bounds__(NW * kWave) k_down_wide_short(FfnArgs a, const int4* __restrict__ plan, int slots) {
  constexpr int kRows = 16 * NW;
  constexpr int NM = wide_planes<MODE, false>();
  constexpr int kB = MODE == MOE_A8 ? 2 : 1;
  constexpr int kSteps = 4;   // I <= 512
  __shared__ WideLds<NM> lds;
  __shared__ float s_pw[kWideTok];
  const Job job = wide_job(plan, (a.H + kRows * PASSES - 1) / (kRows * PASSES), slots);
  if (job.e < 0) return;
  const int e = job.e, row0 = job.row0, np = job.ne;
  const int H = a.H, I = a.I, nsteps = I / kKStep;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = lane_id();
  const int r = lane & 15, g = lane >> 4;
  auto row_of = [&](int n) { return row0 + n; };
  Rows x;
  if constexpr (MODE == MOE_A4)
    x = make_rows(a.h_codes + (size_t)row0 * (I / 2), static_cast<const uint8_t*>(a.h_scales) + (size_t)row0 * (I / 16),
                  np, I);
  else
    x = make_xrows<MODE>(a.h_codes, a.h_scales, row0 + np, I);
  const int ntt = (np + 15) / 16;
  const Stager sg = make_stager<MODE, NM>(np, ntt, I, row_of);

  // the weights of pass p: the wave's 16 rows (clamped past H: computed, not stored)
  const int wc = r * (I / 2) + 16 * g, ws_row = r * (I / 16);
  auto wrows = [&](int p) {
    const int o0 = (job.rb * PASSES + p) * kRows + wave * 16;
    const size_t row16 = (size_t)e * H + (o0 < H ? o0 : H - 16);
    return make_rows(a.dn_codes + row16 * (I / 2), a.dn_scales + row16 * (I / 16), 16, I);
  };
  uint4 fw[2][kSteps], sw[2];
  auto load_pass = [&](int p, auto SET) {
    constexpr int set = decltype(SET)::value;
    const Rows w = wrows(p);
#pragma unroll
    for (int s = 0; s < kSteps; ++s) fw[set][s] = load_wcodes(w, wc, min(s, nsteps - 1));
    sw[set] = load_wscales(w, ws_row, g, 0);
  };
  load_pass(0, std::integral_constant<int, 0>{});
  XFrag<MODE> fx[2];
  load_chunk<MODE>(fx[0], x, sg, 0);
  load_chunk<MODE>(fx[1], x, sg, min(1, (nsteps + 1) / 2 - 1));
  float pw = 1.0f;
  if constexpr (MODE == MOE_A8) {
    token_pow2<NW>(static_cast<const float*>(a.h_scales), I, np, row_of, s_pw);
    __syncthreads();
    pw = s_pw[sg.sn];
  }
  stage_chunk<MODE>(lds.buf, fx[0], sg, pw);
  stage_chunk<MODE>(lds.buf + WideLds<NM>::kBuf, fx[1], sg, pw);
  __syncthreads();   // the only barrier after this point: LDS is read-only below

  const float f = a.dn_wscale[e] * (MODE == MOE_A4 ? a.dn_inscale[e] : 1.0f);
  static_for<0, PASSES>([&](auto P) {
    constexpr int p = decltype(P)::value, set = p % 2;
    if constexpr (p + 1 < PASSES) load_pass(p + 1, std::integral_constant<int, set ^ 1>{});   // in flight during this pass
    __builtin_amdgcn_sched_barrier(0);
    const int o0 = (job.rb * PASSES + p) * kRows + wave * 16;
    if (o0 >= H) return;
    f32x4 acc[kWideTiles];
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    by_tiles(ntt, [&](auto NTc) {
      constexpr int NT = decltype(NTc)::value;
      static_for<0, kSteps>([&](auto U) {
        constexpr int u = decltype(U)::value;
        if (u >= nsteps) return;
        WideOp<MODE> av[4];
        expand_frag<MODE>(fw[set][u], window_scales<u>(sw[set], lane), av);
        const uint8_t* bm = lds.buf + (u / 2) * WideLds<NM>::kBuf + (u % 2) * (kKStep * 2) + 64 * g;
        const int xr = (2 * (u % 2) + (g >> 1)) & 3;   // slot_swz
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int b = 0; b < kB; ++b) {
              const uint4 bv =
                  *reinterpret_cast<const uint4*>(bm + (b * kWideTok + 16 * t + r) * kTokStride + 16 * (j ^ xr));
              acc[t] = wide_mfma<MODE>(av[j], bv, acc[t]);
            }
      });
    });
#pragma unroll
    for (int t = 0; t < kWideTiles; ++t) {
      const int n = 16 * t + r;
      if (t < ntt && n < np) {
        const float ft = MODE == MOE_A8 ? f / s_pw[n] : f;
        const float4 o = make_float4(acc[t][0] * ft, acc[t][1] * ft, acc[t][2] * ft, acc[t][3] * ft);
        *reinterpret_cast<float4*>(a.y + (size_t)(row0 + n) * H + o0 + 4 * g) = o;
      }
    }
  });
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

// Output-row passes of a short-K down workgroup (k_down_wide_short).
constexpr int kDownPasses = 3;

template <int MODE>
static moe_status launch_down(const FfnArgs& a, const int4* plan, int n, const char* what, hipStream_t s) {
  if (a.I <= 4 * kKStep) {
    const int nrb = (a.H + kDownRows * kDownPasses - 1) / (kDownRows * kDownPasses);
    hipLaunchKernelGGL((k_down_wide_short<MODE, kDownWaves, kDownPasses>), dim3(wide_grid(n, nrb)),
                       dim3(kDownWaves * kWave), 0, s, a, plan, n);
    return check_launch(what);
  }
  const int nrb = (a.H + kDownRows - 1) / kDownRows;
  hipLaunchKernelGGL((k_down_wide<MODE, kDownWaves>), dim3(wide_grid(n, nrb)), dim3(kDownWaves * kWave), 0, s, a,
                     plan, n);
  return check_launch(what);
}

moe_status launch_debug_wide(const FfnArgs& a, moe_act_mode mode, void* plan_ws, hipStream_t s) {
  int4* plan = static_cast<int4*>(plan_ws);
  const int n = (a.T + kWideTok - 1) / kWideTok;
  hipLaunchKernelGGL(k_debug_plan, dim3((n + 255) / 256), dim3(256), 0, s, a.T, n, plan);
  moe_status st = check_launch("moe_debug_nvfp4_matmul (plan)");
  if (st != MOE_OK) return st;
  const char* what = "moe_debug_nvfp4_matmul (wide)";
  if (mode == MOE_A16) return launch_down<MOE_A16>(a, plan, n, what, s);
  if (mode == MOE_A8) return launch_down<MOE_A8>(a, plan, n, what, s);
  return launch_down<MOE_A4>(a, plan, n, what, s);
}

template <int MODE>
static moe_status launch_wide(const FfnArgs& a, int stage_mask, void* plan_ws, hipStream_t s) {
  int4* plan = static_cast<int4*>(plan_ws);
  const int n = wide_plan_entries(a.T * a.k, a.E);
  if (stage_mask & 6) {
    hipLaunchKernelGGL(k_wide_plan, dim3(1), dim3(1024), 0, s, a.offsets, a.E, n, plan);
    moe_status st = check_launch("nvfp4_expert_ffn (wide plan)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 2) {
    const int nrb = (a.I + kWideRows - 1) / kWideRows;
    hipLaunchKernelGGL(k_gateup_wide<MODE>, dim3(wide_grid(n, nrb)), dim3(512), 0, s, a, plan, n);
    moe_status st = check_launch("nvfp4_expert_ffn (wide gate/up)");
    if (st != MOE_OK) return st;
  }
  if (stage_mask & 4) return launch_down<MODE>(a, plan, n, "nvfp4_expert_ffn (wide down)", s);
  return MOE_OK;
}

moe_status launch_ffn_wide(const FfnArgs& a, moe_act_mode mode, int stage_mask, void* plan_ws, hipStream_t s) {
  if (mode == MOE_A16) return launch_wide<MOE_A16>(a, stage_mask, plan_ws, s);
  if (mode == MOE_A8) return launch_wide<MOE_A8>(a, stage_mask, plan_ws, s);
  return launch_wide<MOE_A4>(a, stage_mask, plan_ws, s);
}

}  // namespace moe
