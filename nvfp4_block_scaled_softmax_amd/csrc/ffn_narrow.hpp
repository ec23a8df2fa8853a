// The narrow (few-column) expert tiles as device functions, shared by the
// per-stage kernels (ffn_narrow.hip) and the fused decode kernel (decode.hip).
#pragma once
#include "ffn_common.hpp"

namespace moe {

constexpr int kGuRows = 16;    // h rows per gate/up workgroup (= one quantization block)
constexpr int kDnRows = 64;    // output rows per down workgroup
constexpr int kLdsBudget = 60 * 1024;
// Threads of every workgroup that runs these tiles.  A compile-time count: the
// block size read at run time is a vector memory load, and its wait would also
// wait for every weight load in flight.
constexpr int kTileThreads = 256;
constexpr int kTileWaves = kTileThreads / kWave;

constexpr int kStageBatch = 4;

// Tagged words of one row of the 8-bit intermediate (see gateup_tile).
__host__ __device__ constexpr int h8_words(int I) { return I / 4 + I / 16; }

// 8-bit mode, x of tokens 0..T-1 quantized in the tile: every 16-value block of
// a token's bf16 row as act_quant_fp8 computes it (fp8_quant16), written into
// the LDS chunk layout stage_gateup_cols uses (32 codes, then the two blocks'
// fp32 scales), columns by token.
__device__ void stage_gateup_quant_a8(const FfnArgs& a, uint8_t* lds) {
  constexpr int S = ChunkLds<MOE_A8>::kStride;
  const int H = a.H, NC = H / 32, nb = H / 16;
  for (int i = threadIdx.x; i < a.T * nb; i += kTileThreads) {
    const int t = i / nb, b = i % nb;
    const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)t * H + 16 * b);
    const uint4 u0 = src[0], u1 = src[1];
    const uint32_t wv[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = bf16_to_f32(wv[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_to_f32(wv[j] >> 16);
    }
    uint32_t w4[4];
    const float sc = fp8_quant16(v, w4);
    uint8_t* c = lds + ((size_t)t * NC + b / 2) * S;
    *reinterpret_cast<uint4*>(c + 16 * (b % 2)) = make_uint4(w4[0], w4[1], w4[2], w4[3]);
    *reinterpret_cast<float*>(c + 32 + 4 * (b % 2)) = sc;
  }
}

// tok[col]: the token of column col (the 16/8-bit modes read x by token);
// with BY_TOKEN the columns are the tokens 0..ncol-1 themselves.
template <int MODE, bool BY_TOKEN = false>
__device__ void stage_gateup_cols(const FfnArgs& a, int e, int row0, int c0, int ncol,
                                  const int* tok, uint8_t* lds) {
  constexpr int S = ChunkLds<MODE>::kStride;
  const int H = a.H, NC = H / 32;
  if (MODE == MOE_A16 || MODE == kModeQ4) {
    // 4 x 16 B per chunk (q4_g64_fp16: as fp16, paired by nibble)
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC * 4,
        [&](int i) {
          const int col = i / (NC * 4), rem = i % (NC * 4);
          return reinterpret_cast<const uint4*>(a.x + (size_t)(BY_TOKEN ? col : tok[col]) * H)[rem];
        },
        [&](int i, uint4 v) {
          const int col = i / (NC * 4), rem = i % (NC * 4), ch = rem / 4, q = rem % 4;
          if constexpr (MODE == kModeQ4) v = bf16x8_to_f16x8_paired(v);
          *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
        });
  } else if (MODE == MOE_A8) {
    const float* xs = static_cast<const float*>(a.xq_scales);
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC * 2,
        [&](int i) {
          const int col = i / (NC * 2), rem = i % (NC * 2);
          return reinterpret_cast<const uint4*>(a.xq_codes + (size_t)(BY_TOKEN ? col : tok[col]) * H)[rem];
        },
        [&](int i, uint4 v) {
          const int col = i / (NC * 2), rem = i % (NC * 2), ch = rem / 2, q = rem % 2;
          *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
        });
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC,
        [&](int i) {
          const int col = i / NC, ch = i % NC;
          return *reinterpret_cast<const float2*>(xs + (size_t)(BY_TOKEN ? col : tok[col]) * (H / 16) + ch * 2);
        },
        [&](int i, float2 v) {
          const int col = i / NC, ch = i % NC;
          *reinterpret_cast<float2*>(lds + ((size_t)col * NC + ch) * S + 32) = v;
        });
  } else {
    const uint8_t* xs = static_cast<const uint8_t*>(a.xq_scales);
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC * 2,
        [&](int i) {   // (col, matrix, chunk); matrix 0 gate, 1 up
          const int col = i / (NC * 2), q = (i / NC) % 2, ch = i % NC;
          const size_t r = (size_t)(row0 + c0 + col);
          return reinterpret_cast<const uint4*>(a.xq_codes + (r * 2 + q) * (H / 2))[ch];
        },
        [&](int i, uint4 v) {
          const int col = i / (NC * 2), q = (i / NC) % 2, ch = i % NC;
          *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
        });
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC,
        [&](int i) {
          const int col = i / NC, ch = i % NC;
          const size_t r = (size_t)(row0 + c0 + col);
          const uint16_t sg = *reinterpret_cast<const uint16_t*>(xs + (r * 2 + 0) * (H / 16) + 2 * ch);
          const uint16_t su = *reinterpret_cast<const uint16_t*>(xs + (r * 2 + 1) * (H / 16) + 2 * ch);
          return (uint32_t)sg | ((uint32_t)su << 16);
        },
        [&](int i, uint32_t v) {
          const int col = i / NC, ch = i % NC;
          *reinterpret_cast<uint32_t*>(lds + ((size_t)col * NC + ch) * S + 32) = v;
        });
  }
}

template <int MODE, bool COH>
__device__ void stage_down_cols(const FfnArgs& a, int row0, int c0, int ncol, uint8_t* lds) {
  constexpr int S = ChunkLds<MODE>::kStride;
  const int I = a.I, NC = I / 32;
  if (MODE == MOE_A16 || MODE == kModeQ4) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(a.h_codes);
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC * 4,
        [&](int i) {
          const int col = i / (NC * 4), rem = i % (NC * 4);
          return hld128<COH>(h, 2 * ((size_t)(row0 + c0 + col) * I) + 16 * (size_t)rem);
        },
        [&](int i, uint4 v) {
          const int col = i / (NC * 4), rem = i % (NC * 4), ch = rem / 4, q = rem % 4;
          if constexpr (MODE == kModeQ4) v = pair_by_nibble(v);   // fp16 h, paired by nibble
          *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
        });
  } else if (MODE == MOE_A8) {
    const float* hs = static_cast<const float*>(a.h_scales);
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC * 2,
        [&](int i) {
          const int col = i / (NC * 2), rem = i % (NC * 2);
          return hld128<COH>(a.h_codes, (size_t)(row0 + c0 + col) * I + 16 * (size_t)rem);
        },
        [&](int i, uint4 v) {
          const int col = i / (NC * 2), rem = i % (NC * 2), ch = rem / 2, q = rem % 2;
          *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
        });
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC,
        [&](int i) {
          const int col = i / NC, ch = i % NC;
          return hld64<COH>(hs, 4 * ((size_t)(row0 + c0 + col) * (I / 16) + ch * 2));
        },
        [&](int i, uint2 v) {
          const int col = i / NC, ch = i % NC;
          *reinterpret_cast<uint2*>(lds + ((size_t)col * NC + ch) * S + 32) = v;
        });
  } else {
    const uint8_t* hs = static_cast<const uint8_t*>(a.h_scales);
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC,
        [&](int i) {
          const int col = i / NC, ch = i % NC;
          return hld128<COH>(a.h_codes, (size_t)(row0 + c0 + col) * (I / 2) + 16 * (size_t)ch);
        },
        [&](int i, uint4 v) {
          const int col = i / NC, ch = i % NC;
          *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S) = v;
        });
    batched_copy<kTileThreads, kStageBatch>(
        ncol * NC,
        [&](int i) {
          const int col = i / NC, ch = i % NC;
          return (uint32_t)hld16<COH>(hs, (size_t)(row0 + c0 + col) * (I / 16) + 2 * (size_t)ch);
        },
        [&](int i, uint32_t v) {
          const int col = i / NC, ch = i % NC;
          *reinterpret_cast<uint32_t*>(lds + ((size_t)col * NC + ch) * S + 32) = v;
        });
  }
}

// ------------------------------------------------------------------ gate/up
// One tile: 16 h rows (rb) of expert e; 4 waves; wave w owns h rows 4w..4w+3 of
// the tile; lanes 0-31 read the gate rows, lanes 32-63 the up rows; within a
// half-wave, LPR lanes share a row and each reads CPL chunks of it.
// A callable that does nothing (a tile hook that is not needed).
struct NoHook {
  __device__ void operator()() const {}
};

// tmask >= 0: the tile's sorted rows are the tokens of this mask in ascending
// order (so sorted_pairs is not read); -1: the tokens come from sorted_pairs.
// 4-bit mode, quantizing in the tile: x of the tokens in tok (one per column)
// quantized per 16 under the expert's gate and up input scales straight into
// the A4 chunk layout (the arithmetic of the stand-alone quantizers, so the
// codes are the same); with write_ws the codes and scales also go to the
// workspace rows row0 + c0 + col, as the stand-alone quantizer writes them.
__device__ void stage_gateup_quant_a4(const FfnArgs& a, int e, int row0, int c0, int ncol, const int* tok,
                                      uint8_t* lds, bool write_ws) {
  constexpr int S = ChunkLds<MOE_A4>::kStride;
  const int H = a.H, nb = H / 16, NC = H / 32;
  const float g0 = a.gu_inscale[2 * e], g1 = a.gu_inscale[2 * e + 1];
  const bool same = __float_as_uint(g0) == __float_as_uint(g1);
  for (int i = threadIdx.x; i < ncol * nb; i += kTileThreads) {
    const int col = i / nb, b = i % nb, hb = b % 2;
    const uint4* src = reinterpret_cast<const uint4*>(a.x + (size_t)tok[col] * H + (size_t)b * 16);
    const uint4 u0 = src[0], u1 = src[1];
    const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
    float v[16];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      v[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      v[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
    uint32_t lo0, hi0, lo1, hi1;
    const uint32_t s0 = nvfp4_quant16(v, g0, lo0, hi0);
    uint32_t s1 = s0;
    lo1 = lo0;
    hi1 = hi0;
    if (!same) s1 = nvfp4_quant16(v, g1, lo1, hi1);
    uint8_t* c = lds + ((size_t)col * NC + b / 2) * S;
    *reinterpret_cast<uint2*>(c + 8 * hb) = make_uint2(lo0, hi0);
    *reinterpret_cast<uint2*>(c + 16 + 8 * hb) = make_uint2(lo1, hi1);
    c[32 + hb] = (uint8_t)s0;
    c[34 + hb] = (uint8_t)s1;
    if (write_ws) {
      const size_t r = (size_t)(row0 + c0 + col);
      uint8_t* xc = const_cast<uint8_t*>(a.xq_codes);
      uint8_t* xs = static_cast<uint8_t*>(const_cast<void*>(a.xq_scales));
      *reinterpret_cast<uint2*>(xc + (r * 2 + 0) * (H / 2) + (size_t)b * 8) = make_uint2(lo0, hi0);
      *reinterpret_cast<uint2*>(xc + (r * 2 + 1) * (H / 2) + (size_t)b * 8) = make_uint2(lo1, hi1);
      xs[(r * 2 + 0) * nb + b] = (uint8_t)s0;
      xs[(r * 2 + 1) * nb + b] = (uint8_t)s1;
    }
  }
}

// htag: the intermediate is also published as 64-bit words (payload << 32) |
// epoch, each written as one atomic store, for consumers that poll the words:
// 16-bit mode, the bf16 pair (2i, 2i+1) of a row in htag[row * I/2 + i]; 8-bit
// mode, row r's words at htag + r * h8_words(I): four E4M3 codes (values 4i ..
// 4i+3) in word i < I/4, then block b's fp32 scale in word I/4 + b.
// QX (4-bit mode): x is quantized in the tile (stage_gateup_quant_a4) instead of
// read quantized from the workspace; row block 0's tile also writes it there.
// XS (16/8-bit modes, a.T <= max_cols): the caller has staged x of every token
// into LDS (stage_gateup_cols by token) and synchronised; no x load then
// follows the weight loads, so the compute of a chunk waits only for that
// chunk's weights.
template <int MODE, int LPR, int CPL, bool COH = false, bool QX = false, bool XS = false>
__device__ __forceinline__ void gateup_tile(const FfnArgs& a, int e, int row0, int ne, int rb,
                                            int max_cols, uint8_t* lds, int tmask = -1,
                                            uint64_t* htag = nullptr, uint32_t epoch = 0u) {
  __shared__ float part[8][kGuRows][2];
  __shared__ float hbuf[8][kGuRows];
  __shared__ int s_tok[8];
  constexpr int S = ChunkLds<MODE>::kStride;
  constexpr int SLOTS = 32 / LPR;
  constexpr int RP = (4 + SLOTS - 1) / SLOTS;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int H = a.H, I = a.I, NC = H / 32;
  const int i0 = rb * kGuRows;
  const int half = lane >> 5, l32 = lane & 31, slot = l32 / LPR, kl = l32 % LPR;

  // the tokens of the first column group go out before the weights, so that
  // the x loads (issued after the weights) need not wait for the weights
  auto col_pair = [&](int c0) {   // the pair of column lane; its token is pair / k
    const int l = lane_id();
    if ((MODE == MOE_A4 && !QX) || l >= min(max_cols, ne - c0)) return 0;
    if (tmask >= 0) {   // column c0 + l is the mask's (c0 + l)-th token
      uint32_t m = (uint32_t)tmask;
      for (int i = 0; i < c0 + l && m != 0u; ++i) m &= m - 1u;
      return m != 0u ? (__ffs((int)m) - 1) * a.k : 0;
    }
    return (int)hld32<COH>(a.sorted_pairs, 4 * (size_t)(row0 + c0 + l));
  };
  int pair = col_pair(0);
  const bool by_token = XS || (MODE != MOE_A4 && a.T <= max_cols);
  if constexpr (XS) {   // the first column group's tokens, before the weight loads
    if (threadIdx.x < min(max_cols, ne)) s_tok[threadIdx.x] = pair / a.k;
    __syncthreads();
  }
  __builtin_amdgcn_sched_barrier(0);
  // this lane's weight chunks: RP h rows x CPL chunks, all loads in flight
  // together, chunk by chunk in the order the compute below takes them
  uint4 wq[RP][CPL];
  uint32_t wsc[RP][CPL];
  const uint8_t* crow[RP];
  const uint8_t* srow[RP];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int hl = slot * RP + r;  // h row within the wave's four
    const size_t grow = (size_t)e * 2 * I + (size_t)half * I + i0 + wave * 4 + min(hl, 3);
    crow[r] = a.gu_codes + grow * (H / 2);
    srow[r] = a.gu_scales + grow * scale_row_bytes<MODE>(H);
  }
  // Unconditional loads: lanes past the row's chunks or the wave's four rows
  // read a clamped (valid) address and their values are never used.  A load
  // under a branch makes the compiler merge its result with the branch's other
  // value, and that copy waits for the load before the next one is issued.
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = min(kl + j * LPR, NC - 1);
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      wq[r][j] = ld_stream128(crow[r] + 16 * c);
      wsc[r][j] = chunk_scale<MODE>(srow[r], c, a.tiled ? NC : 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);   // every load issued before any use of one
  // Up to max_cols tokens in all (16/8-bit modes): x of every token goes to LDS
  // now (unless the caller staged it), with no wait for the pairs' tokens, and
  // columns index it by token.
  if (!XS && by_token) stage_gateup_cols<MODE, true>(a, e, 0, 0, a.T, nullptr, lds);
  const float wsc_m = MODE == kModeQ4 ? 1.0f : a.gu_wscale[2 * e + half];   // (q4: no multiplier)
  const float in_m = MODE == MOE_A4 ? a.gu_inscale[2 * e + half] : 1.0f;
  const float dn_in = MODE == MOE_A4 ? a.dn_inscale[e] : 0.0f;   // the intermediate's input scale

  for (int c0 = 0; c0 < ne; c0 += max_cols) {
    const int ncol = min(max_cols, ne - c0);
    if (!XS || c0 > 0) {   // (XS: the first group's tokens went to LDS before the loads)
      if (threadIdx.x < ncol) s_tok[threadIdx.x] = pair / a.k;
      __syncthreads();
      if constexpr (MODE == MOE_A4 && QX) stage_gateup_quant_a4(a, e, row0, c0, ncol, s_tok, lds, rb == 0);
      else if (!by_token) stage_gateup_cols<MODE>(a, e, row0, c0, ncol, s_tok, lds);
      __syncthreads();
    }
    for (int col = 0; col < ncol; ++col) {
      const uint8_t* xc = lds + (size_t)(by_token ? s_tok[col] : col) * NC * S;
      // chunk-outer: each activation chunk is read from LDS once for all rows;
      // every row still sums its chunks in ascending order
      float acc[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = kl + j * LPR;
        if (c < NC) {
#pragma unroll
          for (int r = 0; r < RP; ++r)
            acc[r] += chunk_dot<MODE>(wq[r][j], wsc[r][j], xc + (size_t)c * S, half);
        }
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const float v = lane_group_sum<LPR>(acc[r]);
        const int hl = slot * RP + r;
        if (kl == 0 && hl < 4) part[col][wave * 4 + hl][half] = v * wsc_m * in_m;
      }
    }
    __syncthreads();
    // SwiGLU and the intermediate in the mode's precision
    if (MODE == MOE_A16 && htag) {   // two h values per thread, as one tagged word
      for (int t = threadIdx.x; t < ncol * (kGuRows / 2); t += kTileThreads) {
        const int col = t / (kGuRows / 2), hr = 2 * (t % (kGuRows / 2));
        const uint32_t b0 = f32_to_bf16(swiglu(part[col][hr][0], part[col][hr][1]));
        const uint32_t b1 = f32_to_bf16(swiglu(part[col][hr + 1][0], part[col][hr + 1][1]));
        const size_t at = (size_t)(row0 + c0 + col) * I + i0 + hr;
        __hip_atomic_store(&htag[at / 2], (uint64_t)(b0 | b1 << 16) << 32 | epoch, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        hst32<COH>(a.h_codes, 2 * at, b0 | b1 << 16);
      }
    } else {
      for (int t = threadIdx.x; t < ncol * kGuRows; t += kTileThreads) {
        const int col = t / kGuRows, hr = t % kGuRows;
        const float h = swiglu(part[col][hr][0], part[col][hr][1]);
        if (MODE == MOE_A16) {
          hst16<COH>(a.h_codes, 2 * ((size_t)(row0 + c0 + col) * I + i0 + hr), (uint16_t)f32_to_bf16(h));
        } else if (MODE == kModeQ4) {   // the fp16 intermediate
          hst16<COH>(a.h_codes, 2 * ((size_t)(row0 + c0 + col) * I + i0 + hr), (uint16_t)f32_to_f16_bits(h));
        } else {
          hbuf[col][hr] = h;
        }
      }
    }
    if (MODE == MOE_A8 || MODE == MOE_A4) {
      __syncthreads();
      if (threadIdx.x < ncol) {
        const int col = threadIdx.x;
        const size_t r = (size_t)(row0 + c0 + col);
        if (MODE == MOE_A8) {
          uint32_t w4[4];
          const float sc = fp8_quant16(hbuf[col], w4);
          hst128<COH>(a.h_codes, r * I + i0, make_uint4(w4[0], w4[1], w4[2], w4[3]));
          hst32<COH>(a.h_scales, 4 * (r * (I / 16) + rb), __builtin_bit_cast(uint32_t, sc));
          if (htag) {   // the block's 16 codes and its scale as tagged words
            uint64_t* hw = htag + r * h8_words(I);
#pragma unroll
            for (int q = 0; q < 4; ++q)
              __hip_atomic_store(&hw[i0 / 4 + q], (uint64_t)w4[q] << 32 | epoch, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&hw[I / 4 + rb], (uint64_t)__builtin_bit_cast(uint32_t, sc) << 32 | epoch,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        } else {
          uint32_t lo, hi;
          const uint32_t sc = nvfp4_quant16(hbuf[col], dn_in, lo, hi);
          hst64<COH>(a.h_codes, r * (I / 2) + i0 / 2, make_uint2(lo, hi));
          hst8<COH>(a.h_scales, r * (I / 16) + rb, (uint8_t)sc);
        }
      }
    }
    if (c0 + max_cols < ne) pair = col_pair(c0 + max_cols);
  }
}

// ------------------------------------------------------------------ down
// One tile: 64 output rows (rb) of expert e; 4 waves x 16 output rows.
// wait() runs after the weight loads are issued and before the intermediate is
// read: the fused decode kernel waits there for its expert's gate/up tiles.
template <int MODE, int LPR, int CPL, bool COH, typename Wait>
// With ytag, every output value is also published as one 64-bit word
// ytag[row * H + o] = (value bits << 32) | epoch (one atomic store), for a
// consumer that polls the words instead of waiting on a counter.
// With htag (16- and 8-bit activations), h is read from the tagged words that
// gateup_tile publishes, each polled until it carries epoch (a bounded wait on
// abort_word, see Patience; a thread that gives up uses whatever it read).
__device__ __forceinline__ void down_tile(const FfnArgs& a, int e, int row0, int ne, int rb,
                                          int max_cols, uint8_t* lds, Wait&& wait,
                                          uint64_t* ytag = nullptr, uint32_t epoch = 0u,
                                          const uint64_t* htag = nullptr, uint32_t* abort_word = nullptr) {
  __shared__ float outb[8][kDnRows];
  constexpr int S = ChunkLds<MODE>::kStride;
  constexpr int SLOTS = 64 / LPR;
  constexpr int RP = 16 / SLOTS;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int H = a.H, I = a.I, NC = I / 32;
  const int o0 = rb * kDnRows;
  const int slot = lane / LPR, kl = lane % LPR;

  uint4 wq[RP][CPL];
  uint32_t wsc[RP][CPL];
#pragma unroll
  // unconditional loads from clamped addresses, as in gateup_tile: rows past H
  // are computed from a valid row and never stored
  for (int r = 0; r < RP; ++r) {
    const int orow = o0 + wave * 16 + slot * RP + r;
    const size_t grow = (size_t)e * H + min(orow, H - 1);
    const uint8_t* crow = a.dn_codes + grow * (I / 2);
    const uint8_t* srow = a.dn_scales + grow * scale_row_bytes<MODE>(I);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = min(kl + j * LPR, NC - 1);
      wq[r][j] = ld_stream128(crow + 16 * c);
      wsc[r][j] = chunk_scale<MODE>(srow, c, a.tiled ? NC : 0);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  const float scale = MODE == kModeQ4 ? 1.0f : a.dn_wscale[e] * (MODE == MOE_A4 ? a.dn_inscale[e] : 1.0f);
  wait();

  for (int c0 = 0; c0 < ne; c0 += max_cols) {
    const int ncol = min(max_cols, ne - c0);
    __syncthreads();
    if (MODE == MOE_A16 && htag) {
      // word p of a row holds h 2p, 2p+1: chunk p / 16, bytes 4 (p % 16) of it
      const int half = I / 2;
      Patience pat;   // one budget for all of this thread's words
      bool gave_up = false;
      for (int i = threadIdx.x; i < ncol * half; i += kTileThreads) {
        const int col = i / half, p = i % half;
        const uint64_t* w = htag + (size_t)(row0 + c0 + col) * half + p;
        uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while ((uint32_t)v != epoch && !gave_up) {
          if (pat.expired(abort_word)) {
            gave_up = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *reinterpret_cast<uint32_t*>(lds + ((size_t)col * NC + p / 16) * S + 4 * (p % 16)) = (uint32_t)(v >> 32);
      }
    } else if (MODE == MOE_A8 && htag) {
      // a row's words: codes 4p .. 4p+3 in word p < I/4 (chunk p / 8, bytes
      // 4 (p % 8) of it), then block b's scale (chunk b / 2, after its codes)
      const int nw = h8_words(I), ncw = I / 4;
      Patience pat;
      bool gave_up = false;
      for (int i = threadIdx.x; i < ncol * nw; i += kTileThreads) {
        const int col = i / nw, p = i % nw;
        const uint64_t* w = htag + (size_t)(row0 + c0 + col) * nw + p;
        uint64_t v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while ((uint32_t)v != epoch && !gave_up) {
          if (pat.expired(abort_word)) {
            gave_up = true;
            break;
          }
          __builtin_amdgcn_s_sleep(1);
          v = __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        uint8_t* dst = p < ncw ? lds + ((size_t)col * NC + p / 8) * S + 4 * (p % 8)
                               : lds + ((size_t)col * NC + (p - ncw) / 2) * S + 32 + 4 * ((p - ncw) % 2);
        *reinterpret_cast<uint32_t*>(dst) = (uint32_t)(v >> 32);
      }
    } else {
      stage_down_cols<MODE, COH>(a, row0, c0, ncol, lds);
    }
    __syncthreads();
    for (int col = 0; col < ncol; ++col) {
      const uint8_t* xc = lds + (size_t)col * NC * S;
      float acc[RP];
#pragma unroll
      for (int r = 0; r < RP; ++r) acc[r] = 0.0f;
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = kl + j * LPR;
        if (c < NC) {
#pragma unroll
          for (int r = 0; r < RP; ++r)
            acc[r] += chunk_dot<MODE>(wq[r][j], wsc[r][j], xc + (size_t)c * S, 0);
        }
      }
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        const float v = lane_group_sum<LPR>(acc[r]);
        if (kl == 0) outb[col][wave * 16 + slot * RP + r] = v * scale;
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < ncol * kDnRows; t += kTileThreads) {
      const int col = t / kDnRows, o = t % kDnRows;
      if (o0 + o < H) {
        const size_t at = (size_t)(row0 + c0 + col) * H + o0 + o;
        const uint32_t bits = __builtin_bit_cast(uint32_t, outb[col][o]);
        if (ytag) __hip_atomic_store(&ytag[at], (uint64_t)bits << 32 | epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        hst32<COH>(a.y, 4 * at, bits);
      }
    }
  }
}

}  // namespace moe
