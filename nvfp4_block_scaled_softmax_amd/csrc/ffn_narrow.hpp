// The narrow (few-column) expert tiles as device functions, shared by the
// per-stage kernels (ffn_narrow.hip) and the fused decode kernel (decode.hip).
#pragma once
#include "ffn_common.hpp"

namespace moe {

constexpr int kGuRows = 16;    // h rows per gate/up workgroup (= one quantization block)
constexpr int kDnRows = 64;    // output rows per down workgroup
constexpr int kLdsBudget = 60 * 1024;

template <int MODE>
__device__ void stage_gateup_cols(const FfnArgs& a, int e, int row0, int c0, int ncol,
                                  uint8_t* lds) {
  constexpr int S = ChunkLds<MODE>::kStride;
  const int H = a.H, NC = H / 32;
  const int tid = threadIdx.x;
  if (MODE == MOE_A16) {
    // 4 x 16 B per chunk
    for (int i = tid; i < ncol * NC * 4; i += blockDim.x) {
      const int col = i / (NC * 4), rem = i % (NC * 4), ch = rem / 4, q = rem % 4;
      const int t = a.sorted_pairs[row0 + c0 + col] / a.k;
      const uint4 v = reinterpret_cast<const uint4*>(a.x + (size_t)t * H)[ch * 4 + q];
      *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
    }
  } else if (MODE == MOE_A8) {
    const float* xs = static_cast<const float*>(a.xq_scales);
    for (int i = tid; i < ncol * NC * 3; i += blockDim.x) {
      const int col = i / (NC * 3), rem = i % (NC * 3), ch = rem / 3, q = rem % 3;
      const int t = a.sorted_pairs[row0 + c0 + col] / a.k;
      uint8_t* dst = lds + ((size_t)col * NC + ch) * S;
      if (q < 2) {
        *reinterpret_cast<uint4*>(dst + 16 * q) =
            reinterpret_cast<const uint4*>(a.xq_codes + (size_t)t * H)[ch * 2 + q];
      } else {
        *reinterpret_cast<float2*>(dst + 32) =
            *reinterpret_cast<const float2*>(xs + (size_t)t * (H / 16) + ch * 2);
      }
    }
  } else {
    const uint8_t* xs = static_cast<const uint8_t*>(a.xq_scales);
    for (int i = tid; i < ncol * NC * 3; i += blockDim.x) {
      const int col = i / (NC * 3), rem = i % (NC * 3), ch = rem / 3, q = rem % 3;
      const size_t r = (size_t)(row0 + c0 + col);
      uint8_t* dst = lds + ((size_t)col * NC + ch) * S;
      if (q < 2) {   // q = matrix (0 gate, 1 up)
        *reinterpret_cast<uint4*>(dst + 16 * q) =
            reinterpret_cast<const uint4*>(a.xq_codes + (r * 2 + q) * (H / 2))[ch];
      } else {
        const uint16_t sg = *reinterpret_cast<const uint16_t*>(xs + (r * 2 + 0) * (H / 16) + 2 * ch);
        const uint16_t su = *reinterpret_cast<const uint16_t*>(xs + (r * 2 + 1) * (H / 16) + 2 * ch);
        *reinterpret_cast<uint32_t*>(dst + 32) = (uint32_t)sg | ((uint32_t)su << 16);
      }
    }
  }
}

template <int MODE, bool COH>
__device__ void stage_down_cols(const FfnArgs& a, int row0, int c0, int ncol, uint8_t* lds) {
  constexpr int S = ChunkLds<MODE>::kStride;
  const int I = a.I, NC = I / 32;
  const int tid = threadIdx.x;
  if (MODE == MOE_A16) {
    const uint16_t* h = reinterpret_cast<const uint16_t*>(a.h_codes);
    for (int i = tid; i < ncol * NC * 4; i += blockDim.x) {
      const int col = i / (NC * 4), rem = i % (NC * 4), ch = rem / 4, q = rem % 4;
      const uint4 v = hld128<COH>(h, 2 * ((size_t)(row0 + c0 + col) * I) + 16 * (ch * 4 + q));
      *reinterpret_cast<uint4*>(lds + ((size_t)col * NC + ch) * S + 16 * q) = v;
    }
  } else if (MODE == MOE_A8) {
    const float* hs = static_cast<const float*>(a.h_scales);
    for (int i = tid; i < ncol * NC * 3; i += blockDim.x) {
      const int col = i / (NC * 3), rem = i % (NC * 3), ch = rem / 3, q = rem % 3;
      const size_t r = (size_t)(row0 + c0 + col);
      uint8_t* dst = lds + ((size_t)col * NC + ch) * S;
      if (q < 2)
        *reinterpret_cast<uint4*>(dst + 16 * q) = hld128<COH>(a.h_codes, r * I + 16 * (ch * 2 + q));
      else
        *reinterpret_cast<uint2*>(dst + 32) = hld64<COH>(hs, 4 * (r * (I / 16) + ch * 2));
    }
  } else {
    const uint8_t* hs = static_cast<const uint8_t*>(a.h_scales);
    for (int i = tid; i < ncol * NC * 2; i += blockDim.x) {
      const int col = i / (NC * 2), rem = i % (NC * 2), ch = rem / 2, q = rem % 2;
      const size_t r = (size_t)(row0 + c0 + col);
      uint8_t* dst = lds + ((size_t)col * NC + ch) * S;
      if (q == 0)
        *reinterpret_cast<uint4*>(dst) = hld128<COH>(a.h_codes, r * (I / 2) + 16 * ch);
      else
        *reinterpret_cast<uint32_t*>(dst + 32) = hld16<COH>(hs, r * (I / 16) + 2 * ch);
    }
  }
}

// ------------------------------------------------------------------ gate/up
// One tile: 16 h rows (rb) of expert e; 4 waves; wave w owns h rows 4w..4w+3 of
// the tile; lanes 0-31 read the gate rows, lanes 32-63 the up rows; within a
// half-wave, LPR lanes share a row and each reads CPL chunks of it.
template <int MODE, int LPR, int CPL, bool COH = false>
__device__ __forceinline__ void gateup_tile(const FfnArgs& a, int e, int row0, int ne, int rb,
                                            int max_cols, uint8_t* lds) {
  __shared__ float part[8][kGuRows][2];
  __shared__ float hbuf[8][kGuRows];
  constexpr int S = ChunkLds<MODE>::kStride;
  constexpr int SLOTS = 32 / LPR;
  constexpr int RP = (4 + SLOTS - 1) / SLOTS;
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int H = a.H, I = a.I, NC = H / 32;
  const int i0 = rb * kGuRows;
  const int half = lane >> 5, l32 = lane & 31, slot = l32 / LPR, kl = l32 % LPR;

  // this lane's weight chunks: RP h rows x CPL chunks, all loads in flight together
  uint4 wq[RP][CPL];
  uint32_t wsc[RP][CPL];
#pragma unroll
  for (int r = 0; r < RP; ++r) {
    const int hl = slot * RP + r;  // h row within the wave's four
    const size_t grow = (size_t)e * 2 * I + (size_t)half * I + i0 + wave * 4 + hl;
    const uint8_t* crow = a.gu_codes + grow * (H / 2);
    const uint8_t* srow = a.gu_scales + grow * (H / 16);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = kl + j * LPR;
      if (hl < 4 && c < NC) {
        wq[r][j] = *reinterpret_cast<const uint4*>(crow + 16 * c);
        wsc[r][j] = *reinterpret_cast<const uint16_t*>(srow + 2 * c);
      } else {
        wq[r][j] = make_uint4(0u, 0u, 0u, 0u);
        wsc[r][j] = 0u;
      }
    }
  }
  const float wsc_m = a.gu_wscale[2 * e + half];
  const float in_m = MODE == MOE_A4 ? a.gu_inscale[2 * e + half] : 1.0f;

  for (int c0 = 0; c0 < ne; c0 += max_cols) {
    const int ncol = min(max_cols, ne - c0);
    __syncthreads();
    stage_gateup_cols<MODE>(a, e, row0, c0, ncol, lds);
    __syncthreads();
    for (int col = 0; col < ncol; ++col) {
      const uint8_t* xc = lds + (size_t)col * NC * S;
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = kl + j * LPR;
          if (c < NC) acc += chunk_dot<MODE>(wq[r][j], wsc[r][j], xc + (size_t)c * S, half);
        }
        acc = group_sum<LPR>(acc);
        const int hl = slot * RP + r;
        if (kl == 0 && hl < 4) part[col][wave * 4 + hl][half] = acc * wsc_m * in_m;
      }
    }
    __syncthreads();
    // SwiGLU and the intermediate in the mode's precision
    for (int t = threadIdx.x; t < ncol * kGuRows; t += blockDim.x) {
      const int col = t / kGuRows, hr = t % kGuRows;
      const float h = swiglu(part[col][hr][0], part[col][hr][1]);
      if (MODE == MOE_A16) {
        hst16<COH>(a.h_codes, 2 * ((size_t)(row0 + c0 + col) * I + i0 + hr), (uint16_t)f32_to_bf16(h));
      } else {
        hbuf[col][hr] = h;
      }
    }
    if (MODE != MOE_A16) {
      __syncthreads();
      if (threadIdx.x < ncol) {
        const int col = threadIdx.x;
        const size_t r = (size_t)(row0 + c0 + col);
        if (MODE == MOE_A8) {
          uint32_t w4[4];
          const float sc = fp8_quant16(hbuf[col], w4);
          hst128<COH>(a.h_codes, r * I + i0, make_uint4(w4[0], w4[1], w4[2], w4[3]));
          hst32<COH>(a.h_scales, 4 * (r * (I / 16) + rb), __builtin_bit_cast(uint32_t, sc));
        } else {
          uint32_t lo, hi;
          const uint32_t sc = nvfp4_quant16(hbuf[col], a.dn_inscale[e], lo, hi);
          hst64<COH>(a.h_codes, r * (I / 2) + i0 / 2, make_uint2(lo, hi));
          hst8<COH>(a.h_scales, r * (I / 16) + rb, (uint8_t)sc);
        }
      }
    }
  }
}

// ------------------------------------------------------------------ down
// One tile: 64 output rows (rb) of expert e; 4 waves x 16 output rows.
// wait() runs after the weight loads are issued and before the intermediate is
// read: the fused decode kernel waits there for the expert's gate/up tiles.
template <int MODE, int LPR, int CPL, bool COH, typename Wait>
__device__ __forceinline__ void down_tile(const FfnArgs& a, int e, int row0, int ne, int rb,
                                          int max_cols, uint8_t* lds, Wait&& wait) {
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
  for (int r = 0; r < RP; ++r) {
    const int orow = o0 + wave * 16 + slot * RP + r;
    const size_t grow = (size_t)e * H + orow;
    const uint8_t* crow = a.dn_codes + grow * (I / 2);
    const uint8_t* srow = a.dn_scales + grow * (I / 16);
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = kl + j * LPR;
      if (orow < H && c < NC) {
        wq[r][j] = *reinterpret_cast<const uint4*>(crow + 16 * c);
        wsc[r][j] = *reinterpret_cast<const uint16_t*>(srow + 2 * c);
      } else {
        wq[r][j] = make_uint4(0u, 0u, 0u, 0u);
        wsc[r][j] = 0u;
      }
    }
  }
  const float scale = a.dn_wscale[e] * (MODE == MOE_A4 ? a.dn_inscale[e] : 1.0f);
  wait();

  for (int c0 = 0; c0 < ne; c0 += max_cols) {
    const int ncol = min(max_cols, ne - c0);
    __syncthreads();
    stage_down_cols<MODE, COH>(a, row0, c0, ncol, lds);
    __syncthreads();
    for (int col = 0; col < ncol; ++col) {
      const uint8_t* xc = lds + (size_t)col * NC * S;
#pragma unroll
      for (int r = 0; r < RP; ++r) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = kl + j * LPR;
          if (c < NC) acc += chunk_dot<MODE>(wq[r][j], wsc[r][j], xc + (size_t)c * S, 0);
        }
        acc = group_sum<LPR>(acc);
        if (kl == 0) outb[col][wave * 16 + slot * RP + r] = acc * scale;
      }
    }
    __syncthreads();
    for (int t = threadIdx.x; t < ncol * kDnRows; t += blockDim.x) {
      const int col = t / kDnRows, o = t % kDnRows;
      if (o0 + o < H)
        hst32<COH>(a.y, 4 * ((size_t)(row0 + c0 + col) * H + o0 + o), __builtin_bit_cast(uint32_t, outb[col][o]));
    }
  }
}

}  // namespace moe
