// Device helpers of the NVFP4 expert layer for gfx950 (CDNA4, wave64).
//
// Element formats: E2M1 4-bit codes (sign bit 3; magnitudes 0, 0.5, 1, 1.5, 2,
// 3, 4, 6) and E4M3 8-bit codes (OCP E4M3: bias 7, subnormals, S.1111.111 NaN,
// max 448), as in the OCP Microscaling and OFP8 specifications; the expert
// format that uses them is described on the page "Qwen3.8-Flash-Next NVIDIA
// NVFP4 for Infernix (bit-exact)", section "What is bit-exact and what is
// quantized".
//
// Decoding uses the CDNA4 conversion instructions (exact for these formats;
// v_cvt_scalef32_* is called with scale 1.0 because its scale operand only
// contributes a power of two).  Rounding to E4M3 / E2M1 / bf16 is written out
// in integer and compare operations so that ties, saturation and the sign of
// zero are exactly the documented ones.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ bit casts
template <typename To, typename From>
__device__ __forceinline__ To bitcast(const From& f) {
  static_assert(sizeof(To) == sizeof(From), "size");
  To t;
  __builtin_memcpy(&t, &f, sizeof(To));
  return t;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// ------------------------------------------------------------------ decoding
// E4M3 byte (bits 7..0 of b) -> fp32, exact.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
}

// The two E2M1 codes in byte `sel` of w (low nibble first) as f16 / bf16 pairs.
template <int SEL>
__device__ __forceinline__ f16x2 e2m1x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ bf16x2 e2m1x2_to_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, SEL);
}
// Two E4M3 codes in half `HI` of w as an f16 pair (exact: E4M3 fits f16).
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// ------------------------------------------------------------------ rounding
// fp32 -> E4M3 code: nearest, ties to even code, |v| >= 448 (and inf) saturates
// to 0x7E, sign kept (negative zero -> 0x80), NaN -> 0x00.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0u;                  // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;        // >= 448
  if (a >= 0x3C800000u) {                          // >= 2^-6: normal E4M3
    const uint32_t e = (a >> 23) - 120u;           // E4M3 exponent field
    const uint32_t keep = (a >> 20) & 7u, rem = a & 0xFFFFFu;
    uint32_t code = (e << 3) | keep;
    code += (rem > 0x80000u) || (rem == 0x80000u && (keep & 1u));
    return sign | code;
  }
  // subnormal E4M3: multiples of 2^-9; the scaling by 2^9 is exact
  const float n = __builtin_rintf(__uint_as_float(a) * 512.0f);
  return sign | (uint32_t)n;                       // n in [0, 8]; 8 is 0x08 = 2^-6
}

// fp32 -> E2M1 code: nearest, ties to even code, |q| > 6 saturates, sign kept.
__device__ __forceinline__ uint32_t f32_to_e2m1(float q) {
  const float a = __builtin_fabsf(q);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(q) >> 28) & 8u);
}

// NVFP4 quantization of 16 fp32 values under global scale g: returns the E4M3
// block scale and the 16 codes packed as two 32-bit words (value 2i in the
// low nibble of byte i).  Each fp32 operation is one correctly rounded op, in
// the order t = (bamax / 6) / g, d = dec(s) * g, q = v / d.
__device__ __forceinline__ uint32_t nvfp4_quant16(const float* v, float g, uint32_t& lo,
                                                  uint32_t& hi) {
  float bamax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bamax = __builtin_fmaxf(bamax, __builtin_fabsf(v[i]));
  const float t = __fdiv_rn(__fdiv_rn(bamax, 6.0f), g);
  const uint32_t s = f32_to_e4m3(t);
  const float d = __fmul_rn(e4m3_to_f32(s), g);
  lo = 0u;
  hi = 0u;
  if (d > 0.0f) {
#pragma unroll
    for (int i = 0; i < 8; ++i) lo |= f32_to_e2m1(__fdiv_rn(v[i], d)) << (4 * i);
#pragma unroll
    for (int i = 0; i < 8; ++i) hi |= f32_to_e2m1(__fdiv_rn(v[8 + i], d)) << (4 * i);
  }
  return s;
}

// 8-bit mode of 16 fp32 values: fp32 scale s = bamax / 448, codes E4M3(v / s)
// packed four per 32-bit word (value i in byte i % 4 of word i / 4).
__device__ __forceinline__ float fp8_quant16(const float* v, uint32_t* w4) {
  float bamax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) bamax = __builtin_fmaxf(bamax, __builtin_fabsf(v[i]));
  const float s = __fdiv_rn(bamax, 448.0f);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t w = 0u;
    if (s > 0.0f) {
#pragma unroll
      for (int b = 0; b < 4; ++b) w |= f32_to_e4m3(__fdiv_rn(v[4 * q + b], s)) << (8 * b);
    }
    w4[q] = w;
  }
  return s;
}

// silu(g) * u in fp32: g / (1 + exp(-g)) * u.
__device__ __forceinline__ float swiglu(float g, float u) {
  return __fdiv_rn(g, 1.0f + expf(-g)) * u;
}

// ------------------------------------------------------------------ wave helpers
// Sum over aligned groups of N lanes (N a power of two <= 64).
template <int N>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = N / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Copies items 0..n-1 (item i: v = ld(i); st(i, v)) with the workgroup's NT
// threads, B loads in flight per thread before the first store: a staging loop
// that stored each value before the next load would pay one memory round trip
// per item per thread.
template <int NT, int B, typename Ld, typename St>
__device__ __forceinline__ void batched_copy(int n, Ld&& ld, St&& st) {
  using V = decltype(ld(0));
  for (int i0 = threadIdx.x; i0 < n; i0 += B * NT) {
    V v[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = i0 + b * NT;
      if (i < n) v[b] = ld(i);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int i = i0 + b * NT;
      if (i < n) st(i, v[b]);
    }
  }
}


// DPP lane moves within rows of 16 (gfx9 encodings): xor 1, xor 2, mirror in 8, mirror in 16.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

// Maximum over the wave, the same value in every lane: DPP within each row of
// 16 lanes, then the four row results through scalar reads.
__device__ __forceinline__ float wave_max(float v) {
  v = __builtin_fmaxf(v, dpp_f32<kDppXor1>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppXor2>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = __builtin_fmaxf(v, dpp_f32<kDppMirror>(v));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return __builtin_fmaxf(__builtin_fmaxf(r0, r1), __builtin_fmaxf(r2, r3));
}

// Sum over the wave in a fixed order, the same value in every lane.
// Sum over aligned groups of N lanes (N = 2 .. 32), every lane of a group
// receiving the group's total: DPP steps within rows of 16 lanes (pairs, quads,
// halves, rows), one lane shuffle to join two rows.
template <int N>
__device__ __forceinline__ float lane_group_sum(float v) {
  static_assert(N == 2 || N == 4 || N == 8 || N == 16 || N == 32, "group of 2..32 lanes");
  v += dpp_f32<kDppXor1>(v);
  if constexpr (N >= 4) v += dpp_f32<kDppXor2>(v);
  if constexpr (N >= 8) v += dpp_f32<kDppHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<kDppMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16, kWave);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Index of the s-th expert (0-based) with a non-empty segment, or -1; wave-wide,
// every lane gets the answer.  offsets has E + 1 entries.
__device__ __forceinline__ int find_active_expert(const int32_t* offsets, int E, int s) {
  const int lane = lane_id();
  int seen = 0;
  for (int base = 0; base < E; base += kWave * 8) {
    int cnt = 0;
    int e0 = base + lane * 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i;
      if (e < E) cnt += offsets[e + 1] > offsets[e];
    }
    // inclusive prefix over lanes
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int y = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += y;
    }
    const int total = __shfl(incl, kWave - 1, kWave);
    const int target = s - seen;
    if (target < total) {
      // the lane whose range holds the target-th active expert
      const int excl = incl - cnt;
      int found = -1;
      if (target >= excl && target < incl) {
        int r = target - excl;
        for (int i = 0; i < 8; ++i) {
          const int e = e0 + i;
          if (e < E && offsets[e + 1] > offsets[e]) {
            if (r == 0) { found = e; break; }
            --r;
          }
        }
      }
      // broadcast from the lane that found it
      const unsigned long long m = __ballot(found >= 0);
      const int src = __ffsll((long long)m) - 1;
      return __shfl(found, src, kWave);
    }
    seen += total;
  }
  return -1;
}


// ---------------------------------------------------------------------------
// Accesses for data one workgroup hands to another within a kernel.  The L2s
// of the XCDs are not coherent with each other; with COH these go through
// buffer instructions whose cache policy (sc1, device scope) writes through /
// reads past the XCD-local caches, so the handoff needs no L2 write-back or
// invalidate.  Without COH they are plain accesses.  base must be
// wave-uniform; byte offsets stay below 2^31.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7FFFFFFF, 0x00020000);
}
constexpr int kCohPolicy = 16;   // sc1

template <bool COH>
__device__ __forceinline__ void hst8(void* base, size_t off, uint8_t v) {
  if constexpr (COH) __builtin_amdgcn_raw_buffer_store_b8(v, coh_rsrc(base), (int)off, 0, kCohPolicy);
  else static_cast<uint8_t*>(base)[off] = v;
}
template <bool COH>
__device__ __forceinline__ void hst16(void* base, size_t off, uint16_t v) {
  if constexpr (COH) __builtin_amdgcn_raw_buffer_store_b16(v, coh_rsrc(base), (int)off, 0, kCohPolicy);
  else *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(base) + off) = v;
}
template <bool COH>
__device__ __forceinline__ void hst32(void* base, size_t off, uint32_t v) {
  if constexpr (COH) __builtin_amdgcn_raw_buffer_store_b32(v, coh_rsrc(base), (int)off, 0, kCohPolicy);
  else *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + off) = v;
}
template <bool COH>
__device__ __forceinline__ void hst64(void* base, size_t off, uint2 v) {
  typedef unsigned v2u __attribute__((ext_vector_type(2)));
  if constexpr (COH)
    __builtin_amdgcn_raw_buffer_store_b64(v2u{v.x, v.y}, coh_rsrc(base), (int)off, 0, kCohPolicy);
  else *reinterpret_cast<uint2*>(static_cast<uint8_t*>(base) + off) = v;
}
template <bool COH>
__device__ __forceinline__ void hst128(void* base, size_t off, uint4 v) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  if constexpr (COH)
    __builtin_amdgcn_raw_buffer_store_b128(v4u{v.x, v.y, v.z, v.w}, coh_rsrc(base), (int)off, 0, kCohPolicy);
  else *reinterpret_cast<uint4*>(static_cast<uint8_t*>(base) + off) = v;
}
// Loads of data that a call reads once (expert weights, router rows):
// non-temporal, so that streaming them does not displace what the caches hold
// for the rest of the call and the next one (code, arguments, activations).
__device__ __forceinline__ uint4 ld_stream128(const void* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t ld_stream16(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}

template <bool COH>
__device__ __forceinline__ uint16_t hld16(const void* base, size_t off) {
  if constexpr (COH) return __builtin_amdgcn_raw_buffer_load_b16(coh_rsrc(base), (int)off, 0, kCohPolicy);
  else return *reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(base) + off);
}
template <bool COH>
__device__ __forceinline__ uint32_t hld32(const void* base, size_t off) {
  if constexpr (COH) return __builtin_amdgcn_raw_buffer_load_b32(coh_rsrc(base), (int)off, 0, kCohPolicy);
  else return *reinterpret_cast<const uint32_t*>(static_cast<const uint8_t*>(base) + off);
}
template <bool COH>
__device__ __forceinline__ uint2 hld64(const void* base, size_t off) {
  if constexpr (COH) {
    return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(coh_rsrc(base), (int)off, 0, kCohPolicy));
  } else {
    return *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + off);
  }
}
template <bool COH>
__device__ __forceinline__ uint4 hld128(const void* base, size_t off) {
  if constexpr (COH) return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(coh_rsrc(base), (int)off, 0, kCohPolicy));
  else return *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(base) + off);
}

// Waits until every vector memory access this wave issued has completed
// (s_waitcnt vmcnt(0); the other counters untouched).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// A bounded wait between workgroups of one launch.  It gives up when the abort
// word (a counter in the caller's workspace) is non-zero, which means another
// wait of the call, or of an earlier call on the same workspace, has given up;
// or when kWaitTicks of the 100 MHz real-time counter have passed since it
// began, and then it bumps the abort word itself.  So one stalled producer ends
// every wait of the launch within one check, and the count stays non-zero (the
// workspace must be zero-filled again) for the host to see.  The word and the
// clock are checked every 32nd poll; a poll loop calls expired() once per poll.
constexpr uint64_t kWaitTicks = 1ull << 26;   // ~0.67 s; a correct call waits microseconds

struct Patience {
  uint64_t t0;
  uint32_t polls;
  __device__ __forceinline__ Patience() : t0(__builtin_amdgcn_s_memrealtime()), polls(0u) {}
  __device__ __forceinline__ bool expired(uint32_t* abort_word) {
    if ((++polls & 31u) != 0u) return false;
    if (__hip_atomic_load(abort_word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 < kWaitTicks) return false;
    __hip_atomic_fetch_add(abort_word, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  }
};

// ------------------------------------------------------------------ q4_g64_fp16
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);   // v_cvt_f16_f32: nearest even
}

// Eight 16-bit values in element order (v.x = e0 | e1 << 16, ...) rearranged
// into the pairs (e0, e4), (e1, e5), (e2, e6), (e3, e7): the order in which
// q4_expand_pair takes the nibbles of one code dword.
__device__ __forceinline__ uint4 pair_by_nibble(uint4 v) {
  return make_uint4((v.x & 0xFFFFu) | (v.z << 16), (v.x >> 16) | (v.z & 0xFFFF0000u),
                    (v.y & 0xFFFFu) | (v.w << 16), (v.y >> 16) | (v.w & 0xFFFF0000u));
}

// Eight bf16 values in element order as fp16 (nearest even), paired as above.
__device__ __forceinline__ uint4 bf16x8_to_f16x8_paired(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = f32_to_f16_bits(bf16_to_f32(w[i] & 0xFFFFu)) | (f32_to_f16_bits(bf16_to_f32(w[i] >> 16)) << 16);
  return pair_by_nibble(make_uint4(o[0], o[1], o[2], o[3]));
}

// Two int4 codes of a dword (nibbles S and S + 4) as exact fp16 integers: the
// code xor 8 (offset binary u = q + 8) under the exponent of 1024 is 1024 + u
// exactly; one packed fp16 add of -1032 leaves q.  `ob` is the dword xor 0x88888888.
template <int S>
__device__ __forceinline__ f16x2 q4_expand_pair(uint32_t ob) {
  const f16x2 v = bitcast<f16x2>(((ob >> (4 * S)) & 0x000F000Fu) | 0x64006400u);
  const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  return v + bias;
}

// bf16 NaN: what a combine writes for an output whose inputs it gave up on.
constexpr uint16_t kBf16NaN = 0x7FC0;

}  // namespace moe
