/* Host build of the seeded generator in synth_core.h (gcc, -ffp-contract=off). */
#include <stddef.h>
#include "synth_core.h"

/* out[e * n + i] = value i0 + i of stream (seed, tag, layer, expert0 + e, matrix). */
#define SYN_FILL_BODY(STORE)                                                          \
  for (uint32_t e = 0; e < n_expert; ++e) {                                           \
    uint64_t j0 = i0 / 4, j1 = (i0 + n + 3) / 4;                                      \
    _Pragma("omp parallel for schedule(static)")                                      \
    for (int64_t jj = (int64_t)j0; jj < (int64_t)j1; ++jj) {                          \
      float v[4];                                                                     \
      syn_normal4(seed, tag, layer, expert0 + e, matrix, (uint64_t)jj, sigma, v);     \
      for (int q = 0; q < 4; ++q) {                                                   \
        uint64_t gi = (uint64_t)jj * 4 + q;                                           \
        if (gi >= i0 && gi < i0 + n) { STORE; }                                       \
      }                                                                               \
    }                                                                                 \
  }

void synth_normal_f32(float* out, uint64_t i0, uint64_t n, uint32_t seed, uint32_t tag,
                      uint32_t layer, uint32_t expert0, uint32_t n_expert, uint32_t matrix,
                      double sigma) {
  SYN_FILL_BODY(out[(size_t)e * n + (gi - i0)] = v[q])
}

void synth_normal_bf16(uint16_t* out, uint64_t i0, uint64_t n, uint32_t seed, uint32_t tag,
                       uint32_t layer, uint32_t expert0, uint32_t n_expert, uint32_t matrix,
                       double sigma) {
  SYN_FILL_BODY(out[(size_t)e * n + (gi - i0)] = syn_f32_to_bf16(v[q]))
}

/* Raw Philox words: out[4j + w] = word w of counter (j, 0, expert | matrix<<16, layer). */
void synth_u32(uint32_t* out, uint64_t n4, uint32_t seed, uint32_t tag, uint32_t layer,
               uint32_t expert, uint32_t matrix) {
  for (uint64_t j = 0; j < n4; ++j) {
    syn_u32x4 r = syn_philox4x32_10((uint32_t)j, (uint32_t)(j >> 32),
                                    (expert & 0xFFFFu) | (matrix << 16), layer, seed, tag);
    for (int w = 0; w < 4; ++w) out[4 * j + w] = r.v[w];
  }
}

void synth_philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                  uint32_t k1, uint32_t* out4) {
  syn_u32x4 r = syn_philox4x32_10(c0, c1, c2, c3, k0, k1);
  for (int w = 0; w < 4; ++w) out4[w] = r.v[w];
}
