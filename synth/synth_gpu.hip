// Device build of the seeded generator in synth_core.h (hipcc -ffp-contract=off).
// Bit-identical to the host build: only IEEE double + - * / and sqrt are used.
#include <hip/hip_runtime.h>
#include "synth_core.h"

template <bool BF16>
__global__ void __launch_bounds__(256) k_synth_normal(void* out, uint64_t i0, uint64_t n,
                                                      uint32_t seed, uint32_t tag, uint32_t layer,
                                                      uint32_t expert0, uint32_t matrix,
                                                      double sigma) {
  const uint32_t e = blockIdx.y;
  const uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x + i0 / 4;
  const uint64_t j1 = (i0 + n + 3) / 4;
  if (j >= j1) return;
  float v[4];
  syn_normal4(seed, tag, layer, expert0 + e, matrix, j, sigma, v);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint64_t gi = j * 4 + q;
    if (gi >= i0 && gi < i0 + n) {
      const size_t o = (size_t)e * n + (gi - i0);
      if (BF16) ((uint16_t*)out)[o] = syn_f32_to_bf16(v[q]);
      else ((float*)out)[o] = v[q];
    }
  }
}

template <bool BF16>
static int launch(void* out, uint64_t i0, uint64_t n, uint32_t seed, uint32_t tag, uint32_t layer,
                  uint32_t expert0, uint32_t n_expert, uint32_t matrix, double sigma,
                  hipStream_t s) {
  if (!out || n == 0 || n_expert == 0 || n_expert > 65535u) return -1;
  const uint64_t nj = (i0 + n + 3) / 4 - i0 / 4;
  const uint64_t nb = (nj + 255) / 256;
  if (nb > 0x7FFFFFFFull) return -1;
  hipLaunchKernelGGL(k_synth_normal<BF16>, dim3((unsigned)nb, n_expert), dim3(256), 0, s, out, i0,
                     n, seed, tag, layer, expert0, matrix, sigma);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

extern "C" int synth_gpu_normal_f32(float* out, uint64_t i0, uint64_t n, uint32_t seed,
                                    uint32_t tag, uint32_t layer, uint32_t expert0,
                                    uint32_t n_expert, uint32_t matrix, double sigma,
                                    hipStream_t s) {
  return launch<false>(out, i0, n, seed, tag, layer, expert0, n_expert, matrix, sigma, s);
}

extern "C" int synth_gpu_normal_bf16(uint16_t* out, uint64_t i0, uint64_t n, uint32_t seed,
                                     uint32_t tag, uint32_t layer, uint32_t expert0,
                                     uint32_t n_expert, uint32_t matrix, double sigma,
                                     hipStream_t s) {
  return launch<true>(out, i0, n, seed, tag, layer, expert0, n_expert, matrix, sigma, s);
}
