// Per-element arithmetic of the dynamic quantizer, shared by the standalone
// quantizer kernels and the decode GEMM's fused-quantization prologue so
// that both produce the same codes and scales bit for bit:
//   s = fl(amax / Q), Q = 127 (int8) or 448 (E4M3); s = 1 when amax == 0;
//   code = round(fl(x / s)) (round-half-even), clamped to the format.
// Formats and granularity: [Summary] "Put algorithm selection inside the
// search space"; [Noticias] "El backend lineal de Helion / Alcance" (English
// summary of "Building a High-Performance and Portable vLLM Linear Backend
// with Helion"; "Helion entra al backend lineal de vLLM y supera a CUTLASS en
// Hopper").
#pragma once

#include "device_common.hpp"

namespace qlk {

__device__ __forceinline__ float abs_bf16_max8(const u32x4& v, float m) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m = fmaxf(m, bf16_to_f32(v[i] & 0x7fffu));
    m = fmaxf(m, bf16_to_f32((v[i] >> 16) & 0x7fffu));
  }
  return m;
}

// Eight codes of one 16-byte bf16 vector.  r = fl(1/s) selects the
// reciprocal path (exact at the code level for s >= 2^-96, see div_fast);
// r = 0 selects the division.  E4M3 codes come from the
// conversion instruction on the clamped quotients, two at a time.
template <int FMT>
__device__ __forceinline__ u32x2 quant8(const u32x4& v, float s, float r) {
  float t[8];
  if (r != 0.0f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[2 * i] = div_fast(bf16_to_f32(v[i] & 0xffffu), s, r);
      t[2 * i + 1] = div_fast(bf16_to_f32(v[i] >> 16), s, r);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      t[2 * i] = __fdiv_rn(bf16_to_f32(v[i] & 0xffffu), s);
      t[2 * i + 1] = __fdiv_rn(bf16_to_f32(v[i] >> 16), s);
    }
  }
  if constexpr (FMT == FMT_INT8) {
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = int8_code(t[i]);
    u32x2 out = {c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24), c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
    return out;
  } else {
    uint32_t lo = e4m3_pk2<false>(clamp448(t[0]), clamp448(t[1]), 0u);
    lo = e4m3_pk2<true>(clamp448(t[2]), clamp448(t[3]), lo);
    uint32_t hi = e4m3_pk2<false>(clamp448(t[4]), clamp448(t[5]), 0u);
    hi = e4m3_pk2<true>(clamp448(t[6]), clamp448(t[7]), hi);
    u32x2 out = {lo, hi};
    return out;
  }
}

template <int FMT>
__device__ __forceinline__ float scale_of(float amax) {
  const float Q = FMT == FMT_INT8 ? 127.0f : 448.0f;
  return amax > 0.0f ? __fdiv_rn(amax, Q) : 1.0f;
}

// Reciprocal for quant8: fl(1/s), or 0 (take the division) below 2^-96.
__device__ __forceinline__ float recip_of(float s) {
  return s >= FAST_DIV_MIN_SCALE ? __fdiv_rn(1.0f, s) : 0.0f;
}

}  // namespace qlk
