// Device helpers shared by the gfx950 kernels of the quantized linear:
// vector types, raw buffer loads with hardware out-of-range zeroing, matrix
// core wrappers, and the exact rounding helpers (bf16, E4M3, int8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "decode_args.hpp"

namespace qlk {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Byte offset that lies beyond every buffer's num_records: a raw buffer load
// at this offset returns zeros and issues no memory request.
constexpr uint32_t OOB = 0x80000000u;

// Raw buffer resource over `bytes` bytes starting at `p` (gfx9 word3).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Same with the non-temporal cache policy (data read once: weights).
__device__ __forceinline__ u32x4 bload16_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

__device__ __forceinline__ float bload_f32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ int bload_u8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (int)__builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// 32 bytes of one row of a 128-wide K block held by one lane: `lo` covers
// K offsets [16*g, 16*g+16) and `hi` [64+16*g, 64+16*g+16) of the block,
// g = lane / 16.  Activations and weights use the same lane -> K map, so the
// unscaled matrix core pairs equal K indices whatever its internal K order
// is.  This map is also the order in which the scaled E4M3 instruction
// groups K: the scale byte of lane 16*b + r multiplies K offsets
// [32*b, 32*b+32) of row r -- for b < 2 the `lo` pieces of lane groups 2b
// and 2b+1, for b >= 2 their `hi` pieces (checked on gfx950 with one-hot
// operands and a distinct power-of-two scale per lane group).
struct Frag {
  u32x4 lo, hi;
};

// int8 x int8 -> int32, 16x16 output tile, K = 64 per instruction.
__device__ __forceinline__ i32x4 mma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8((i32x4)a, (i32x4)b, c, 0, 0, 0);
}

// E4M3 x E4M3 -> fp32, 16x16 output tile, K = 128 per instruction (format
// selectors 0/0 = E4M3 for both operands; zero scale operands select the
// unscaled matrix-core instruction).
__device__ __forceinline__ f32x4 mma_f8(const Frag& a, const Frag& b, f32x4 c) {
  i32x8 av = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w,
              (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
  i32x8 bv = {(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w,
              (int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
}

// E4M3 x E4M3 -> fp32 with E8M0 block scales: `sa` / `sb` (low byte) are this
// lane's scales of the first / second operand, row l%16 and 32-wide K block
// l/16 of the 128-wide step; each product is multiplied by 2^(sa-127) *
// 2^(sb-127).
__device__ __forceinline__ f32x4 mma_f8_mx(const Frag& a, const Frag& b, f32x4 c, int sa, int sb) {
  i32x8 av = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w,
              (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
  i32x8 bv = {(int)b.lo.x, (int)b.lo.y, (int)b.lo.z, (int)b.lo.w,
              (int)b.hi.x, (int)b.hi.y, (int)b.hi.z, (int)b.hi.w};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, sa, 0, sb);
}

// E4M3 activations x E2M1 weights (MXFP4) -> fp32 with E8M0 block scales.
// The E2M1 operand is 16 bytes a lane: K [32*(l/16), +32) of row l%16 of the
// 128-wide step, two values a byte, low nibble first -- the same K as the
// E4M3 operand's `lo` / `hi` pieces in their order, and scaled by the same
// lane's scale byte (checked on gfx950 with one-hot operands).  W_FIRST: the
// weights are the first operand (Swap-AB).
template <bool W_FIRST>
__device__ __forceinline__ f32x4 mma_f8f4_mx(const Frag& a, u32x4 w, f32x4 c, int sa, int sw) {
  i32x8 av = {(int)a.lo.x, (int)a.lo.y, (int)a.lo.z, (int)a.lo.w,
              (int)a.hi.x, (int)a.hi.y, (int)a.hi.z, (int)a.hi.w};
  i32x8 wv = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
  if constexpr (W_FIRST)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, av, c, 4, 0, 0, sw, 0, sa);
  else
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, wv, c, 0, 4, 0, sa, 0, sw);
}

// binary32 -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Two E4M3 codes by the conversion instruction (v_cvt_pk_fp8_f32): a and b,
// already clamped to [-448, 448], rounded to nearest even, into byte 0 / 1
// (HI = false) or byte 2 / 3 (HI = true) of `old`.  It agrees with the OCP
// E4M3 definition on every clamped input, signed zeros and subnormal results
// included: the GPU tests compare it with the oracle's encoder around every
// rounding midpoint and on every bf16 value.
template <bool HI>
__device__ __forceinline__ uint32_t e4m3_pk2(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float clamp448(float t) { return __builtin_amdgcn_fmed3f(t, -448.0f, 448.0f); }

// int8 code of an already divided value t: round half to even, clamp to +-127.
__device__ __forceinline__ uint32_t int8_code(float t) {
  float q = __builtin_rintf(t);
  q = fminf(fmaxf(q, -127.0f), 127.0f);
  return (uint32_t)((int)q) & 0xffu;
}

// fl(x / s) at the code level from r = fl(1/s), with one multiply and two
// fused corrections on |x|: q0 = fl(|x|*r), e = fma(-q0, s, |x|) (the
// remainder, exact), q = fma(e, r, q0), then x's sign (so -0 keeps its sign,
// as in -0/s).  q can still differ from fl(|x|/s) by one ulp, but for every
// bf16 x with |x| <= amax, s = fl(amax/Q) >= 2^-96, the rounded code is the
// same -- checked exhaustively over all such (|x|, amax) pairs for Q = 127
// and 448.  Rows with a smaller scale take the division.
constexpr float FAST_DIV_MIN_SCALE = 1.2621774483536189e-29f;  // 2^-96
__device__ __forceinline__ float div_fast(float x, float s, float r) {
  const float ax = __builtin_fabsf(x);
  const float q0 = __fmul_rn(ax, r);
  const float e = __fmaf_rn(-q0, s, ax);
  return __builtin_copysignf(__fmaf_rn(e, r, q0), x);
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// orders global memory, which makes every wave wait for all of its
// outstanding global loads (vmcnt 0) first; here loads issued before the
// barrier stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Maximum of non-negative values over each row of 16 lanes (lanes 16a ..
// 16a+15), returned to every lane of the row: DPP lane swaps (xor 1, xor 2
// by quad permutation, then the half-row and row mirrors).
__device__ __forceinline__ float row16_max_nonneg(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xf, 0xf, false)));
  return v;
}

// Maximum over the wave of non-negative values, returned wave-uniform: DPP
// lane swaps inside each row of 16 (xor 1, xor 2 by quad permutation, then
// the half-row and row mirrors), then the four row results by readlane.
__device__ __forceinline__ float wave_max_nonneg(float v) {
  const int b = __float_as_int(row16_max_nonneg(v));
  return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
               fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

}  // namespace qlk
