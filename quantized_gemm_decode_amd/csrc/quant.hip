// Quantizer kernels for gfx950: the dynamic activation quantizer (per token,
// or per 1x128 group for Block_FP8) and the offline weight quantizer (per
// output channel, or per 128x128 block for Block_FP8).
//
// Formats and granularity: [Summary] "Put algorithm selection inside the
// search space" (last paragraph) and [Noticias] "El backend lineal de Helion
// / Alcance".  The pages give no formula; the rule here is symmetric absmax:
//   s = fl(amax / Q), Q = 127 (int8) or 448 (E4M3); s = 1 when amax == 0;
//   code = round-half-even(fl(x / s)), clamped to [-127, 127] for int8, or
//   clamped to [-448, 448] and rounded to nearest-even E4M3.
// Both divisions are IEEE binary32 divisions (__fdiv_rn), and fp32
// subnormals are kept, so the codes and scales are a deterministic function
// of the bf16 input.  amax is a wavefront reduction (DPP/swizzle shuffles)
// followed by an LDS reduction across the workgroup's waves.
//
// [Summary] = English summary of "Building a High-Performance and Portable
// vLLM Linear Backend with Helion" (yuxiaoba.github.io); [Noticias] = "Helion
// entra al backend lineal de vLLM y supera a CUTLASS en Hopper".
#include <algorithm>

#include "decode_args.hpp"
#include "device_common.hpp"
#include "quant_common.hpp"

namespace qlk {

constexpr int QT = 256;  // threads per quantizer workgroup

template <int NT>
__device__ __forceinline__ float block_max(float m, float* red) {
  m = wave_max_nonneg(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < NT / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}

// Byte offset of codes (row, k .. k+7) in the packed activation layout: the
// 2 KB tile (row / 16, k / 128) at (row/16 * G + k/128) * 2048, inside it byte
// h*1024 + l*16 + j holds row 16t + l%16, K offset 128kb + 64h + 16(l/16) + j
// (the layout of packed weights; 8 consecutive codes stay in one 16-byte piece).
__device__ __forceinline__ size_t packed_offset(uint32_t row, uint32_t k, uint32_t G) {
  const uint32_t kk = k & 127u;
  return ((size_t)(row >> 4) * G + (k >> 7)) * 2048u + (kk >> 6) * 1024u +
         ((row & 15u) + 16u * ((kk >> 4) & 3u)) * 16u + (kk & 15u);
}

// PARTS workgroups per row; the row stays in registers (VPT 16-byte vectors
// per thread) between the amax pass and the quantize pass.  Each of a row's
// workgroups reads the whole row and reduces its amax (a few operations per
// value), then quantizes only its own 1/PARTS of the row (some ninety
// operations per 8 values): on a long row that arithmetic, not the loads,
// bounds the launch, and one compute unit per row left most of the chip
// idle.  PACKED writes the packed activation layout instead of row-major
// codes: the grid then also covers the padding rows up to a multiple of 16
// and the padding K up to a multiple of 128, which get zero codes (and no
// scale).
template <int FMT, int VPT, bool PACKED, int NT, int PARTS = 1>
__global__ void __launch_bounds__(NT) quant_rows_reg_kernel(const uint16_t* __restrict__ x, uint32_t R, uint32_t C,
                                                            uint8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float red[NT / 64];
  const uint32_t row = blockIdx.x / PARTS;
  const uint32_t part = blockIdx.x - row * PARTS;
  const bool real = row < R;
  const uint16_t* xr = x + (size_t)row * C;
  const uint32_t G = (C + 127u) / 128u;
  const uint32_t CW = PACKED ? G * 128u : C;  // code columns written
  u32x4 v[VPT];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const uint32_t e = (uint32_t)(i * NT + threadIdx.x) * 8u;
    v[i] = (real && e < C) ? *reinterpret_cast<const u32x4*>(xr + e) : u32x4{0, 0, 0, 0};
    amax = abs_bf16_max8(v[i], amax);
  }
  amax = block_max<NT>(amax, red);
  const float sc = scale_of<FMT>(amax);
  const float rc = recip_of(sc);
  // this workgroup's vectors of the row: [v_lo, v_hi) of the CW/8 written
  const uint32_t nv = CW / 8u;
  const uint32_t v_lo = PARTS == 1 ? 0u : nv * part / PARTS, v_hi = PARTS == 1 ? nv : nv * (part + 1u) / PARTS;
#pragma unroll
  for (int i = 0; i < VPT; ++i) {
    const uint32_t vi = (uint32_t)(i * NT) + threadIdx.x;
    if (vi >= v_lo && vi < v_hi) {
      const uint32_t e = vi * 8u;
      const size_t off = PACKED ? packed_offset(row, e, G) : (size_t)row * C + e;
      *reinterpret_cast<u32x2*>(q + off) = quant8<FMT>(v[i], sc, rc);
    }
  }
  if (threadIdx.x == 0 && real && part == 0) s[row] = sc;
}

// Rows too long for registers: two streaming passes (the second re-reads from cache).
template <int FMT, bool PACKED>
__global__ void __launch_bounds__(QT) quant_rows_stream_kernel(const uint16_t* __restrict__ x, uint32_t R, uint32_t C,
                                                               uint8_t* __restrict__ q, float* __restrict__ s) {
  __shared__ float red[QT / 64];
  const uint32_t row = blockIdx.x;
  const bool real = row < R;
  const uint16_t* xr = x + (size_t)row * C;
  const uint32_t G = (C + 127u) / 128u;
  const uint32_t CW = PACKED ? G * 128u : C;
  float amax = 0.0f;
  if (real)
    for (uint32_t e = threadIdx.x * 8u; e < C; e += QT * 8u)
      amax = abs_bf16_max8(*reinterpret_cast<const u32x4*>(xr + e), amax);
  amax = block_max<QT>(amax, red);
  const float sc = scale_of<FMT>(amax);
  const float rc = recip_of(sc);
  for (uint32_t e = threadIdx.x * 8u; e < CW; e += QT * 8u) {
    const u32x4 v = (real && e < C) ? *reinterpret_cast<const u32x4*>(xr + e) : u32x4{0, 0, 0, 0};
    const size_t off = PACKED ? packed_offset(row, e, G) : (size_t)row * C + e;
    *reinterpret_cast<u32x2*>(q + off) = quant8<FMT>(v, sc, rc);
  }
  if (threadIdx.x == 0 && real) s[row] = sc;
}

// Block_FP8 activations: groups of 128 contiguous elements along K (K % 128
// == 0, so group id = m * K/128 + g is also the s_a index); 16 lanes per
// group, 8 elements per lane; the group amax reduces over the 16 lanes (one
// DPP row: groups start at multiples of 16 lanes).
// PACKED: codes in the packed activation layout; groups of the padding rows
// (up to a multiple of 16 rows, `ngroups_out` in all) get zero codes.
template <bool PACKED>
__global__ void __launch_bounds__(QT) quant_groups_kernel(const uint16_t* __restrict__ x, uint32_t ngroups,
                                                          uint32_t ngroups_out, uint32_t G,
                                                          uint8_t* __restrict__ q, float* __restrict__ s) {
  const uint32_t gid = blockIdx.x * (QT / 16) + (threadIdx.x >> 4);
  const uint32_t li = threadIdx.x & 15u;
  const bool ok = gid < ngroups;
  const size_t e = (size_t)gid * 128u + li * 8u;
  const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(x + e) : u32x4{0, 0, 0, 0};
  const float amax = row16_max_nonneg(abs_bf16_max8(v, 0.0f));   // the group's 16 lanes are a DPP row
  const float sc = scale_of<FMT_FP8>(amax);
  if (gid < (PACKED ? ngroups_out : ngroups)) {
    const size_t off = PACKED ? packed_offset(gid / G, (gid % G) * 128u + li * 8u, G) : e;
    *reinterpret_cast<u32x2*>(q + off) = quant8<FMT_FP8>(v, sc, recip_of(sc));
  }
  if (ok && li == 0) s[gid] = sc;
}

// Block_FP8 weights: one workgroup per 128x128 block (nb, g); thread t covers
// 8 columns (t % 16) of rows t/16 + 16 i; rows >= N of a ragged last block
// row are not part of the block.
__global__ void __launch_bounds__(QT) quant_wblocks_kernel(const uint16_t* __restrict__ w, uint32_t N,
                                                           uint32_t K, uint8_t* __restrict__ q,
                                                           float* __restrict__ s) {
  __shared__ float red[QT / 64];
  const uint32_t g = blockIdx.x, nb = blockIdx.y, G = gridDim.x;
  const uint32_t c = (threadIdx.x & 15u) * 8u;
  const uint32_t r0 = threadIdx.x >> 4;
  u32x4 v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t n = nb * 128u + r0 + 16u * i;
    v[i] = n < N ? *reinterpret_cast<const u32x4*>(w + (size_t)n * K + g * 128u + c) : u32x4{0, 0, 0, 0};
    amax = abs_bf16_max8(v[i], amax);
  }
  amax = block_max<QT>(amax, red);
  const float sc = scale_of<FMT_FP8>(amax);
  const float rc = recip_of(sc);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t n = nb * 128u + r0 + 16u * i;
    if (n < N) *reinterpret_cast<u32x2*>(q + (size_t)n * K + g * 128u + c) = quant8<FMT_FP8>(v[i], sc, rc);
  }
  if (threadIdx.x == 0) s[nb * G + g] = sc;
}

__global__ void fill_zero_u16_kernel(uint16_t* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0;
}

// Packed weight tiles: tile (t, kb) -- rows 16t..16t+15, K bytes 128kb..128kb+127 --
// is 2 KB at (t*G + kb)*2048; byte h*1024 + l*16 + j of the tile is
// W[16t + l%16][128kb + 64h + 16(l/16) + j] (zero outside N x K).  One thread
// moves one 16-byte piece; K % 16 == 0 keeps every piece wholly in or out.
__global__ void __launch_bounds__(256) pack_weight_kernel(const uint8_t* __restrict__ w, uint32_t N, uint32_t K,
                                                          uint32_t G, uint32_t pieces, uint8_t* __restrict__ out) {
  const uint32_t pc = blockIdx.x * 256u + threadIdx.x;
  if (pc >= pieces) return;
  const uint32_t l = pc & 63u, h = (pc >> 6) & 1u, tk = pc >> 7;
  const uint32_t kb = tk % G, t = tk / G;
  const uint32_t row = t * 16u + (l & 15u);
  const uint32_t k = kb * 128u + h * 64u + (l >> 4) * 16u;
  u32x4 v = {0, 0, 0, 0};
  if (row < N && k < K) v = *reinterpret_cast<const u32x4*>(w + (size_t)row * K + k);
  *reinterpret_cast<u32x4*>(out + (size_t)pc * 16u) = v;
}

hipError_t launch_pack_weight(const void* w_q, int64_t N, int64_t K, void* w_packed, hipStream_t st) {
  const uint32_t NT = (uint32_t)((N + 15) / 16), G = (uint32_t)((K + 127) / 128);
  const uint32_t pieces = NT * G * 128u;
  pack_weight_kernel<<<dim3((pieces + 255u) / 256u), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(w_q), (uint32_t)N, (uint32_t)K, G, pieces, static_cast<uint8_t*>(w_packed));
  return hipGetLastError();
}

template <int FMT, bool PACKED, int NT>
static hipError_t rows_dispatch_nt(const void* x, int64_t R, int64_t C, void* q, float* s, hipStream_t st) {
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  uint8_t* qp = static_cast<uint8_t*>(q);
  const int64_t vecs = (C + 7) / 8;
  const int64_t vpt = (vecs + NT - 1) / NT;
  const int64_t rows = PACKED ? (R + 15) / 16 * 16 : R;
  const dim3 grid((unsigned)rows), block(NT);
  const uint32_t r = (uint32_t)R, c = (uint32_t)C;
  // the few rows of decode activations (at most 64): a row's quantization
  // split over 2 workgroups for 1024 < C <= 2048 values, 4 up to 16384, 8 up
  // to 32768, 16 up to 65536 (measured: each doubling of the parts up to
  // these shortened the launch; the amax pass every part repeats is cheap)
  const bool split = NT == 1024 && R <= 64;
  if (vpt <= 1 && split && vecs > 256)
    quant_rows_reg_kernel<FMT, 1, PACKED, NT, 4><<<dim3((unsigned)(rows * 4)), block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 1 && split && vecs > 128)
    quant_rows_reg_kernel<FMT, 1, PACKED, NT, 2><<<dim3((unsigned)(rows * 2)), block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 1)
    quant_rows_reg_kernel<FMT, 1, PACKED, NT><<<grid, block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 2 && split)
    quant_rows_reg_kernel<FMT, 2, PACKED, NT, 4><<<dim3((unsigned)(rows * 4)), block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 2)
    quant_rows_reg_kernel<FMT, 2, PACKED, NT><<<grid, block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 4 && split)
    quant_rows_reg_kernel<FMT, 4, PACKED, NT, 8><<<dim3((unsigned)(rows * 8)), block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 4)
    quant_rows_reg_kernel<FMT, 4, PACKED, NT><<<grid, block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 8 && split)
    quant_rows_reg_kernel<FMT, 8, PACKED, NT, 16><<<dim3((unsigned)(rows * 16)), block, 0, st>>>(xp, r, c, qp, s);
  else if (vpt <= 8)
    quant_rows_reg_kernel<FMT, 8, PACKED, NT><<<grid, block, 0, st>>>(xp, r, c, qp, s);
  else if constexpr (NT == QT) {
    if (vpt <= 16)
      quant_rows_reg_kernel<FMT, 16, PACKED, NT><<<grid, block, 0, st>>>(xp, r, c, qp, s);
    else
      quant_rows_stream_kernel<FMT, PACKED><<<grid, block, 0, st>>>(xp, r, c, qp, s);
  }
  return hipGetLastError();
}

// Few rows (activations at decode token counts): 1024 threads a row, so each
// lane quantizes at most a few vectors; many rows (weights): 256.
template <int FMT, bool PACKED>
static hipError_t rows_dispatch(const void* x, int64_t R, int64_t C, void* q, float* s, hipStream_t st) {
  if (R <= 256 && C <= 8 * 8 * 1024) return rows_dispatch_nt<FMT, PACKED, 1024>(x, R, C, q, s, st);
  return rows_dispatch_nt<FMT, PACKED, QT>(x, R, C, q, s, st);
}

hipError_t launch_quant_rows(int fmt, const void* x, int64_t R, int64_t C, void* q, float* s, bool packed,
                             hipStream_t st) {
  if (packed) {
    if (fmt == FMT_INT8) return rows_dispatch<FMT_INT8, true>(x, R, C, q, s, st);
    return rows_dispatch<FMT_FP8, true>(x, R, C, q, s, st);
  }
  if (fmt == FMT_INT8) return rows_dispatch<FMT_INT8, false>(x, R, C, q, s, st);
  return rows_dispatch<FMT_FP8, false>(x, R, C, q, s, st);
}

hipError_t launch_quant_groups(const void* x, int64_t M, int64_t K, void* q, float* s, bool packed,
                               hipStream_t st) {
  const int64_t G = K / 128;
  const int64_t ng = M * G;
  const int64_t ng_out = packed ? (M + 15) / 16 * 16 * G : ng;
  const dim3 grid((unsigned)((ng_out + QT / 16 - 1) / (QT / 16))), block(QT);
  if (packed)
    quant_groups_kernel<true><<<grid, block, 0, st>>>(static_cast<const uint16_t*>(x), (uint32_t)ng, (uint32_t)ng_out,
                                                      (uint32_t)G, static_cast<uint8_t*>(q), s);
  else
    quant_groups_kernel<false><<<grid, block, 0, st>>>(static_cast<const uint16_t*>(x), (uint32_t)ng,
                                                       (uint32_t)ng_out, (uint32_t)G, static_cast<uint8_t*>(q), s);
  return hipGetLastError();
}

hipError_t launch_quant_wblocks(const void* w, int64_t N, int64_t K, void* q, float* s, hipStream_t st) {
  const dim3 grid((unsigned)(K / 128), (unsigned)((N + 127) / 128)), block(QT);
  quant_wblocks_kernel<<<grid, block, 0, st>>>(static_cast<const uint16_t*>(w), (uint32_t)N, (uint32_t)K,
                                               static_cast<uint8_t*>(q), s);
  return hipGetLastError();
}

// MXFP8 (OCP microscaling, E4M3 elements): a block is 32 consecutive values
// of a row; its shared exponent is e = floor(log2(amax)) - 8 (8: exponent of
// E4M3's largest normal), clamped to [-127, 127], -127 for an all-zero block,
// stored as the E8M0 byte e + 127; each element is x * 2^-e (exact: a power
// of two; a product below the binary32 normals is far below E4M3's smallest
// subnormal, so its rounding cannot change the code) clamped to +-448 and
// rounded to E4M3.
// EMAX: exponent of the element format's largest normal (E4M3 8, E2M1 2).
template <int EMAX>
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t u = __float_as_uint(amax);   // amax >= 0, finite
  if (u == 0u) return -127;
  const int fl2 = u >= 0x00800000u ? (int)(u >> 23) - 127   // normal
                                   : (31 - (int)__clz(u)) - 149;  // subnormal: u * 2^-149
  return max(-127, fl2 - EMAX);
}

// Four lanes (a DPP quad) per block, 8 values (one 16-byte load) a lane.
// PACKED: codes in the packed activation layout and scales in lane order
// (byte (row/16 * G + k/128)*64 + row%16 + 16*((k%128)/32)); the padding
// rows up to a multiple of 16 (`rows_out`) get zero codes and zero scales.
template <bool PACKED>
__global__ void __launch_bounds__(256) quant_mx_kernel(const uint16_t* __restrict__ x, uint32_t R, uint32_t rows_out,
                                                       uint32_t C, uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const uint32_t kpr = C / 8u;                   // 8-value pieces per row
  const uint32_t row = t / kpr;
  const uint32_t k = (t - row * kpr) * 8u;
  const bool ok = row < R;
  const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(x + (size_t)row * C + k) : u32x4{0, 0, 0, 0};
  float m = abs_bf16_max8(v, 0.0f);
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  const int e = mx_exponent<8>(m);
  const float f = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, a normal binary32
  uint32_t c0 = 0u, c1 = 0u;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = clamp448(__fmul_rn(__uint_as_float(w[i] << 16), f));
    const float b = clamp448(__fmul_rn(__uint_as_float(w[i] & 0xffff0000u), f));
    if (i < 2)
      c0 = (i == 0) ? e4m3_pk2<false>(a, b, c0) : e4m3_pk2<true>(a, b, c0);
    else
      c1 = (i == 2) ? e4m3_pk2<false>(a, b, c1) : e4m3_pk2<true>(a, b, c1);
  }
  if (row < (PACKED ? rows_out : R)) {
    const size_t off = PACKED ? packed_offset(row, k, C / 128u) : (size_t)row * C + k;
    *reinterpret_cast<u32x2*>(q + off) = ok ? u32x2{c0, c1} : u32x2{0u, 0u};
  }
  if ((k & 31u) == 0u) {
    if (PACKED && row < rows_out)
      s[((size_t)(row >> 4) * (C / 128u) + (k >> 7)) * 64u + (row & 15u) + 16u * ((k >> 5) & 3u)] =
          ok ? (uint8_t)(e + 127) : (uint8_t)0;
    else if (!PACKED && ok)
      s[(size_t)row * (C / 32u) + k / 32u] = (uint8_t)(e + 127);
  }
}

// MXFP4 weights: as quant_mx_kernel with E2M1 elements -- e = floor(log2(amax))
// - 2 (6 = 1.5 * 2^2), elements w * 2^-e clamped to +-6 and rounded to the
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code (mantissa bit
// 0): the code counts the rounding boundaries below |t|, a boundary that |t|
// meets exactly counting only when the code above it is even.  Codes two a
// byte, low nibble first, row-major [R, C/2].
__device__ __forceinline__ uint32_t e2m1_code(float t) {
  const float a = fabsf(t);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(t) >> 28) & 0x8u);
}

__global__ void __launch_bounds__(256) quant_mx4_kernel(const uint16_t* __restrict__ w, uint32_t R, uint32_t C,
                                                        uint8_t* __restrict__ q, uint8_t* __restrict__ s) {
  const uint32_t t = blockIdx.x * 256u + threadIdx.x;
  const uint32_t kpr = C / 8u;
  const uint32_t row = t / kpr;
  const uint32_t k = (t - row * kpr) * 8u;
  const bool ok = row < R;
  const u32x4 v = ok ? *reinterpret_cast<const u32x4*>(w + (size_t)row * C + k) : u32x4{0, 0, 0, 0};
  float m = abs_bf16_max8(v, 0.0f);
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0xB1, 0xF, 0xF, false)));
  m = fmaxf(m, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(m), 0x4E, 0xF, 0xF, false)));
  const int e = mx_exponent<2>(m);
  const float f = __uint_as_float((uint32_t)(127 - e) << 23);   // 2^-e, a normal binary32 (e <= 125)
  uint32_t codes = 0u;
  const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float a = __builtin_amdgcn_fmed3f(__fmul_rn(__uint_as_float(wv[i] << 16), f), -6.0f, 6.0f);
    const float b = __builtin_amdgcn_fmed3f(__fmul_rn(__uint_as_float(wv[i] & 0xffff0000u), f), -6.0f, 6.0f);
    codes |= (e2m1_code(a) | (e2m1_code(b) << 4)) << (8 * i);
  }
  if (ok) {
    *reinterpret_cast<uint32_t*>(q + (size_t)row * (C / 2u) + k / 2u) = codes;
    if ((k & 31u) == 0u) s[(size_t)row * (C / 32u) + k / 32u] = (uint8_t)(e + 127);
  }
}

hipError_t launch_quant_mx4(const void* w, int64_t N, int64_t K, void* q, uint8_t* s, hipStream_t st) {
  const int64_t threads = N * (K / 8);
  quant_mx4_kernel<<<dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, st>>>(
      static_cast<const uint16_t*>(w), (uint32_t)N, (uint32_t)K, static_cast<uint8_t*>(q), s);
  return hipGetLastError();
}

// One thread per 16-byte piece of the packed MXFP4 weight layout.
__global__ void __launch_bounds__(256) pack_weight_fp4_kernel(const uint8_t* __restrict__ w, uint32_t N,
                                                              uint32_t K, uint32_t G, uint32_t total,
                                                              uint8_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;   // piece index
  if (i >= total) return;
  const uint32_t l = i & 63u;
  const uint32_t kb = (i >> 6) % G;
  const uint32_t t = (i >> 6) / G;
  const uint32_t row = t * 16u + (l & 15u);
  u32x4 v = {0u, 0u, 0u, 0u};
  if (row < N) v = *reinterpret_cast<const u32x4*>(w + (size_t)row * (K / 2u) + kb * 64u + (l >> 4) * 16u);
  *reinterpret_cast<u32x4*>(out + (size_t)i * 16u) = v;
}

hipError_t launch_pack_weight_fp4(const void* w_q, int64_t N, int64_t K, void* w_packed, hipStream_t st) {
  const int64_t G = K / 128;
  const int64_t total = (N + 15) / 16 * G * 64;
  pack_weight_fp4_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(w_q), (uint32_t)N, (uint32_t)K, (uint32_t)G, (uint32_t)total,
      static_cast<uint8_t*>(w_packed));
  return hipGetLastError();
}

// One thread per byte of the lane-order MXFP8 scale layout.
__global__ void __launch_bounds__(256) pack_mx_scales_kernel(const uint8_t* __restrict__ s, uint32_t R, uint32_t G,
                                                             uint32_t total, uint8_t* __restrict__ out) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i >= total) return;
  const uint32_t l = i & 63u;
  const uint32_t kb = (i >> 6) % G;
  const uint32_t t = (i >> 6) / G;
  const uint32_t row = t * 16u + (l & 15u);
  out[i] = row < R ? s[(size_t)row * (G * 4u) + kb * 4u + (l >> 4)] : (uint8_t)0;
}

hipError_t launch_pack_mx_scales(const void* s, int64_t R, int64_t K, void* packed, hipStream_t st) {
  const int64_t G = K / 128;
  const int64_t total = (R + 15) / 16 * G * 64;
  pack_mx_scales_kernel<<<dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st>>>(
      static_cast<const uint8_t*>(s), (uint32_t)R, (uint32_t)G, (uint32_t)total, static_cast<uint8_t*>(packed));
  return hipGetLastError();
}

hipError_t launch_quant_mx(const void* x, int64_t R, int64_t C, void* q, uint8_t* s, bool packed, hipStream_t st) {
  const int64_t rows_out = packed ? (R + 15) / 16 * 16 : R;
  const int64_t threads = rows_out * (C / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (packed)
    quant_mx_kernel<true><<<grid, block, 0, st>>>(static_cast<const uint16_t*>(x), (uint32_t)R, (uint32_t)rows_out,
                                                  (uint32_t)C, static_cast<uint8_t*>(q), s);
  else
    quant_mx_kernel<false><<<grid, block, 0, st>>>(static_cast<const uint16_t*>(x), (uint32_t)R, (uint32_t)rows_out,
                                                   (uint32_t)C, static_cast<uint8_t*>(q), s);
  return hipGetLastError();
}

// The E4M3 encoder alone: two values per thread, clamped, by the conversion
// instruction every FP8 quantizer uses.
__global__ void __launch_bounds__(256) encode_e4m3_kernel(const float* __restrict__ x, uint32_t n,
                                                          uint8_t* __restrict__ q) {
  const uint32_t i = (blockIdx.x * 256u + threadIdx.x) * 2u;
  if (i >= n) return;
  const float a = clamp448(x[i]);
  const float b = i + 1u < n ? clamp448(x[i + 1u]) : 0.0f;
  const uint32_t c = e4m3_pk2<false>(a, b, 0u);
  q[i] = (uint8_t)(c & 0xffu);
  if (i + 1u < n) q[i + 1u] = (uint8_t)((c >> 8) & 0xffu);
}

hipError_t launch_encode_e4m3(const float* x, int64_t n, void* q, hipStream_t st) {
  const int64_t blocks = (n + 511) / 512;
  encode_e4m3_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(x, (uint32_t)n, static_cast<uint8_t*>(q));
  return hipGetLastError();
}

hipError_t launch_fill_zero_bf16(void* y, int64_t count, hipStream_t st) {
  const int64_t blocks = std::min<int64_t>((count + 255) / 256, 4096);
  fill_zero_u16_kernel<<<dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, st>>>(
      static_cast<uint16_t*>(y), (size_t)count);
  return hipGetLastError();
}

}  // namespace qlk
