// Weight-streaming quantized GEMM for decode token counts (M <= 32) on gfx950.
//
// What it computes: Y[m, n] = epilogue(sum_k A_q[m, k] * W_q[n, k]) with the
// scales of the format fused in -- the scaled quantized linear of the Helion
// linear-backend pages ([Summary] "Put algorithm selection inside the search
// space"; [Noticias] "¿Cómo se implementa el kernel?").  The page's single
// GEMM carries two algorithmic switches, and so does this kernel:
//   * split_k: the K range is cut into chunks, one workgroup per (N tile,
//     chunk); partial sums meet in an int32 / fp32 workspace through device
//     atomics and the last workgroup to arrive applies the epilogue.  (The
//     page zeroes the bf16 output and adds bf16 partials atomically; here the
//     partials stay int32 / fp32 so INT8 remains exact.)
//   * swap_ab: the page rewrites A@B as (B^T@A^T)^T; here that decides which
//     operand feeds the matrix core's first input, i.e. whether a lane's four
//     accumulator registers run along M or along N.
// Decode is HBM-bound (the weights are read once and dominate traffic), so
// the design streams weights, not tiles: every lane pulls 32 bytes of one
// weight row per 128-wide K block straight into registers with raw buffer
// loads (an out-of-range offset returns zeros without a memory request, so
// ragged N / K edges and the pipeline tail need no branches), two batches of
// `PF` blocks in flight per wave.  Activations (<= 32 x K bytes) are either
// staged once per workgroup into LDS with LDS-DMA buffer loads, laid out so
// every ds_read_b128 is a contiguous 1 KB wave read, or fetched per K block
// from L2 next to the weights.
//
// Sources: [Summary] = English summary of "Building a High-Performance and
// Portable vLLM Linear Backend with Helion" (yuxiaoba.github.io);
// [Noticias] = "Helion entra al backend lineal de vLLM y supera a CUTLASS en
// Hopper" (noticias.mechatronicstore.cl).
#pragma once

#include "decode_args.hpp"
#include "device_common.hpp"

namespace qlk {

template <int FMT>
struct AccOf {
  typedef f32x4 T;
};
template <>
struct AccOf<FMT_INT8> {
  typedef i32x4 T;
};

// Fixed epilogue order for the per-token formats: bf16(fl(fl(acc * s_a) * s_w)).
__device__ __forceinline__ uint32_t epilogue_scaled(float accf, float sa, float sw) {
  float t = __fmul_rn(accf, sa);
  t = __fmul_rn(t, sw);
  return bf16_rne(t);
}

template <int FMT, bool SWAP, int MT, int RG, int NW, int PF, bool ALDS>
__global__ void __launch_bounds__(NW * 64) qgemm_decode_kernel(DecodeArgs p) {
  using Acc = typename AccOf<FMT>::T;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int WK = p.waves_k;
  const int wn = wave / WK;
  const int wk = wave - wn * WK;
  const int BN = (NW / WK) * RG * 16;
  const int tile = blockIdx.x / p.split;
  const int chunk = blockIdx.x - tile * p.split;
  const int kb0 = chunk * p.chunk_kb;
  const int kb1 = min(p.G, kb0 + p.chunk_kb);
  const int nkc = kb1 - kb0;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int row_base = tile * BN + wn * RG * 16;

  const uint32_t M = (uint32_t)p.M, N = (uint32_t)p.N, K = (uint32_t)p.K;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w, N * K);
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, M * K);

  // Loop-invariant lane offsets.  A row past the end gets a base of 2^31:
  // adding any in-range K offset (< 2^30) keeps it beyond num_records
  // (<= 2^30) without wrapping, so its loads return zeros.
  const uint32_t glo = (uint32_t)g * 16u;
  uint32_t wbase[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const uint32_t row = (uint32_t)(row_base + rg * 16 + r16);
    wbase[rg] = row < N ? row * K + glo : OOB;
  }
  uint32_t abase[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t m = (uint32_t)(mt * 16 + r16);
    abase[mt] = m < M ? m * K + glo : OOB;
  }

  // ---- this wave's K blocks: kb0 + wk + j*WK, j < nkw
  const int nkw = nkc > wk ? (nkc - wk + WK - 1) / WK : 0;
  const int nbatch = (nkw + PF - 1) / PF;

  Acc acc[RG][MT];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[rg][mt] = Acc{0, 0, 0, 0};

  Frag wb0[PF][RG], wb1[PF][RG];
  Frag ab0[PF][MT], ab1[PF][MT];
  float sa0[PF][MT][4], sa1[PF][MT][4];
  float sw0[PF][RG], sw1[PF][RG];

  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(p.sa, (FMT == FMT_BLOCK ? M * (uint32_t)p.G : M) * 4u);
  const __amdgpu_buffer_rsrc_t rsw =
      make_rsrc(p.sw, (FMT == FMT_BLOCK ? ((N + 127u) / 128u) * (uint32_t)p.G : N) * 4u);

  // Issue one batch of PF K blocks.  A K block past this wave's range, or
  // the part of a ragged last block beyond K, reads as zeros: `rem` (uniform)
  // is the number of valid K bytes left in the block, and a lane's piece is
  // in range when its K offset inside the block is below it.
  auto issue = [&](Frag(&wb)[PF][RG], Frag(&ab)[PF][MT], float(&sab)[PF][MT][4],
                   float(&swb)[PF][RG], int batch) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      const int j = batch * PF + q;
      const bool ok = j < nkw;
      const int kb = ok ? kb0 + wk + j * WK : kb0;
      const uint32_t kofs = (uint32_t)kb * 128u;
      const uint32_t rem = ok ? K - kofs : 0u;
      const bool lo_ok = glo < rem;
      const bool hi_ok = glo + 64u < rem;
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        wb[q][rg].lo = bload16(rw, lo_ok ? wbase[rg] + kofs : OOB);
        wb[q][rg].hi = bload16(rw, hi_ok ? wbase[rg] + kofs + 64u : OOB);
      }
      if constexpr (!ALDS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          ab[q][mt].lo = bload16(ra, lo_ok ? abase[mt] + kofs : OOB);
          ab[q][mt].hi = bload16(ra, hi_ok ? abase[mt] + kofs + 64u : OOB);
        }
      }
      if constexpr (FMT == FMT_BLOCK) {
        const uint32_t Gu = (uint32_t)p.G;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int r = 0; r < (SWAP ? 1 : 4); ++r) {
            const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
            sab[q][mt][r] = bload_f32(rsa, (ok && m < M) ? (m * Gu + (uint32_t)kb) * 4u : OOB);
          }
        }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const uint32_t row0 = (uint32_t)(row_base + rg * 16);
          swb[q][rg] = bload_f32(rsw, (ok && row0 < N) ? ((row0 >> 7) * Gu + (uint32_t)kb) * 4u : OOB);
        }
      }
    }
    // keep the whole batch issued before the matrix-core work that follows
    __builtin_amdgcn_sched_barrier(0);
  };

  auto consume = [&](Frag(&wb)[PF][RG], Frag(&ab)[PF][MT], float(&sab)[PF][MT][4],
                     float(&swb)[PF][RG], int batch) {
#pragma unroll
    for (int q = 0; q < PF; ++q) {
      Frag af[MT];
      if constexpr (ALDS) {
        const int j = batch * PF + q;
        const int kbl = j < nkw ? wk + j * WK : 0;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const uint8_t* base = smem + ((kbl * MT + mt) * 2) * 1024 + lane * 16;
          af[mt].lo = *reinterpret_cast<const u32x4*>(base);
          af[mt].hi = *reinterpret_cast<const u32x4*>(base + 1024);
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) af[mt] = ab[q][mt];
      }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (FMT == FMT_INT8) {
            if (SWAP) {
              acc[rg][mt] = mma_i8(wb[q][rg].lo, af[mt].lo, acc[rg][mt]);
              acc[rg][mt] = mma_i8(wb[q][rg].hi, af[mt].hi, acc[rg][mt]);
            } else {
              acc[rg][mt] = mma_i8(af[mt].lo, wb[q][rg].lo, acc[rg][mt]);
              acc[rg][mt] = mma_i8(af[mt].hi, wb[q][rg].hi, acc[rg][mt]);
            }
          } else if constexpr (FMT == FMT_FP8) {
            acc[rg][mt] = SWAP ? mma_f8(wb[q][rg], af[mt], acc[rg][mt])
                               : mma_f8(af[mt], wb[q][rg], acc[rg][mt]);
          } else {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 part = SWAP ? mma_f8(wb[q][rg], af[mt], z) : mma_f8(af[mt], wb[q][rg], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float f = sab[q][mt][SWAP ? 0 : r] * swb[q][rg];
              acc[rg][mt][r] = __builtin_fmaf(part[r], f, acc[rg][mt][r]);
            }
          }
        }
      }
    }
  };

  // Two batches in flight: the loop enters and repeats with the same pair of
  // buffers outstanding (batch b in wb0, b+1 in wb1), and each buffer is
  // refilled right after it has been consumed.
  issue(wb0, ab0, sa0, sw0, 0);
  issue(wb1, ab1, sa1, sw1, 1);

  // ---- stage this chunk's activations in LDS (after the first weight
  // batches are in flight, so their HBM latency overlaps the staging): one 1 KB block per
  // (K block, token tile, half); lane l of a block holds token 16*mt + l%16,
  // K bytes [h*64 + 16*(l/16), +16) of the K block.
  if constexpr (ALDS) {
    const int nblk = nkc * MT * 2;
    for (int b = wave; b < nblk; b += NW) {
      const int h = b & 1;
      const int mt = (b >> 1) % MT;
      const int kbl = (b >> 1) / MT;
      const uint32_t m = (uint32_t)(mt * 16 + r16);
      const uint32_t k = (uint32_t)(kb0 + kbl) * 128u + (uint32_t)h * 64u + (uint32_t)g * 16u;
      const uint32_t off = (m < M && k < K) ? m * K + k : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(smem + b * 1024), 16, off, 0, 0, 0);
    }
    __syncthreads();
  }

  for (int b = 0; b < nbatch; b += 2) {
    consume(wb0, ab0, sa0, sw0, b);
    issue(wb0, ab0, sa0, sw0, b + 2);
    consume(wb1, ab1, sa1, sw1, b + 1);
    issue(wb1, ab1, sa1, sw1, b + 3);
  }

  // ---- reduce the waves that shared a K chunk (fixed order: deterministic)
  constexpr int NACC = RG * MT * 4;
  if (WK > 1) {
    __syncthreads();
    int* red = reinterpret_cast<int*>(smem);
    if (wk != 0) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = (rg * MT + mt) * 4 + r;
            red[(wave * NACC + i) * 64 + lane] = __builtin_bit_cast(int, acc[rg][mt][r]);
          }
    }
    __syncthreads();
    if (wk == 0) {
      for (int w2 = 1; w2 < WK; ++w2) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = (rg * MT + mt) * 4 + r;
              const int v = red[((wave + w2) * NACC + i) * 64 + lane];
              if constexpr (FMT == FMT_INT8)
                acc[rg][mt][r] += v;
              else
                acc[rg][mt][r] += __builtin_bit_cast(float, v);
            }
      }
    }
  }

  // ---- split-K: combine partial sums through the workspace
  if (p.split > 1) {
    if (wk == 0) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t n = SWAP ? (uint32_t)(row_base + rg * 16 + 4 * g + r)
                                    : (uint32_t)(row_base + rg * 16 + r16);
            const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
            if (m < M && n < N) {
              if constexpr (FMT == FMT_INT8)
                __hip_atomic_fetch_add(reinterpret_cast<int*>(p.ws) + (size_t)m * N + n, acc[rg][mt][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              else
                __hip_atomic_fetch_add(reinterpret_cast<float*>(p.ws) + (size_t)m * N + n, acc[rg][mt][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (unsigned)(p.split - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    if (wk == 0) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t n = SWAP ? (uint32_t)(row_base + rg * 16 + 4 * g + r)
                                    : (uint32_t)(row_base + rg * 16 + r16);
            const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
            if (m < M && n < N) {
              int* slot = reinterpret_cast<int*>(p.ws) + (size_t)m * N + n;
              const int v = __hip_atomic_exchange(slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if constexpr (FMT == FMT_INT8)
                acc[rg][mt][r] = v;
              else
                acc[rg][mt][r] = __builtin_bit_cast(float, v);
            }
          }
    }
    if (tid == 0) __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (wk != 0) return;

  // ---- epilogue: scales, bf16 rounding, store
  const bool vec4 = SWAP && (N & 3u) == 0;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint32_t out[4];
      uint32_t nn[4], mm[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        nn[r] = SWAP ? (uint32_t)(row_base + rg * 16 + 4 * g + r) : (uint32_t)(row_base + rg * 16 + r16);
        mm[r] = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
        const bool ok = mm[r] < M && nn[r] < N;
        if constexpr (FMT == FMT_BLOCK) {
          out[r] = bf16_rne(acc[rg][mt][r]);
          if (ok && p.acc_out)
            reinterpret_cast<float*>(p.acc_out)[(size_t)mm[r] * N + nn[r]] = acc[rg][mt][r];
        } else {
          const float sa = ok ? p.sa[mm[r]] : 0.f;
          const float sw = ok ? p.sw[nn[r]] : 0.f;
          float accf;
          if constexpr (FMT == FMT_INT8)
            accf = __int2float_rn(acc[rg][mt][r]);
          else
            accf = acc[rg][mt][r];
          out[r] = epilogue_scaled(accf, sa, sw);
          if (ok && p.acc_out) {
            if constexpr (FMT == FMT_INT8)
              reinterpret_cast<int*>(p.acc_out)[(size_t)mm[r] * N + nn[r]] = acc[rg][mt][r];
            else
              reinterpret_cast<float*>(p.acc_out)[(size_t)mm[r] * N + nn[r]] = acc[rg][mt][r];
          }
        }
      }
      if (vec4 && mm[0] < M && nn[3] < N) {
        u32x2 v = {out[0] | (out[1] << 16), out[2] | (out[3] << 16)};
        *reinterpret_cast<u32x2*>(p.y + (size_t)mm[0] * N + nn[0]) = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mm[r] < M && nn[r] < N) p.y[(size_t)mm[r] * N + nn[r]] = (uint16_t)out[r];
      }
    }
  }
}

// Instantiation table for one format: every (swap, mt, rg, nw, pf, alds)
// combination the planner may choose.
template <int FMT>
hipError_t decode_dispatch(const DecodeKey& k, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                           const DecodeArgs& a, bool probe_only) {
#define QL_TRY(SW, MT_, RG_, NW_, PF_, AL)                                                         \
  if (k.swap == SW && k.mt == MT_ && k.rg == RG_ && k.nw == NW_ && k.pf == PF_ && k.alds == AL) { \
    if (probe_only) return hipSuccess;                                                            \
    qgemm_decode_kernel<FMT, SW, MT_, RG_, NW_, PF_, AL><<<grid, block, lds, s>>>(a);             \
    return hipGetLastError();                                                                     \
  }
#define QL_TRY_AL(SW, MT_, RG_, NW_, PF_) QL_TRY(SW, MT_, RG_, NW_, PF_, 0) QL_TRY(SW, MT_, RG_, NW_, PF_, 1)
#define QL_TRY_PF(SW, MT_, RG_, NW_) QL_TRY_AL(SW, MT_, RG_, NW_, 2) QL_TRY_AL(SW, MT_, RG_, NW_, 4)
#define QL_TRY_RG(SW, MT_, NW_) QL_TRY_PF(SW, MT_, 1, NW_) QL_TRY_PF(SW, MT_, 2, NW_)
#define QL_TRY_MT(SW, NW_) QL_TRY_RG(SW, 1, NW_) QL_TRY_RG(SW, 2, NW_)
  QL_TRY_MT(false, 4)
  QL_TRY_MT(true, 4)
#undef QL_TRY_MT
#undef QL_TRY_RG
#undef QL_TRY_PF
#undef QL_TRY_AL
#undef QL_TRY
  return hipErrorInvalidDeviceFunction;
}

}  // namespace qlk
