// Weight-streaming quantized GEMM for decode token counts (M <= 64) on gfx950.
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
// Fused quantization (activation mode 4, small M): the workgroup reads the
// bf16 rows of X itself, reduces each row's amax, and writes the codes of its
// own K range into LDS -- the dynamic quantizer's arithmetic, bit for bit --
// while its first weight batches are already in flight, so a linear is one
// launch instead of two.  Its first workgroup per chunk range also writes the
// codes (packed layout) and scales out, as the standalone quantizer would.
//
// Sources: [Summary] = English summary of "Building a High-Performance and
// Portable vLLM Linear Backend with Helion" (yuxiaoba.github.io);
// [Noticias] = "Helion entra al backend lineal de vLLM y supera a CUTLASS en
// Hopper" (noticias.mechatronicstore.cl).
#pragma once

#include "decode_args.hpp"
#include "device_common.hpp"
#include "quant_common.hpp"

namespace qlk {

template <int FMT>
struct AccOf {
  typedef f32x4 T;
};
template <>
struct AccOf<FMT_INT8> {
  typedef i32x4 T;
};

// 32-bit pattern of one accumulator element.  (Element values are copied to
// a scalar first: a bit-cast applied directly to an ext-vector element
// lvalue has been seen to read element 0 for every index.)
__device__ __forceinline__ int bits_of(int v) { return v; }
__device__ __forceinline__ int bits_of(float v) { return __float_as_int(v); }

// Fixed epilogue order for the per-token formats: bf16(fl(fl(acc * s_a) * s_w)).
__device__ __forceinline__ uint32_t epilogue_scaled(float accf, float sa, float sw) {
  float t = __fmul_rn(accf, sa);
  t = __fmul_rn(t, sw);
  return bf16_rne(t);
}

// GLU: the weight is a merged gate/up projection (rows [0, N/2) gate, rows
// [N/2, N) up) and the output is silu(gate) * up, [M, N/2]: a wave's two
// 16-row groups are gate rows c.. and the up rows N/2 + c.. of the same
// output columns, so both values of an output element meet in one lane.
//
// Arguments: the operands and sizes the prologue needs come first, as 14
// words the hardware preloads into SGPRs at wave launch (the library is
// built with a kernel-argument preload count of 9), so the first weight and
// scale loads do not wait for a read of the kernel-argument segment; the
// full argument block follows and supplies what only later code uses.
// `a_or_x` is X for the fused-quantization modes and A_q otherwise; `shape`
// packs waves_k (5 bits), split (9 bits), chunk_kb (14 bits) and the row
// tile in units of 8 rows (4 bits; 0: the workgroup's waves_n * 16 * RG).
template <int FMT, bool SWAP, int MT, int RG, int NW, int PF, int AL, int WM, bool GLU>
__global__ void __launch_bounds__(NW * 64)
    qgemm_decode_kernel(const void* a_or_x, const uint8_t* w_in, const float* sa_in, const float* sw_in,
                        uint32_t* amax_in, int M_in, int N_in, int K_in, int shape, DecodeArgs args) {
  constexpr bool FUSED = AL == 4 || AL == 5;          // activations quantized here from bf16 X
  DecodeArgs p = args;
  if constexpr (FUSED)
    p.x = static_cast<const uint16_t*>(a_or_x);
  else
    p.a = static_cast<const uint8_t*>(a_or_x);
  p.w = w_in;
  p.sa = sa_in;
  p.sw = sw_in;
  p.amax = amax_in;
  p.M = M_in;
  p.N = N_in;
  p.K = K_in;
  p.G = (K_in + 127) / 128;
  p.waves_k = shape & 31;
  p.split = (shape >> 5) & 511;
  p.chunk_kb = (shape >> 14) & 16383;
  // Row tile: a workgroup owns rows [tile * BN, tile * BN + BN) of N.  By
  // default BN is what its waves cover; a plan may give it fewer, any
  // multiple of 8 (for example 24 rows, so that N = 6144 spreads over 256
  // compute units instead of 192 workgroups of 32 rows), and the rows of its
  // last row group beyond the tile are neither loaded nor stored.
  const int row_tile = (int)(((uint32_t)shape >> 28) * 8u);
  // the workgroup reads only its K chunk of X: Block_FP8 (1 x 128 groups are
  // local) and activation mode 5 (per-token amax given by the producer of X)
  constexpr bool CHUNKED = FUSED && (FMT == FMT_BLOCK || AL == 5);
  constexpr bool ALDS = AL == 1 || AL == 3 || FUSED;  // activations read from LDS
  constexpr bool AP = AL == 2;                        // packed activations, read per K block like packed weights
  constexpr bool WL = WM == W_LDS_TRANSPOSE;
  constexpr bool WP = WM == W_PACKED;
  static_assert(!FUSED || (MT == 1 && WP), "fused quantization: one token tile, packed weights");
  static_assert(AL != 5 || ((FMT == FMT_FP8 || FMT == FMT_INT8) && !GLU), "given amax: per-token formats");
  static_assert(!GLU || (RG == 2 && WP), "SiLU-and-mul: a gate and an up row group per wave, packed weights");
  static_assert(FMT != FMT_MX || (!FUSED && !GLU), "MXFP8: quantized activations in, plain bf16 out");
  static_assert(FMT != FMT_MX4 || (!FUSED && !GLU && WP), "MXFP4: packed weights, quantized activations");
  constexpr bool MXS = FMT == FMT_MX || FMT == FMT_MX4;   // E8M0 block scales in the matrix instruction
  constexpr uint32_t WTILE = FMT == FMT_MX4 ? 1024u : 2048u;   // packed weight tile bytes
  using Acc = typename AccOf<FMT>::T;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // A plan other than activation mode 5 given its input's amax buffer (the
  // consumer end of the gate_up -> down chain, quantizing X by itself):
  // nothing here reads the buffer, so workgroup 0 clears it for the next
  // producer.
  if constexpr (!GLU && AL != 5) {
    if (p.amax && blockIdx.x == 0)
      for (uint32_t v = (uint32_t)tid; v < AMAX_WORDS / 4u; v += (uint32_t)(NW * 64))
        reinterpret_cast<u32x4*>(p.amax)[v] = u32x4{0u, 0u, 0u, 0u};
  }
  const int WK = p.waves_k;
  const int wn = wave / WK;
  const int wk = wave - wn * WK;
  const int BN = (!GLU && row_tile) ? row_tile : (NW / WK) * RG * 16;
  const int tile = blockIdx.x / p.split;
  const int chunk = blockIdx.x - tile * p.split;
  const int kb0 = chunk * p.chunk_kb;
  const int kb1 = min(p.G, kb0 + p.chunk_kb);
  const int nkc = kb1 - kb0;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int row_base = tile * BN + wn * RG * 16;

  const uint32_t M = (uint32_t)p.M, N = (uint32_t)p.N, K = (uint32_t)p.K;
  // rows this workgroup may load and store (GLU plans use obase / IH instead)
  const uint32_t row_end = min(N, (uint32_t)(tile * BN + BN));
  // GLU: output columns obase.. of this wave; weight rows of its row groups
  const uint32_t IH = N / 2u;
  const int obase = tile * (NW / WK) * 16 + wn * 16;
  auto grow = [&](int rg) -> int { return GLU ? (rg == 0 ? obase : (int)IH + obase) : row_base + rg * 16; };
  // is the element at offset x of row group rg a real output?
  auto rowok = [&](int rg, uint32_t x) -> bool {
    return GLU ? (uint32_t)obase + x < IH : (uint32_t)grow(rg) + x < row_end;
  };
  const uint32_t NT16 = (N + 15u) / 16u;  // 16-row groups (tiles along N of the packed layout)
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w, WP ? NT16 * (uint32_t)p.G * WTILE : N * K);
  const uint32_t MT16 = (M + 15u) / 16u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, (AL >= 2) ? MT16 * (uint32_t)p.G * 2048u : M * K);

  // Loop-invariant lane offsets.  A row past the end gets a base of 2^31:
  // adding any in-range K offset (< 2^30) keeps it beyond num_records
  // (<= 2^30) without wrapping, so its loads return zeros.
  const uint32_t glo = (uint32_t)g * 16u;
  uint32_t wbase[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const uint32_t row = (uint32_t)(grow(rg) + r16);
    wbase[rg] = row < row_end ? row * K + glo : OOB;
  }
  // WL (coalesced weight stream): the two loads of a (row group, K block)
  // each cover 8 whole rows x 128 bytes -- lane l takes row 8*i + l/8 and
  // 16-byte chunk l%8 -- and an LDS transpose hands the matrix core its
  // operand layout afterwards.
  const uint32_t c16 = (uint32_t)(lane & 7) * 16u;
  uint32_t wbase_c[RG][2];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t row = (uint32_t)(grow(rg) + 8 * i + (lane >> 3));
      wbase_c[rg][i] = row < row_end ? row * K + c16 : OOB;
    }
  // WP (packed tiles): tile (t, kb) is 2 KB at (t*G + kb)*2048 holding exactly
  // the two 16-byte pieces every lane feeds the matrix core, lane l's `lo` at
  // l*16 and `hi` at 1024 + l*16; padding rows / K are zeros in the tile.
  // MXFP4: 1 KB tiles, one 16-byte piece a lane (32 E2M1 values).  A row
  // group that starts inside a tile (a row tile that is not a multiple of
  // 16) reads each lane's row from the tile that holds it: row r sits in
  // tile r/16 at the lane slot of row r%16 (for an aligned group, the lane's
  // own slot).
  uint32_t wbase_p[RG];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    if constexpr (GLU || FMT == FMT_MX4) {
      const uint32_t t = (uint32_t)(grow(rg) / 16);
      wbase_p[rg] = (t < NT16 && rowok(rg, 0)) ? t * (uint32_t)p.G * WTILE + (uint32_t)lane * 16u : OOB;
    } else {
      const uint32_t row = (uint32_t)(grow(rg) + r16);
      wbase_p[rg] = row < row_end ? (row / 16u) * (uint32_t)p.G * WTILE + ((row & 15u) + 16u * (uint32_t)g) * 16u
                                  : OOB;
    }
  }
  // LDS slots of the transpose: 2 per wave, each RG x 2 KB, after the
  // staged activations.
  const int wl_base = (ALDS ? p.chunk_kb * MT * 2048 : 0) + wave * (2 * RG * 2048);

  // Activation lane bases.  Row-major: row m, K offset 16g of each block.
  // Packed: lane l's two pieces of tile (mt, kb) at (mt*G + kb)*2048 + l*16
  // (+1024).  Lanes of tokens >= M get OOB in both, so at small M a load
  // instruction moves only the valid rows.
  uint32_t abase[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const uint32_t m = (uint32_t)(mt * 16 + r16);
    if constexpr (AP)
      abase[mt] = m < M ? (uint32_t)mt * (uint32_t)p.G * 2048u + (uint32_t)lane * 16u : OOB;
    else
      abase[mt] = m < M ? m * K + glo : OOB;
  }

  // Fused LDS image: the wave amax partials (64 floats) at FA_RED, s_a of the
  // 16 tokens at FA_SC, a 16-byte zero slot at FA_ZERO, then
  // the codes of token m at FA0 + m*CH for this chunk's K range.  CH adds 64
  // bytes to the chunk so consecutive tokens start 16 banks apart.  Lanes of
  // tokens >= M read the zero slot for every K block.  Block_FP8 keeps its
  // group scales s_a[m, kb0 + kbl] after the codes, at FA_SB + (m*chunk_kb + kbl)*4.
  constexpr int FA_RED = 0, FA_SC = 256, FA_ZERO = 384, FA0 = 512;
  const int CH = p.chunk_kb * 128 + 64;
  const int FA_SB = FA0 + p.M * CH;
  const bool real_tok = (uint32_t)r16 < M;
  const int fa_lane = real_tok ? FA0 + r16 * CH + g * 16 : FA_ZERO;
  const int fa_step = real_tok ? 128 : 0;
  const int fa_hi = real_tok ? 64 : 0;

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

  // MXFP8 scales are bytes in lane order: 64 per (16-row group, K block)
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(
      p.sa, MXS ? MT16 * (uint32_t)p.G * 64u : (FMT == FMT_BLOCK ? M * (uint32_t)p.G : M) * 4u);
  const __amdgpu_buffer_rsrc_t rsw = make_rsrc(
      p.sw, MXS ? NT16 * (uint32_t)p.G * 64u
                : (FMT == FMT_BLOCK ? ((N + 127u) / 128u) * (uint32_t)p.G : N) * 4u);
  // MXFP8: the scale byte lane l hands the matrix core with K block kb (that
  // of row l%16 of the operand's 16-row group and 32-wide block 4*kb + l/16)
  // is byte l of the group's 64 for that block, so a wave reads 64
  // contiguous bytes.  Padding rows hold 0 (their operand rows are zero).
  uint32_t xsa[MT], xsw[RG];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
    xsa[mt] = (uint32_t)mt < MT16 ? (uint32_t)mt * (uint32_t)p.G * 64u + (uint32_t)lane : OOB;
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) {
    const uint32_t t = (uint32_t)(grow(rg) / 16);
    xsw[rg] = (t < NT16 && rowok(rg, 0)) ? t * (uint32_t)p.G * 64u + (uint32_t)lane : OOB;
  }

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
      if constexpr (WP) {
        const uint32_t tofs = (uint32_t)kb * WTILE;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          wb[q][rg].lo = bload16_nt(rw, ok ? wbase_p[rg] + tofs : OOB);
          if constexpr (FMT == FMT_MX4)
            wb[q][rg].hi = u32x4{0u, 0u, 0u, 0u};
          else
            wb[q][rg].hi = bload16_nt(rw, ok ? wbase_p[rg] + tofs + 1024u : OOB);
        }
      } else if constexpr (WL) {
        const bool c_ok = c16 < rem;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          wb[q][rg].lo = bload16(rw, c_ok ? wbase_c[rg][0] + kofs : OOB);
          wb[q][rg].hi = bload16(rw, c_ok ? wbase_c[rg][1] + kofs : OOB);
        }
      } else {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          wb[q][rg].lo = bload16(rw, lo_ok ? wbase[rg] + kofs : OOB);
          wb[q][rg].hi = bload16(rw, hi_ok ? wbase[rg] + kofs + 64u : OOB);
        }
      }
      if constexpr (AP) {
        const uint32_t tofs = (uint32_t)kb * 2048u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          ab[q][mt].lo = bload16(ra, ok ? abase[mt] + tofs : OOB);
          ab[q][mt].hi = bload16(ra, ok ? abase[mt] + tofs + 1024u : OOB);
        }
      } else if constexpr (!ALDS) {
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
            if constexpr (FUSED)
              sab[q][mt][r] = 0.f;   // read from LDS when consumed
            else
              sab[q][mt][r] = bload_f32(rsa, (ok && m < M) ? (m * Gu + (uint32_t)kb) * 4u : OOB);
          }
        }
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          // the 128-row block of this lane's row(s): its one row (standard
          // orientation) or its four rows 4g..4g+3, which never straddle a
          // 128-row boundary (groups start at multiples of 8); a row group
          // of a row tile may straddle one, so the block is taken per lane
          const uint32_t rs = (uint32_t)grow(rg) + (SWAP ? 4u * (uint32_t)g : (uint32_t)r16);
          swb[q][rg] = bload_f32(rsw, (ok && rs < N) ? ((rs >> 7) * Gu + (uint32_t)kb) * 4u : OOB);
        }
      }
      if constexpr (MXS) {
        // scale bytes ride in the float slots as raw bits (no arithmetic touches them)
        const uint32_t sofs = (uint32_t)kb * 64u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) sab[q][mt][0] = __int_as_float(bload_u8(rsa, ok ? xsa[mt] + sofs : OOB));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) swb[q][rg] = __int_as_float(bload_u8(rsw, ok ? xsw[rg] + sofs : OOB));
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
      if constexpr (FUSED) {
        const int j = batch * PF + q;
        const int kbl = j < nkw ? wk + j * WK : 0;
        const uint8_t* base = smem + fa_lane + kbl * fa_step;
        af[0].lo = *reinterpret_cast<const u32x4*>(base);
        af[0].hi = *reinterpret_cast<const u32x4*>(base + fa_hi);
        if constexpr (FMT == FMT_BLOCK) {
#pragma unroll
          for (int r = 0; r < (SWAP ? 1 : 4); ++r) {
            const uint32_t m = SWAP ? (uint32_t)r16 : (uint32_t)(4 * g + r);
            sab[q][0][r] = (j < nkw && m < M)
                               ? reinterpret_cast<const float*>(smem + FA_SB)[m * (uint32_t)p.chunk_kb + (uint32_t)kbl]
                               : 0.f;
          }
        }
      } else if constexpr (ALDS) {
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
      // Weight operands.  WL: write the 8-row x 128-byte pieces to this wave's
      // LDS slot (16-byte chunk c of row r at r*128 + (c ^ (r/2 % 8))*16, a
      // swizzle that keeps both the writes and the operand reads free of bank
      // conflicts), then read row l%16, chunks l/16 and 4 + l/16 back.
      Frag wf[RG];
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        if constexpr (WL) {
          uint8_t* slot = smem + wl_base + (q & 1) * (RG * 2048) + rg * 2048;
          const int wr0 = lane >> 3, wc = lane & 7;
          *reinterpret_cast<u32x4*>(slot + wr0 * 128 + ((wc ^ ((wr0 >> 1) & 7)) << 4)) = wb[q][rg].lo;
          const int wr1 = 8 + wr0;
          *reinterpret_cast<u32x4*>(slot + wr1 * 128 + ((wc ^ ((wr1 >> 1) & 7)) << 4)) = wb[q][rg].hi;
          const int sw = (r16 >> 1) & 7;
          wf[rg].lo = *reinterpret_cast<const u32x4*>(slot + r16 * 128 + ((g ^ sw) << 4));
          wf[rg].hi = *reinterpret_cast<const u32x4*>(slot + r16 * 128 + (((4 + g) ^ sw) << 4));
        } else {
          wf[rg] = wb[q][rg];
        }
      }
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if constexpr (FMT == FMT_INT8) {
            if (SWAP) {
              acc[rg][mt] = mma_i8(wf[rg].lo, af[mt].lo, acc[rg][mt]);
              acc[rg][mt] = mma_i8(wf[rg].hi, af[mt].hi, acc[rg][mt]);
            } else {
              acc[rg][mt] = mma_i8(af[mt].lo, wf[rg].lo, acc[rg][mt]);
              acc[rg][mt] = mma_i8(af[mt].hi, wf[rg].hi, acc[rg][mt]);
            }
          } else if constexpr (FMT == FMT_FP8) {
            acc[rg][mt] = SWAP ? mma_f8(wf[rg], af[mt], acc[rg][mt])
                               : mma_f8(af[mt], wf[rg], acc[rg][mt]);
          } else if constexpr (FMT == FMT_MX) {
            const int xa = __float_as_int(sab[q][mt][0]);
            const int xw = __float_as_int(swb[q][rg]);
            acc[rg][mt] = SWAP ? mma_f8_mx(wf[rg], af[mt], acc[rg][mt], xw, xa)
                               : mma_f8_mx(af[mt], wf[rg], acc[rg][mt], xa, xw);
          } else if constexpr (FMT == FMT_MX4) {
            const int xa = __float_as_int(sab[q][mt][0]);
            const int xw = __float_as_int(swb[q][rg]);
            acc[rg][mt] = mma_f8f4_mx<SWAP>(af[mt], wf[rg].lo, acc[rg][mt], xa, xw);
          } else {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 part = SWAP ? mma_f8(wf[rg], af[mt], z) : mma_f8(af[mt], wf[rg], z);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              // (P_g * s_a) * s_w: the group sum meets the activation scale
              // first, so a tiny s_a cannot underflow a product of scales
              const float t = __fmul_rn(part[r], sab[q][mt][SWAP ? 0 : r]);
              acc[rg][mt][r] = __builtin_fmaf(t, swb[q][rg], acc[rg][mt][r]);
            }
          }
        }
      }
    }
  };

  // ---- scales of the per-token formats for the epilogue, issued before any
  // other load: they depend on nothing, so their latency passes while the
  // first weight batches are on their way, also where a wave has only a few
  // K blocks to stream (measured 2-4 % faster on such points than issuing
  // them after the first batches).  Issued first, they are older than every
  // load the explicit waits below count.  Fused plans load them after their
  // prologue (below).
  float esa[MT][4], esw[RG][4];
  if constexpr (FMT != FMT_BLOCK && !MXS && !FUSED) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
        esa[mt][r] = (SWAP && r > 0) ? 0.f : bload_f32(rsa, m < M ? m * 4u : OOB);
      }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t n = (uint32_t)grow(rg) + (SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16);
        esw[rg][r] = (!SWAP && r > 0) ? 0.f : bload_f32(rsw, n < N ? n * 4u : OOB);
      }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- stage this chunk's activations in LDS first, with LDS-DMA buffer
  // loads (no registers; their completion is awaited below, after the first
  // weight batches are in flight): one 1 KB block b per (K block kbl, token
  // tile mt, half h), b = (kbl*MT + mt)*2 + h, in which lane l holds token
  // 16*mt + l%16, K bytes [h*64 + 16*(l/16), +16) of the K block.  Packed
  // activations hold exactly these blocks contiguously; row-major ones are
  // gathered 16 rows x 16 bytes at a time.
  if constexpr (ALDS && !FUSED) {
    const int nblk = nkc * MT * 2;
    for (int b = wave; b < nblk; b += NW) {
      const int h = b & 1;
      const int mt = (b >> 1) % MT;
      const int kbl = (b >> 1) / MT;
      uint32_t off;
      if constexpr (AL == 3) {
        off = (uint32_t)mt < MT16
                  ? ((uint32_t)mt * (uint32_t)p.G + (uint32_t)(kb0 + kbl)) * 2048u + (uint32_t)h * 1024u +
                        (uint32_t)lane * 16u
                  : OOB;
      } else {
        const uint32_t m = (uint32_t)(mt * 16 + r16);
        const uint32_t k = (uint32_t)(kb0 + kbl) * 128u + (uint32_t)h * 64u + (uint32_t)g * 16u;
        off = (m < M && k < K) ? m * K + k : OOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          ra, (__attribute__((address_space(3))) void*)(smem + b * 1024), 16, off, 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- fused quantization, part 1: X is read first, so that waiting for it
  // below leaves the weight batches issued after it in flight.  With K a
  // multiple of 512 each wave's 64 consecutive 16-byte pieces (one load
  // instruction) lie in one token row; the workgroup holds XP pieces a lane,
  // 16384 values in all.
  // Block_FP8 needs only this chunk's K range (its 1 x 128 groups are
  // local): pieces run row by row over the chunk, nkc*16 a row, and the 16
  // lanes of a row of the wave hold one group.
  constexpr int XP = FUSED ? 32 / NW : 1;
  u32x4 xv[XP];
  const uint32_t upr = K / 512u;                 // per-token: wave pieces per token row
  const uint32_t ppr = (uint32_t)nkc * 16u;      // chunked: pieces per row of the chunk
  // Activation mode 5: every replica's maxima of the M tokens, AMW words a
  // thread, loaded first (older than the X and weight loads, so the wait for
  // X covers them).  The producer was an earlier kernel of the stream, whose
  // atomics were complete and visible device-wide when it ended, so plain
  // loads see them.  The maxima over the replicas are folded in LDS
  // (FA_RED, zeroed here) after that wait.
  constexpr int AMW = AL == 5 ? (int)((AMAX_REPLICAS * 16u + NW * 64 - 1) / (NW * 64)) : 1;
  uint32_t amw[AMW];
  if constexpr (AL == 5) {
    const __amdgpu_buffer_rsrc_t ram = make_rsrc(p.amax, AMAX_WORDS * 4u);
    const uint32_t nwords = AMAX_REPLICAS * M;
#pragma unroll
    for (int i = 0; i < AMW; ++i) {
      const uint32_t j = (uint32_t)(tid + NW * 64 * i);
      const uint32_t r = j / M;
      amw[i] = __float_as_uint(bload_f32(ram, j < nwords ? (r * AMAX_LINE + (j - r * M)) * 4u : OOB));
    }
    if (tid < (int)AMAX_LINE) reinterpret_cast<uint32_t*>(smem + FA_RED)[tid] = 0u;
  }
  if constexpr (FUSED) {
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, M * K * 2u);
    const uint32_t npc = CHUNKED ? M * ppr : M * K / 8u;
    // a wave issues only the loads whose pieces exist (a wave-uniform test;
    // the wait below counts the weight loads, which are all younger)
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const uint32_t P = (uint32_t)(tid + NW * 64 * i);
      xv[i] = u32x4{0u, 0u, 0u, 0u};
      if ((uint32_t)(wave * 64 + NW * 64 * i) < npc) {
        uint32_t off;
        if constexpr (CHUNKED) {
          const uint32_t m = P / ppr, w = P - m * ppr;
          off = (m * K + (uint32_t)kb0 * 128u + w * 8u) * 2u;
        } else {
          off = P * 16u;
        }
        xv[i] = bload16(rx, P < npc ? off : OOB);
      }
    }
    if (tid < 4) reinterpret_cast<uint32_t*>(smem + FA_ZERO)[tid] = 0u;
    __builtin_amdgcn_sched_barrier(0);
  }

  // Two batches in flight: the loop enters and repeats with the same pair of
  // buffers outstanding (batch b in wb0, b+1 in wb1), and each buffer is
  // refilled right after it has been consumed.  (Four batches during a fused
  // prologue, so that the weight stream would not idle while X is read and
  // quantized, made the FP8 and INT8 fused launches 3-24 % slower: the
  // prologue's cost is its quantization arithmetic, not a weight stall.)
  issue(wb0, ab0, sa0, sw0, 0);
  issue(wb1, ab1, sa1, sw1, 1);

  // ---- fused quantization, part 2: wait for X only, then per token row:
  // amax (each wave's partial, then the row's partials), s = fl(amax/Q) and
  // fl(1/s) in every wave that holds a piece of the row, and the codes of
  // this chunk's K range into LDS.
  if constexpr (FUSED && FMT == FMT_BLOCK) {
    // weight loads and weight-scale loads of the two batches, issued after X
    constexpr int NW_LOADS = 2 * PF * 3 * RG;
    static_assert(NW_LOADS <= 63, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((NW_LOADS & 15) | (7 << 4) | (15 << 8) | ((NW_LOADS >> 4) << 14));
    float* ssb = reinterpret_cast<float*>(smem + FA_SB);
    const uint32_t npc = M * ppr;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const uint32_t P = (uint32_t)(tid + NW * 64 * i);
      if ((uint32_t)(wave * 64 + NW * 64 * i) >= npc) continue;   // no piece of this wave
      const float gmax = row16_max_nonneg(abs_bf16_max8(xv[i], 0.0f));
      if (P < npc) {
        const uint32_t m = P / ppr, w = P - m * ppr;
        const float sc = scale_of<FMT>(gmax);
        *reinterpret_cast<u32x2*>(smem + FA0 + m * (uint32_t)CH + w * 8u) = quant8<FMT>(xv[i], sc, recip_of(sc));
        if ((w & 15u) == 0u) ssb[m * (uint32_t)p.chunk_kb + (w >> 4)] = sc;
      }
    }
    lds_barrier();
    if (p.aq_out && tile == 0) {
      for (uint32_t v = (uint32_t)tid; v < M * (uint32_t)nkc; v += (uint32_t)(NW * 64)) {
        const uint32_t m = v / (uint32_t)nkc, kbl = v - m * (uint32_t)nkc;
        p.sa_out[m * (uint32_t)p.G + (uint32_t)kb0 + kbl] = ssb[m * (uint32_t)p.chunk_kb + kbl];
      }
    }
  } else if constexpr (AL == 5) {
    constexpr int NW_LOADS = 2 * PF * 2 * RG;  // weight loads of the two batches, issued after X
    static_assert(NW_LOADS <= 63, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((NW_LOADS & 15) | (7 << 4) | (15 << 8) | ((NW_LOADS >> 4) << 14));
    float* ssc = reinterpret_cast<float*>(smem + FA_SC);
    uint32_t* amx = reinterpret_cast<uint32_t*>(smem + FA_RED);
    lds_barrier();   // the zeroed token maxima
    {
      const uint32_t nwords = AMAX_REPLICAS * M;
#pragma unroll
      for (int i = 0; i < AMW; ++i) {
        const uint32_t j = (uint32_t)(tid + NW * 64 * i);
        if (j < nwords) __hip_atomic_fetch_max(amx + (j % M), amw[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
    lds_barrier();
    const uint32_t npc = M * ppr;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const uint32_t P = (uint32_t)(tid + NW * 64 * i);
      if ((uint32_t)(wave * 64 + NW * 64 * i) >= npc) continue;   // no piece of this wave
      if (P < npc) {
        const uint32_t m = P / ppr, w = P - m * ppr;
        const float sc = scale_of<FMT>(__uint_as_float(amx[m]));
        *reinterpret_cast<u32x2*>(smem + FA0 + m * (uint32_t)CH + w * 8u) = quant8<FMT>(xv[i], sc, recip_of(sc));
        if (w == 0u) ssc[m] = sc;
      }
    }
    lds_barrier();
    // Every wave of this workgroup has read the buffer (the wait above), so
    // count the workgroup: in its group's counter, and the workgroup that
    // completes a group in the counter of groups.  The one that completes
    // the last group -- every workgroup of the grid has then read the
    // maxima -- zeroes the replicas (wave 0); each counter is reset by the
    // workgroup that completed it.
    if (wave == 0) {
      uint32_t last = 0;
      if (lane == 0) {
        const uint32_t grp = blockIdx.x % AMAX_GROUPS;
        const uint32_t members = (gridDim.x - grp + AMAX_GROUPS - 1u) / AMAX_GROUPS;
        uint32_t* gctr = p.amax + AMAX_CTR0 + grp * AMAX_LINE;
        if (__hip_atomic_fetch_add(gctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == members - 1u) {
          __hip_atomic_exchange(gctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const uint32_t ngroups = min(gridDim.x, AMAX_GROUPS);
          if (__hip_atomic_fetch_add(p.amax + AMAX_TOP, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              ngroups - 1u) {
            __hip_atomic_exchange(p.amax + AMAX_TOP, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = 1;
          }
        }
      }
      if (__builtin_amdgcn_readfirstlane(last)) {
        for (uint32_t v = (uint32_t)lane; v < AMAX_CTR0 / 4u; v += 64u)
          reinterpret_cast<u32x4*>(p.amax)[v] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (p.aq_out && tile == 0 && chunk == 0 && (uint32_t)tid < M) p.sa_out[tid] = ssc[tid];
  } else if constexpr (FUSED) {
    constexpr int NW_LOADS = 2 * PF * 2 * RG;  // weight loads of the two batches, issued after X
    static_assert(NW_LOADS <= 63, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((NW_LOADS & 15) | (7 << 4) | (15 << 8) | ((NW_LOADS >> 4) << 14));
    float* red = reinterpret_cast<float*>(smem + FA_RED);
    float* ssc = reinterpret_cast<float*>(smem + FA_SC);
    const uint32_t nu = M * upr;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const uint32_t u = (uint32_t)(wave + NW * i);
      if (u >= nu) continue;   // wave-uniform: no piece of this wave
      const float m = wave_max_nonneg(abs_bf16_max8(xv[i], 0.0f));
      if (lane == 0) red[u] = m;
    }
    lds_barrier();
    const uint32_t k_lo = (uint32_t)kb0 * 128u, k_hi = (uint32_t)kb1 * 128u;
#pragma unroll
    for (int i = 0; i < XP; ++i) {
      const uint32_t u = (uint32_t)(wave + NW * i);
      if (u < nu) {
        const uint32_t m = u / upr;
        float amax = 0.0f;
        for (uint32_t v = m * upr; v < (m + 1u) * upr; ++v) amax = fmaxf(amax, red[v]);
        const float sc = scale_of<FMT>(amax);
        if (lane == 0 && u == m * upr) ssc[m] = sc;
        const uint32_t k = (u - m * upr) * 512u + (uint32_t)lane * 8u;
        if (k >= k_lo && k < k_hi)
          *reinterpret_cast<u32x2*>(smem + FA0 + m * (uint32_t)CH + (k - k_lo)) =
              quant8<FMT>(xv[i], sc, recip_of(sc));
      }
    }
    lds_barrier();
    if (p.aq_out && tile == 0 && chunk == 0 && (uint32_t)tid < M) p.sa_out[tid] = ssc[tid];
  }
  // The codes leave the kernel as the standalone quantizer writes them: this
  // chunk's packed tiles (token tile 0; rows >= M zero), spread over the
  // chunk's workgroups.  (The scales were written above.)
  if constexpr (FUSED) {
    if (p.aq_out) {
      const uint32_t nunits = (uint32_t)nkc * 128u;  // 16-byte units: K block x half x lane
      for (uint32_t u = (uint32_t)(tile * NW * 64 + tid); u < nunits; u += (uint32_t)(p.n_tiles * NW * 64)) {
        const uint32_t kbl = u >> 7, h = (u >> 6) & 1u, l = u & 63u;
        const uint32_t row = l & 15u;
        const uint32_t k = kbl * 128u + h * 64u + (l >> 4) * 16u;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row < M) v = *reinterpret_cast<const u32x4*>(smem + FA0 + row * (uint32_t)CH + k);
        *reinterpret_cast<u32x4*>(p.aq_out + (size_t)((uint32_t)kb0 + kbl) * 2048u + h * 1024u + l * 16u) = v;
      }
    }
  }

  // Fused plans: the token scales the prologue computed and the weight
  // scales, for the epilogue.  (Issued before X instead, the weight-scale
  // loads made the fused launches up to 16 % slower.)
  if constexpr (FMT != FMT_BLOCK && !MXS && FUSED) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
        esa[mt][r] = m < M ? reinterpret_cast<const float*>(smem + FA_SC)[m] : 0.f;
      }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t n = (uint32_t)grow(rg) + (SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16);
        esw[rg][r] = (!SWAP && r > 0) ? 0.f : bload_f32(rsw, n < N ? n * 4u : OOB);
      }
  }

  // ---- activations staged in LDS: wait for the staging copies (issued
  // before the weight batches, and vmcnt counts in issue order) while the
  // weight batches stay in flight, then make LDS visible workgroup-wide.
  if constexpr (ALDS && !FUSED) {
    // loads of the two batches, all issued after the copies: 2*RG weight loads
    // per K block (a lower bound where scale loads follow; MXFP4 weights take
    // one load per row group, then RG + MT scale loads, 2*RG + MT in all)
    constexpr int NW_LOADS = 2 * PF * (FMT == FMT_MX4 ? 2 * RG + MT : 2 * RG);
    static_assert(NW_LOADS <= 63, "vmcnt holds 6 bits");
    __builtin_amdgcn_s_waitcnt((NW_LOADS & 15) | (7 << 4) | (15 << 8) | ((NW_LOADS >> 4) << 14));
    lds_barrier();
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
            red[(wave * NACC + i) * 64 + lane] = bits_of(acc[rg][mt][r]);
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
                acc[rg][mt][r] += __int_as_float(v);
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
            const uint32_t x = SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16;
            const uint32_t n = (uint32_t)grow(rg) + x;
            const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
            if (m < M && rowok(rg, x)) {
              if constexpr (FMT == FMT_INT8)
                __hip_atomic_fetch_add(reinterpret_cast<int*>(p.ws) + (size_t)m * N + n, acc[rg][mt][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              else
                __hip_atomic_fetch_add(reinterpret_cast<float*>(p.ws) + (size_t)m * N + n, acc[rg][mt][r],
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
    }
    // Every access to the workspace and the counters is a device-scope atomic
    // read-modify-write, which the hardware performs at a point coherent for
    // all XCDs, so no L2 write-back / invalidate (an agent-scope fence) is
    // needed -- only that this workgroup's adds have completed before its
    // arrival is counted: wait for every outstanding memory operation.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned prev = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (unsigned)(p.split - 1));
    }
    __syncthreads();
    if (!s_last) return;
    if (wk == 0) {
#pragma unroll
      for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t x = SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16;
            const uint32_t n = (uint32_t)grow(rg) + x;
            const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
            if (m < M && rowok(rg, x)) {
              int* slot = reinterpret_cast<int*>(p.ws) + (size_t)m * N + n;
              const int v = __hip_atomic_exchange(slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              if constexpr (FMT == FMT_INT8)
                acc[rg][mt][r] = v;
              else
                acc[rg][mt][r] = __int_as_float(v);
            }
          }
    }
    if (tid == 0) __hip_atomic_exchange(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  if (wk != 0) return;

  // ---- SiLU-and-mul epilogue: the gate (row group 0) and up (1) values of
  // an output element are the binary32 epilogue values of the two rows;
  // h = g / (1 + exp(-g)) * u, rounded to bf16 once, stored to Y [M, N/2].
  if constexpr (GLU) {
    // |bf16(h)| of each stored element, for the per-token amax of H
    float habs[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t x = SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16;
        const uint32_t m = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
        habs[mt][r] = 0.0f;
        float t[2];
#pragma unroll
        for (int rg = 0; rg < 2; ++rg) {
          if constexpr (FMT == FMT_BLOCK || MXS) {
            t[rg] = acc[rg][mt][r];
          } else {
            float accf;
            if constexpr (FMT == FMT_INT8)
              accf = __int2float_rn(acc[rg][mt][r]);
            else
              accf = acc[rg][mt][r];
            t[rg] = __fmul_rn(__fmul_rn(accf, esa[mt][SWAP ? 0 : r]), esw[rg][SWAP ? r : 0]);
          }
        }
        const float h = __fmul_rn(__fdiv_rn(t[0], 1.0f + expf(-t[0])), t[1]);
        if (m < M && rowok(0, x)) {
          const uint32_t hb = bf16_rne(h);
          p.y[(size_t)m * IH + (uint32_t)obase + x] = (uint16_t)hb;
          habs[mt][r] = bf16_to_f32(hb & 0x7fffu);
        }
      }
    }
    // Per-token amax of H for a consumer that quantizes it (activation mode
    // 5): the largest |h| of each token over this wave's columns, then an
    // atomic maximum on its binary32 bit pattern (non-negative, so the
    // integer order is the numeric one; exact whatever the order).
    if (p.amax) {
      // this wave's replica of the maxima (spreads the atomics over lines)
      uint32_t* am = p.amax + ((uint32_t)blockIdx.x * (uint32_t)(NW / WK) + (uint32_t)wn) % AMAX_REPLICAS * AMAX_LINE;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if constexpr (SWAP) {
          // lane: token 16mt + r16, columns 4g..4g+3 -> fold r, then the four lane groups
          float v = fmaxf(fmaxf(habs[mt][0], habs[mt][1]), fmaxf(habs[mt][2], habs[mt][3]));
          v = fmaxf(v, __shfl_xor(v, 16));
          v = fmaxf(v, __shfl_xor(v, 32));
          const uint32_t m = (uint32_t)(mt * 16 + r16);
          if (g == 0 && m < M)
            __hip_atomic_fetch_max(am + m, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          // lane: column r16, tokens 16mt + 4g + r -> fold the 16 columns of the DPP row
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float v = row16_max_nonneg(habs[mt][r]);
            const uint32_t m = (uint32_t)(mt * 16 + 4 * g + r);
            if (r16 == 0 && m < M)
              __hip_atomic_fetch_max(am + m, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    return;
  }

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
        nn[r] = (uint32_t)grow(rg) + (SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16);
        mm[r] = SWAP ? (uint32_t)(mt * 16 + r16) : (uint32_t)(mt * 16 + 4 * g + r);
        const bool ok = mm[r] < M && nn[r] < row_end;
        if constexpr (FMT == FMT_BLOCK || MXS) {
          out[r] = bf16_rne(acc[rg][mt][r]);
          if (ok && p.acc_out)
            reinterpret_cast<float*>(p.acc_out)[(size_t)mm[r] * N + nn[r]] = acc[rg][mt][r];
        } else {
          const float sa = esa[mt][SWAP ? 0 : r];
          const float sw = esw[rg][SWAP ? r : 0];
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
      if (vec4 && mm[0] < M && nn[3] < row_end) {
        u32x2 v = {out[0] | (out[1] << 16), out[2] | (out[3] << 16)};
        *reinterpret_cast<u32x2*>(p.y + (size_t)mm[0] * N + nn[0]) = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (mm[r] < M && nn[r] < row_end) p.y[(size_t)mm[r] * N + nn[r]] = (uint16_t)out[r];
      }
    }
  }
}

// Instantiation table for one format.  Row-major weights (direct or LDS
// transpose) and LDS-staged activations use 4-wave workgroups with 16 or 32
// rows per wave and 2- or 4-block batches.  Packed weights additionally get
// 8- and 16-wave workgroups, 64 rows per wave and 1-block batches.  A shape
// whose buffers would not fit the register file of its occupancy (256
// VGPRs a wave up to 8 waves per workgroup, 128 at 16 waves) is not
// instantiated, and the planner rejects it.
template <int FMT, int NW_, int SW, int MT_, int RG_, int PF_>
constexpr bool decode_config_fits() {
  if (NW_ == 4 && RG_ <= 2 && PF_ >= 2 && MT_ <= 2) {
    // the original 4-wave shapes (checked one by one against the compiler)
    if (MT_ == 2 && RG_ == 2 && PF_ == 4) return false;
    if (FMT == FMT_BLOCK && MT_ == 2 && PF_ == 4 && !SW) return false;
    return true;
  }
  // two batches of PF blocks of (RG weight + MT activation) fragments, 8 VGPRs each
  const int buffers = 2 * PF_ * (RG_ + MT_) * 8;
  const int scales =
      FMT == FMT_BLOCK ? 2 * PF_ * (4 * MT_ + RG_) : (FMT == FMT_MX || FMT == FMT_MX4) ? 2 * PF_ * (MT_ + RG_) : 0;
  const int accs = RG_ * MT_ * 4;
  const int budget = NW_ >= 16 ? 128 : 256;
  // Block_FP8 keeps per-block partial products and scale factors live as well
  const int estimate = (buffers + scales + accs + 40) * (FMT == FMT_BLOCK ? 135 : 100) / 100;
  if (estimate > budget) return false;
  if (NW_ * RG_ * MT_ > 64) return false;  // cross-wave reduction must fit 64 KB of LDS
  return true;
}

// MXFP8 shapes whose register allocation spills (checked one by one against
// the compiler's resource report): the scaled instruction keeps its
// operands and scale bytes in VGPRs, which costs more than the unscaled E4M3
// path, above all with two token tiles held in registers (AL == 2).
template <int NW_, int MT_, int RG_, int PF_, int AL>
constexpr bool mx_spills() {
  if (NW_ == 4) return MT_ == 2 && RG_ == 1 && PF_ == 4 && AL == 2;
  if (NW_ == 8)
    return (MT_ == 1 && RG_ == 4 && PF_ == 2) || (MT_ == 2 && PF_ == 2 && (RG_ == 2 || AL == 2)) ||
           (MT_ == 2 && RG_ == 4 && AL == 2) || (MT_ == 4 && (PF_ == 2 || RG_ == 2));
  if (NW_ == 16) return MT_ == 2 && (RG_ == 2 || AL == 2);
  return false;
}

// The MXFP4 shapes that spill (same check): its weight fragments are half as
// large, so only some shapes holding activations in registers remain.
template <int NW_, int MT_, int RG_, int PF_, int AL>
constexpr bool mx4_spills() {
  if (AL != 2) return false;
  if (NW_ == 8)
    return (MT_ == 1 && RG_ == 4 && PF_ == 2) || (MT_ == 2 && RG_ == 2 && PF_ == 2) ||
           (MT_ == 4 && (PF_ == 2 || RG_ == 2));
  if (NW_ == 16) return MT_ == 2 && RG_ == 2;
  return false;
}

// Fused quantization adds 32/NW 16-byte X pieces a lane to the buffers in
// flight; it serves one token tile and packed weights.
template <int FMT, int NW_, int SW, int MT_, int RG_, int PF_, int AL, int WM_>
constexpr bool decode_variant_ok() {
  if constexpr (FMT == FMT_MX) {
    if (mx_spills<NW_, MT_, RG_, PF_, AL>()) return false;
  }
  if constexpr (FMT == FMT_MX4) {
    if (mx4_spills<NW_, MT_, RG_, PF_, AL>()) return false;
  }
  if constexpr (AL == 5) {
    if (FMT != FMT_FP8 && FMT != FMT_INT8) return false;
  }
  if constexpr (AL == 4 || AL == 5) {
    if (MT_ != 1 || WM_ != W_PACKED) return false;
    const int estimate = 2 * PF_ * (RG_ + MT_) * 8 + RG_ * MT_ * 4 + 40 + 4 * (32 / NW_);
    return estimate <= (NW_ >= 16 ? 128 : 256) && decode_config_fits<FMT, NW_, SW, MT_, RG_, PF_>();
  }
  return decode_config_fits<FMT, NW_, SW, MT_, RG_, PF_>();
}

template <int FMT, int NW_, int SW, int MT_, int RG_, int PF_, int AL, int WM_, int GLU = 0>
hipError_t decode_try(const DecodeKey& k, dim3 grid, dim3 block, size_t lds, hipStream_t s, const DecodeArgs& a,
                      bool probe_only, bool* hit) {
  // MXFP8 / MXFP4 are served with packed weights and packed activations only
  constexpr bool mx_ok =
      (FMT != FMT_MX && FMT != FMT_MX4) || (GLU == 0 && WM_ == W_PACKED && (AL == 2 || AL == 3));
  if constexpr (mx_ok && decode_variant_ok<FMT, NW_, SW, MT_, RG_, PF_, AL, WM_>()) {
    if (k.swap == SW && k.mt == MT_ && k.rg == RG_ && k.nw == NW_ && k.pf == PF_ && k.alds == AL && k.wm == WM_ &&
        k.glu == GLU) {
      *hit = true;
      auto fn = qgemm_decode_kernel<FMT, SW != 0, MT_, RG_, NW_, PF_, AL, WM_, GLU != 0>;
      if (probe_only) {
        // LDS beyond the default 64 KB needs the per-kernel opt-in (gfx950: 160 KB a workgroup)
        if (lds > 64 * 1024)
          return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
        return hipSuccess;
      }
      constexpr bool FUSED = AL == 4 || AL == 5;
      fn<<<grid, block, lds, s>>>(FUSED ? static_cast<const void*>(a.x) : static_cast<const void*>(a.a), a.w, a.sa,
                                  a.sw, a.amax, a.M, a.N, a.K, decode_shape_word(a), a);
      return hipGetLastError();
    }
  }
  return hipSuccess;
}

template <int FMT>
hipError_t decode_dispatch(const DecodeKey& k, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                           const DecodeArgs& a, bool probe_only) {
  bool hit = false;
  hipError_t e = hipSuccess;
#define QL_TRY(NW_, SW, MT_, RG_, PF_, AL, WM_)                                                       \
  e = decode_try<FMT, NW_, SW, MT_, RG_, PF_, AL, WM_>(k, grid, block, lds, s, a, probe_only, &hit); \
  if (hit) return e;
  // 4 waves, every weight mode and activation staging
#define QL_TRY_WL(SW, MT_, RG_, PF_, AL) \
  QL_TRY(4, SW, MT_, RG_, PF_, AL, 0) QL_TRY(4, SW, MT_, RG_, PF_, AL, 1) QL_TRY(4, SW, MT_, RG_, PF_, AL, 2)
#define QL_TRY_AL(SW, MT_, RG_, PF_)                                                      \
  QL_TRY_WL(SW, MT_, RG_, PF_, 0) QL_TRY_WL(SW, MT_, RG_, PF_, 1) QL_TRY(4, SW, MT_, RG_, PF_, 2, 2) \
  QL_TRY(4, SW, MT_, RG_, PF_, 3, 2) QL_TRY(4, SW, MT_, RG_, PF_, 4, 2) QL_TRY(4, SW, MT_, RG_, PF_, 5, 2)
#define QL_TRY_PF(SW, MT_, RG_) QL_TRY_AL(SW, MT_, RG_, 2) QL_TRY_AL(SW, MT_, RG_, 4)
#define QL_TRY_RG(SW, MT_) QL_TRY_PF(SW, MT_, 1) QL_TRY_PF(SW, MT_, 2)
  // packed weights, activations (row-major or packed) from L2: wider workgroups,
  // longer rows, 1-block batches
#define QL_TRY_PA(NW_, SW, MT_, RG_, PF_)                                                      \
  QL_TRY(NW_, SW, MT_, RG_, PF_, 0, 2) QL_TRY(NW_, SW, MT_, RG_, PF_, 2, 2) QL_TRY(NW_, SW, MT_, RG_, PF_, 3, 2) \
  QL_TRY(NW_, SW, MT_, RG_, PF_, 4, 2) QL_TRY(NW_, SW, MT_, RG_, PF_, 5, 2)
#define QL_TRY_P(NW_, SW, MT_, RG_) QL_TRY_PA(NW_, SW, MT_, RG_, 1) QL_TRY_PA(NW_, SW, MT_, RG_, 2)
#define QL_TRY_PN(SW, MT_)                                                                    \
  QL_TRY_PA(4, SW, MT_, 1, 1) QL_TRY_PA(4, SW, MT_, 2, 1) QL_TRY_P(4, SW, MT_, 4)             \
  QL_TRY_P(8, SW, MT_, 1) QL_TRY_P(8, SW, MT_, 2) QL_TRY_P(8, SW, MT_, 4)                 \
  QL_TRY_P(16, SW, MT_, 1) QL_TRY_P(16, SW, MT_, 2) QL_TRY_P(16, SW, MT_, 4)
  // four token tiles (M <= 64): packed weights, activations from L2
#define QL_TRY_P4(NW_, SW, RG_, PF_) QL_TRY(NW_, SW, 4, RG_, PF_, 0, 2) QL_TRY(NW_, SW, 4, RG_, PF_, 2, 2)
#define QL_TRY_PN4(SW)                                                                            \
  QL_TRY_P4(4, SW, 1, 1) QL_TRY_P4(4, SW, 1, 2) QL_TRY_P4(4, SW, 2, 1) QL_TRY_P4(4, SW, 2, 2)     \
  QL_TRY_P4(4, SW, 4, 1) QL_TRY_P4(8, SW, 1, 1) QL_TRY_P4(8, SW, 1, 2) QL_TRY_P4(8, SW, 2, 1)     \
  QL_TRY_P4(8, SW, 2, 2)
  // SiLU-and-mul epilogue: 32 rows a wave (a gate and an up group), packed
  // weights, activations packed from L2 or quantized in the kernel
#define QL_TRY_G1(NW_, SW, MT_, PF_, AL)                                                        \
  e = decode_try<FMT, NW_, SW, MT_, 2, PF_, AL, 2, 1>(k, grid, block, lds, s, a, probe_only, &hit); \
  if (hit) return e;
#define QL_TRY_G(SW, MT_)                                                                      \
  QL_TRY_G1(4, SW, MT_, 1, 2) QL_TRY_G1(4, SW, MT_, 2, 2) QL_TRY_G1(8, SW, MT_, 1, 2)            \
  QL_TRY_G1(8, SW, MT_, 2, 2) QL_TRY_G1(4, SW, MT_, 1, 4) QL_TRY_G1(4, SW, MT_, 2, 4)            \
  QL_TRY_G1(8, SW, MT_, 1, 4) QL_TRY_G1(8, SW, MT_, 2, 4)
#define QL_TRY_MT(SW) QL_TRY_RG(SW, 1) QL_TRY_RG(SW, 2) QL_TRY_PN(SW, 1) QL_TRY_PN(SW, 2) QL_TRY_PN4(SW) \
  QL_TRY_G(SW, 1) QL_TRY_G(SW, 2)
  QL_TRY_MT(0)
  QL_TRY_MT(1)
#undef QL_TRY_MT
#undef QL_TRY_G
#undef QL_TRY_G1
#undef QL_TRY_PN4
#undef QL_TRY_P4
#undef QL_TRY_PN
#undef QL_TRY_P
#undef QL_TRY_PA
#undef QL_TRY_RG
#undef QL_TRY_PF
#undef QL_TRY_AL
#undef QL_TRY_WL
#undef QL_TRY
  return hipErrorInvalidDeviceFunction;
}

}  // namespace qlk
