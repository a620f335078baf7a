// Tiled quantized GEMM for token counts beyond the decode range (M > 32) on
// gfx950.
//
// Same operation as the decode kernel -- Y = epilogue(A_q . W_q^T) with the
// format's scales fused ([Summary] "Put algorithm selection inside the
// search space"; [Noticias] "¿Cómo se implementa el kernel?") -- but once M
// reaches the hundreds the GEMM stops being a weight stream and becomes a
// matrix-core problem, so this kernel is a classic output-tiled GEMM: each
// workgroup owns a BM x BN output tile, and both operands pass through LDS so
// that every byte loaded from L2 feeds TM or TN matrix-core instructions.
// The pages hand these shapes to the default library path beyond their graph
// threshold ([Summary] "Hybrid dispatch addresses runtime overhead"); here
// they stay in the same library, with the same split_k / swap_ab switches.
//
// Structure (512 threads = 8 waves in a 2 x 4 grid, wave tile TM x TN =
// BM/2 x BN/4 -- Block_FP8 below 128 x 256: 256 threads, 4 waves in a 2 x 2
// grid; the 256 x 256 tile's 128 x 64 wave tile reads a quarter fewer LDS
// bytes per flop, and half the L2 bytes per flop, of 128 x 128):
//   * K advances in 128-wide blocks.  Per block, every thread loads its
//     16-byte pieces of the A tile (BM x 128) and the B tile (BN x 128) from
//     global memory into registers, and writes them into one of two LDS
//     stages in matrix-core operand order: a 16-row x 128 group becomes a
//     2 KB tile whose lane-l reads at l*16 and 1024 + l*16 give the lane its
//     two 16-byte pieces (the packed weight and activation layouts are
//     exactly this order, so packed operands copy through verbatim).  The loads for block k+1 are in
//     flight while the matrix cores work on block k: the workgroup barriers
//     order LDS only, so they do not wait for outstanding global loads.
//   * Each wave reads its TM/16 A fragments and, one at a time, its TN/16 B
//     fragments (contiguous 1 KB LDS reads), and accumulates TM/16 x TN/16
//     16x16 tiles (v_mfma_scale_f32_16x16x128_f8f6f4 for E4M3, two
//     v_mfma_i32_16x16x64_i8 for int8).  Block_FP8 applies the 1x128 and
//     128x128 scales per K block, as the decode kernel does.
//   * Split-K and the epilogue follow the decode kernel: device-scope
//     atomics into an int32 / fp32 workspace, the last workgroup of a tile
//     applies the scales and stores bf16.
//   * Workgroups are renumbered so that each XCD (which receives every
//     eighth workgroup) works on a contiguous run of tiles, and tiles run in
//     groups of 8 tile-rows so neighbouring workgroups share weight panels in
//     that XCD's L2.
#pragma once

#include "decode_args.hpp"
#include "device_common.hpp"

namespace qlk {

template <int FMT>
struct TiledAcc {
  typedef f32x4 T;
};
template <>
struct TiledAcc<FMT_INT8> {
  typedef i32x4 T;
};

// Waves along N of a tile's wave grid (along M there are always 2): 8-wave
// workgroups, whose extra waves hide the operand loads (measured on the 14B
// shapes: 10-13 % faster at M = 256 with 64 x 128 and 128 x 128 tiles, 11-19 %
// on the long-K down projection at M >= 1024 with 128 x 256).  Block_FP8
// keeps 4 waves below 128 x 256: its per-row scales would spill there.
template <int FMT, int BM, int BN>
constexpr int tiled_waves_n() {
  return (FMT != FMT_BLOCK || BM * BN >= 128 * 256) ? 4 : 2;
}

template <int FMT, bool SWAP, int BM, int BN, int WM, int PF, bool AP, int NS>
__global__ void __launch_bounds__((64 * 2 * tiled_waves_n<FMT, BM, BN>())) qgemm_tiled_kernel(DecodeArgs p) {
  constexpr int WGN = tiled_waves_n<FMT, BM, BN>();
  constexpr int NW = 2 * WGN;              // waves per workgroup
  constexpr int NT = 64 * NW;              // threads
  constexpr int TM = BM / 2, TN = BN / WGN;  // wave tile
  constexpr int IM = TM / 16, IN = TN / 16;
  // MXFP4: E2M1 weights, 64 bytes a row per K block (1 KB packed tiles)
  constexpr bool MXS = FMT == FMT_MX || FMT == FMT_MX4;   // E8M0 block scales in the matrix instruction
  constexpr int WB = FMT == FMT_MX4 ? 64 : 128;          // weight bytes per row per K block
  constexpr int WT = 16 * WB;                            // bytes of one packed weight tile
  constexpr int STAGE = BM * 128 + BN * WB;  // bytes of one LDS stage
  constexpr int PA = BM * 8 / NT;          // 16-byte A pieces per thread per K block
  constexpr int PB = BN * (WB / 16) / NT;
  constexpr bool WP = WM == W_PACKED;
  static_assert(FMT != FMT_MX4 || (WP && AP && NS == 0), "MXFP4: packed operands, register ring");
  using Acc = typename TiledAcc<FMT>::T;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wy = wave / WGN, wx = wave % WGN;
  const int r16 = lane & 15, g = lane >> 4;

  const uint32_t M = (uint32_t)p.M, N = (uint32_t)p.N, K = (uint32_t)p.K;
  const uint32_t G = (uint32_t)p.G;
  const uint32_t NT16 = (N + 15u) / 16u;

  // ---- workgroup -> (tile, K chunk): XCD-contiguous runs, grouped raster
  const int total = (int)gridDim.x;
  const int bid = (int)blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = total >> 3, rem = total & 7;
  const int logical = xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
  const int chunk = logical % p.split;
  const int tile = logical / p.split;
  const int tiles_m = (p.M + BM - 1) / BM;
  const int tiles_n = p.tiles_n;
  constexpr int GM = 8;
  const int group = tile / (GM * tiles_n);
  const int first_m = group * GM;
  const int gm = min(GM, tiles_m - first_m);
  const int in_group = tile - group * GM * tiles_n;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;
  const uint32_t m0 = (uint32_t)tm * BM, n0 = (uint32_t)tn * BN;

  const int kb0 = chunk * p.chunk_kb;
  const int kb1 = min(p.G, kb0 + p.chunk_kb);
  const int nk = kb1 - kb0;

  const uint32_t MT16 = (M + 15u) / 16u;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.a, AP ? MT16 * G * 2048u : M * K);
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(p.w, WP ? NT16 * G * (uint32_t)WT : N * K);
  // MXFP8 scales: E8M0 bytes in lane order, 64 per (16-row group, K block)
  const __amdgpu_buffer_rsrc_t rsa =
      make_rsrc(p.sa, MXS ? MT16 * G * 64u : (FMT == FMT_BLOCK ? M * G : M) * 4u);
  const __amdgpu_buffer_rsrc_t rsw =
      make_rsrc(p.sw, MXS ? NT16 * G * 64u : (FMT == FMT_BLOCK ? ((N + 127u) / 128u) * G : N) * 4u);

  // ---- global -> registers for one K block (zeros outside the matrices)
  // a ring of PF register slots: K block b of the chunk lives in slot b % PF
  u32x4 pa[PF][PA], pb[PF][PB];
  auto load_block = [&](int kb, int sl) {
    const bool in = kb < kb1;   // blocks past the chunk read as zeros (no branch, no memory request)
    const uint32_t kofs = (uint32_t)kb * 128u;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const uint32_t q = (uint32_t)(i * NT + tid);
      if constexpr (AP) {
        const uint32_t t = m0 / 16u + (q >> 7);
        pa[sl][i] = bload16(ra, (in && t < MT16) ? (t * G + (uint32_t)kb) * 2048u + (q & 127u) * 16u : OOB);
      } else {
        const uint32_t m = m0 + (q >> 3), k = kofs + (q & 7u) * 16u;
        pa[sl][i] = bload16(ra, (in && m < M && k < K) ? m * K + k : OOB);
      }
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const uint32_t q = (uint32_t)(i * NT + tid);
      if constexpr (WP) {
        constexpr uint32_t QT = (uint32_t)WT / 16u;   // 16-byte pieces of a tile
        const uint32_t t = n0 / 16u + q / QT;
        pb[sl][i] = bload16(rw, (in && t < NT16) ? (t * G + (uint32_t)kb) * (uint32_t)WT + (q % QT) * 16u : OOB);
      } else {
        const uint32_t n = n0 + (q >> 3), k = kofs + (q & 7u) * 16u;
        pb[sl][i] = bload16(rw, (in && n < N && k < K) ? n * K + k : OOB);
      }
    }
  };
  // ---- registers -> one LDS stage, in operand order: row r, 16-byte chunk
  // c = 4h + g of a 16-row group lands at h*1024 + (r + 16g)*16 of its 2 KB tile
  auto store_block = [&](int buf, int sl) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int q = i * NT + tid;
      if constexpr (AP) {
        *reinterpret_cast<u32x4*>(base + q * 16) = pa[sl][i];
      } else {
        const int row = q >> 3, c = q & 7;
        *reinterpret_cast<u32x4*>(base + (row >> 4) * 2048 + (c >> 2) * 1024 + ((row & 15) + 16 * (c & 3)) * 16) =
            pa[sl][i];
      }
    }
    uint8_t* bbase = base + BM * 128;
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int q = i * NT + tid;
      if constexpr (WP) {
        *reinterpret_cast<u32x4*>(bbase + q * 16) = pb[sl][i];
      } else {
        const int row = q >> 3, c = q & 7;
        *reinterpret_cast<u32x4*>(bbase + (row >> 4) * 2048 + (c >> 2) * 1024 + ((row & 15) + 16 * (c & 3)) * 16) =
            pb[sl][i];
      }
    }
  };

  // ---- Block_FP8 scale factors of one K block for this lane's elements
  // (non-swapped: 4 token rows per 16x16 tile; swapped: 1 token per tile);
  // MXFP8: the E8M0 byte this lane hands the matrix core with each A and B
  // fragment (kept as raw bits in the float slots)
  constexpr int SA_N = FMT == FMT_BLOCK ? (SWAP ? IM : IM * 4) : MXS ? IM : 1;
  constexpr int SW_N = (FMT == FMT_BLOCK || MXS) ? IN : 1;
  float sa_nx[PF][SA_N], sw_nx[PF][SW_N];
  auto load_scales = [&](int kb, int sl) {
    if constexpr (FMT == FMT_BLOCK) {
#pragma unroll
      for (int i = 0; i < IM; ++i) {
#pragma unroll
        for (int r = 0; r < (SWAP ? 1 : 4); ++r) {
          const uint32_t m = m0 + (uint32_t)(wy * TM + 16 * i) + (SWAP ? (uint32_t)r16 : (uint32_t)(4 * g + r));
          sa_nx[sl][SWAP ? i : i * 4 + r] = bload_f32(rsa, (kb < kb1 && m < M) ? (m * G + (uint32_t)kb) * 4u : OOB);
        }
      }
#pragma unroll
      for (int j = 0; j < IN; ++j) {
        const uint32_t nb = n0 + (uint32_t)(wx * TN + 16 * j);
        sw_nx[sl][j] = bload_f32(rsw, (kb < kb1 && nb < N) ? ((nb >> 7) * G + (uint32_t)kb) * 4u : OOB);
      }
    } else if constexpr (MXS) {
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        const uint32_t t = m0 / 16u + (uint32_t)(wy * IM + i);
        sa_nx[sl][i] = __int_as_float(
            bload_u8(rsa, (kb < kb1 && t < MT16) ? (t * G + (uint32_t)kb) * 64u + (uint32_t)lane : OOB));
      }
#pragma unroll
      for (int j = 0; j < IN; ++j) {
        const uint32_t t = n0 / 16u + (uint32_t)(wx * IN + j);
        sw_nx[sl][j] = __int_as_float(
            bload_u8(rsw, (kb < kb1 && t < NT16) ? (t * G + (uint32_t)kb) * 64u + (uint32_t)lane : OOB));
      }
    } else {
      (void)kb;
      (void)sl;
    }
  };

  Acc acc[IM][IN];
#pragma unroll
  for (int i = 0; i < IM; ++i)
#pragma unroll
    for (int j = 0; j < IN; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  auto mma_tile = [&](const Frag& a, const Frag& b, int i, int j, const float (&sa_c)[SA_N],
                      const float (&sw_c)[SW_N]) {
    if constexpr (FMT == FMT_INT8) {
      if (SWAP) {
        acc[i][j] = mma_i8(b.lo, a.lo, acc[i][j]);
        acc[i][j] = mma_i8(b.hi, a.hi, acc[i][j]);
      } else {
        acc[i][j] = mma_i8(a.lo, b.lo, acc[i][j]);
        acc[i][j] = mma_i8(a.hi, b.hi, acc[i][j]);
      }
    } else if constexpr (FMT == FMT_FP8) {
      acc[i][j] = SWAP ? mma_f8(b, a, acc[i][j]) : mma_f8(a, b, acc[i][j]);
    } else if constexpr (FMT == FMT_MX) {
      const int xa = __float_as_int(sa_c[i]), xw = __float_as_int(sw_c[j]);
      acc[i][j] = SWAP ? mma_f8_mx(b, a, acc[i][j], xw, xa) : mma_f8_mx(a, b, acc[i][j], xa, xw);
    } else if constexpr (FMT == FMT_MX4) {
      const int xa = __float_as_int(sa_c[i]), xw = __float_as_int(sw_c[j]);
      acc[i][j] = mma_f8f4_mx<SWAP>(a, b.lo, acc[i][j], xa, xw);
    } else {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const f32x4 part = SWAP ? mma_f8(b, a, z) : mma_f8(a, b, z);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // (P_g * s_a) * s_w, as in the decode kernel
        const float t = __fmul_rn(part[r], sa_c[SWAP ? i : i * 4 + r]);
        acc[i][j][r] = __builtin_fmaf(t, sw_c[j], acc[i][j][r]);
      }
    }
  };
  // The operand with fewer fragments stays in registers for the whole K
  // block; the other streams through, one fragment feeding a row (or
  // column) of matrix-core instructions, so LDS reads overlap the math.
  auto compute = [&](int buf, const float (&sa_c)[SA_N], const float (&sw_c)[SW_N]) {
    const uint8_t* as = smem + buf * STAGE + (wy * IM) * 2048 + lane * 16;
    const uint8_t* bs = smem + buf * STAGE + BM * 128 + (wx * IN) * WT + lane * 16;
    // a B fragment: the two 16-byte pieces of a 2 KB tile, or MXFP4's one of a 1 KB tile
    auto bfrag = [&](int j) -> Frag {
      Frag f;
      f.lo = *reinterpret_cast<const u32x4*>(bs + j * WT);
      if constexpr (FMT == FMT_MX4)
        f.hi = u32x4{0u, 0u, 0u, 0u};
      else
        f.hi = *reinterpret_cast<const u32x4*>(bs + j * WT + 1024);
      return f;
    };
    if constexpr (IM > IN) {
      Frag bf[IN];
#pragma unroll
      for (int j = 0; j < IN; ++j) bf[j] = bfrag(j);
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        Frag af;
        af.lo = *reinterpret_cast<const u32x4*>(as + i * 2048);
        af.hi = *reinterpret_cast<const u32x4*>(as + i * 2048 + 1024);
#pragma unroll
        for (int j = 0; j < IN; ++j) mma_tile(af, bf[j], i, j, sa_c, sw_c);
      }
    } else {
      Frag af[IM];
#pragma unroll
      for (int i = 0; i < IM; ++i) {
        af[i].lo = *reinterpret_cast<const u32x4*>(as + i * 2048);
        af[i].hi = *reinterpret_cast<const u32x4*>(as + i * 2048 + 1024);
      }
#pragma unroll
      for (int j = 0; j < IN; ++j) {
        const Frag bf = bfrag(j);
#pragma unroll
        for (int i = 0; i < IM; ++i) mma_tile(af[i], bf, i, j, sa_c, sw_c);
      }
    }
  };

  // ---- main loop: LDS stage it&1 holds K block kb0+it while blocks
  // kb0+it+1 .. kb0+it+PF are in flight in the register ring (NS == 0), or
  // an NS-stage LDS ring filled by LDS-DMA (NS > 0)
  float sa_c[SA_N], sw_c[SW_N];
  auto take_scales = [&](int sl) {
#pragma unroll
    for (int i = 0; i < SA_N; ++i) sa_c[i] = sa_nx[sl][i];
#pragma unroll
    for (int j = 0; j < SW_N; ++j) sw_c[j] = sw_nx[sl][j];
  };
  // The loop runs a multiple of PF blocks with every load issued
  // unconditionally: blocks past the chunk are zeros and add nothing, and
  // the fixed instruction stream lets the compiler wait for exactly the
  // oldest ring slot instead of draining all loads in flight.
  if constexpr (NS > 0) {
    // ---- packed operands straight into an NS-stage LDS ring with LDS-DMA
    // buffer loads (no staging registers).  A stage is the A tile's BM/16
    // and the B tile's BN/16 2 KB tiles, each copied as two 1 KB wave loads;
    // every wave issues DW of them per stage (wave w takes the halves
    // w, w + NW, w + 2NW, ...), so "stage it has landed" is
    // "at most (NS-2)*DW of this wave's loads outstanding" followed by a
    // barrier.  The refill of stage it-1's buffer goes out right after that
    // barrier, before the matrix cores start on stage it.
    static_assert(WP && AP && FMT != FMT_BLOCK, "the LDS-DMA ring reads packed operands");
    constexpr int TA = BM / 16, TB = BN / 16;
    constexpr int DA = 2 * TA / NW, DB = 2 * TB / NW;
    static_assert(DA * NW == 2 * TA && DB * NW == 2 * TB, "whole 1 KB halves per wave");
    constexpr int DW = DA + DB;
    constexpr int ALLOW = (NS - 2) * DW;
    static_assert(ALLOW <= 63, "vmcnt holds 6 bits");
    // wave w copies 1 KB halves j = w + NW*i: tile j/2 = w/2 + (NW/2)*i, half w%2
    const uint32_t a_lane = (m0 / 16u + (uint32_t)(wave >> 1)) * G * 2048u + (uint32_t)(wave & 1) * 1024u +
                            (uint32_t)lane * 16u;
    const uint32_t b_lane = (n0 / 16u + (uint32_t)(wave >> 1)) * G * 2048u + (uint32_t)(wave & 1) * 1024u +
                            (uint32_t)lane * 16u;
    const int lds_wave = (wave >> 1) * 2048 + (wave & 1) * 1024;
    auto dma_stage = [&](int kb, int buf) {
      const bool in = kb < kb1;
      uint8_t* base = smem + buf * STAGE + lds_wave;
      const uint32_t kofs = (uint32_t)kb * 2048u;
#pragma unroll
      for (int i = 0; i < DA; ++i) {
        const uint32_t t = m0 / 16u + (uint32_t)(wave >> 1) + (uint32_t)(NW / 2) * (uint32_t)i;
        const uint32_t off = (in && t < MT16) ? a_lane + (uint32_t)i * (uint32_t)(NW / 2) * G * 2048u + kofs : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (__attribute__((address_space(3))) void*)(base + i * NW * 1024),
                                                 16, off, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < DB; ++i) {
        const uint32_t t = n0 / 16u + (uint32_t)(wave >> 1) + (uint32_t)(NW / 2) * (uint32_t)i;
        const uint32_t off = (in && t < NT16) ? b_lane + (uint32_t)i * (uint32_t)(NW / 2) * G * 2048u + kofs : OOB;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rw, (__attribute__((address_space(3))) void*)(base + BM * 128 + i * NW * 1024), 16, off, 0, 0, 0);
      }
    };
    if (nk > 0) {
      float sa_c[SA_N], sw_c[SW_N];
#pragma unroll
      for (int i = 0; i < SA_N; ++i) sa_c[i] = 0.f;
#pragma unroll
      for (int j = 0; j < SW_N; ++j) sw_c[j] = 0.f;
#pragma unroll
      for (int st = 0; st < NS - 1; ++st) dma_stage(kb0 + st, st);
      // unrolled by NS so every stage index is a constant; the loop runs a
      // multiple of NS blocks, those past the chunk being zeros
      for (int it0 = 0; it0 < nk; it0 += NS) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
          __builtin_amdgcn_s_waitcnt((ALLOW & 15) | (7 << 4) | (15 << 8) | ((ALLOW >> 4) << 14));
          lds_barrier();
          dma_stage(kb0 + it0 + q + NS - 1, (q + NS - 1) % NS);
          compute(q, sa_c, sw_c);
        }
      }
    }
  } else if (nk > 0) {
    const int nloop = (nk + PF - 1) / PF * PF;
    load_block(kb0, 0);
    load_scales(kb0, 0);
    store_block(0, 0);
    take_scales(0);
#pragma unroll
    for (int q = 1; q <= PF; ++q) {
      load_block(kb0 + q, q % PF);
      load_scales(kb0 + q, q % PF);
    }
    lds_barrier();   // the ring's loads stay in flight
    for (int it0 = 0; it0 < nloop; it0 += PF) {
#pragma unroll
      for (int q = 0; q < PF; ++q) {
        const int it = it0 + q;
        compute(it & 1, sa_c, sw_c);
        const int sl = (q + 1) % PF;   // holds block it+1 (it0 is a multiple of PF)
        store_block((it + 1) & 1, sl);
        take_scales(sl);
        load_block(kb0 + it + 1 + PF, sl);
        load_scales(kb0 + it + 1 + PF, sl);
        lds_barrier();
      }
    }
  }

  // element (i, j, r) of this lane -> (token m, output column n)
  auto elem_m = [&](int i, int r) -> uint32_t {
    return m0 + (uint32_t)(wy * TM + 16 * i) + (SWAP ? (uint32_t)r16 : (uint32_t)(4 * g + r));
  };
  auto elem_n = [&](int j, int r) -> uint32_t {
    return n0 + (uint32_t)(wx * TN + 16 * j) + (SWAP ? (uint32_t)(4 * g + r) : (uint32_t)r16);
  };

  // ---- split-K: partial sums meet in the workspace (see the decode kernel)
  if (p.split > 1) {
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int j = 0; j < IN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t m = elem_m(i, r), n = elem_n(j, r);
          if (m < M && n < N) {
            if constexpr (FMT == FMT_INT8)
              __hip_atomic_fetch_add(reinterpret_cast<int*>(p.ws) + (size_t)m * N + n, acc[i][j][r],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
              __hip_atomic_fetch_add(reinterpret_cast<float*>(p.ws) + (size_t)m * N + n, acc[i][j][r],
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned prev =
          __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = (prev == (unsigned)(p.split - 1));
    }
    __syncthreads();
    if (!s_last) return;
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int j = 0; j < IN; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t m = elem_m(i, r), n = elem_n(j, r);
          if (m < M && n < N) {
            int* slot = reinterpret_cast<int*>(p.ws) + (size_t)m * N + n;
            const int v = __hip_atomic_exchange(slot, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if constexpr (FMT == FMT_INT8)
              acc[i][j][r] = v;
            else
              acc[i][j][r] = __int_as_float(v);
          }
        }
    if (tid == 0) __hip_atomic_exchange(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue.  The per-token formats need one s_a per token row and one
  // s_w per output column this lane holds: IM x (1 or 4) and IN x (4 or 1)
  // values, loaded once (not per element, which would keep hundreds of
  // loads in flight next to the accumulators).
  constexpr bool SCALED_IN_K = FMT == FMT_BLOCK || MXS;   // no scale epilogue
  constexpr int EA = SCALED_IN_K ? 1 : (SWAP ? 1 : 4), EW = SCALED_IN_K ? 1 : (SWAP ? 4 : 1);
  float ea[IM][EA], ew[IN][EW];
  if constexpr (!SCALED_IN_K) {
#pragma unroll
    for (int i = 0; i < IM; ++i)
#pragma unroll
      for (int r = 0; r < EA; ++r) {
        const uint32_t m = elem_m(i, r);
        ea[i][r] = bload_f32(rsa, m < M ? m * 4u : OOB);
      }
#pragma unroll
    for (int j = 0; j < IN; ++j)
#pragma unroll
      for (int r = 0; r < EW; ++r) {
        const uint32_t n = elem_n(j, r);
        ew[j][r] = bload_f32(rsw, n < N ? n * 4u : OOB);
      }
  }
  const bool vec4 = SWAP && (N & 3u) == 0;
#pragma unroll
  for (int i = 0; i < IM; ++i) {
#pragma unroll
    for (int j = 0; j < IN; ++j) {
      uint32_t out[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t m = elem_m(i, r), n = elem_n(j, r);
        const bool ok = m < M && n < N;
        if constexpr (SCALED_IN_K) {
          out[r] = bf16_rne(acc[i][j][r]);
          if (ok && p.acc_out) reinterpret_cast<float*>(p.acc_out)[(size_t)m * N + n] = acc[i][j][r];
        } else {
          const float sa = ea[i][EA == 4 ? r : 0];
          const float sw = ew[j][EW == 4 ? r : 0];
          float accf;
          if constexpr (FMT == FMT_INT8)
            accf = __int2float_rn(acc[i][j][r]);
          else
            accf = acc[i][j][r];
          float t = __fmul_rn(accf, sa);
          t = __fmul_rn(t, sw);
          out[r] = bf16_rne(t);
          if (ok && p.acc_out) {
            if constexpr (FMT == FMT_INT8)
              reinterpret_cast<int*>(p.acc_out)[(size_t)m * N + n] = acc[i][j][r];
            else
              reinterpret_cast<float*>(p.acc_out)[(size_t)m * N + n] = acc[i][j][r];
          }
        }
      }
      const uint32_t mm0 = elem_m(i, 0), nn0 = elem_n(j, 0);
      if (vec4 && mm0 < M && nn0 + 3 < N) {
        u32x2 v = {out[0] | (out[1] << 16), out[2] | (out[3] << 16)};
        *reinterpret_cast<u32x2*>(p.y + (size_t)mm0 * N + nn0) = v;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t m = elem_m(i, r), n = elem_n(j, r);
          if (m < M && n < N) p.y[(size_t)m * N + n] = (uint16_t)out[r];
        }
      }
      // one 16x16 tile at a time: keeps the scheduler from reading many
      // accumulator tiles out of the matrix-core registers at once
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Tile shapes instantiated per format: a wave holds (BM/32) x (BN/64) 16x16
// accumulator tiles (8 waves) or (BM/32) x (BN/32) (4 waves), at most 128
// registers; the 256 x 256 tile holds 8 x 4 and exists for the LDS-DMA ring
// of 2 stages only.
// Block_FP8 in the standard orientation also keeps four token scales per
// accumulator tile row live, so its largest tiles are left out as well.
template <int FMT, int SW, int BM, int BN, int PF, int NS>
constexpr bool tiled_config_fits() {
  // the LDS-DMA ring has no per-block scale path: Block_FP8 and MXFP8 use the register ring
  constexpr bool MXS = FMT == FMT_MX || FMT == FMT_MX4;
  if (BM * BN == 256 * 256) return NS == 2 && FMT != FMT_BLOCK && !MXS;
  if (NS > 0) return FMT != FMT_BLOCK && !MXS && NS * (BM + BN) * 128 <= 160 * 1024 && BM * BN <= 128 * 256;
  if (FMT == FMT_BLOCK && !SW && BM * BN > 128 * 128) return false;
  // MXFP8's scale bytes ride in the ring too: a two-block ring on the largest
  // register-ring tiles spills (checked against the compiler's resource report)
  if (MXS && BM * BN >= 128 * 256 && PF > 1) return false;
  if (PF * (BM + BN) > 768) return false;  // ring of PF K blocks: at most 96 VGPRs a lane
  if (FMT == FMT_BLOCK && BM * BN > 128 * 128 && PF > 1) return false;
  return BM * BN <= 128 * 256;
}

template <int FMT, int SW, int BM, int BN, int WM_, int PF, int AP, int NS>
hipError_t tiled_try(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a, bool probe_only,
                     bool* hit) {
  // MXFP4: packed E2M1 weights and packed activations only
  if constexpr (tiled_config_fits<FMT, SW, BM, BN, PF, NS>() && (FMT != FMT_MX4 || (WM_ == W_PACKED && AP == 1))) {
    if (k.swap == SW && k.bm == BM && k.bn == BN && k.wm == WM_ && k.pf == PF && k.ap == AP && k.ns == NS) {
      *hit = true;
      auto fn = qgemm_tiled_kernel<FMT, SW != 0, BM, BN, WM_, PF, AP != 0, NS>;
      if (probe_only) {
        // stages above the default 64 KB need the per-kernel opt-in (gfx950: 160 KB per workgroup)
        return hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)lds);
      }
      fn<<<grid, dim3(64 * 2 * tiled_waves_n<FMT, BM, BN>()), lds, s>>>(a);
      return hipGetLastError();
    }
  }
  return hipSuccess;
}

template <int FMT>
hipError_t tiled_dispatch(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                          bool probe_only) {
  bool hit = false;
  hipError_t e = hipSuccess;
#define QL_TT(SW, BM, BN, WM_, PF, AP)                                                  \
  e = tiled_try<FMT, SW, BM, BN, WM_, PF, AP, 0>(k, grid, lds, s, a, probe_only, &hit); \
  if (hit) return e;
  // packed operands through the LDS-DMA ring of NS stages (prefetch field = 1)
#define QL_TD(SW, BM, BN, NS)                                                          \
  e = tiled_try<FMT, SW, BM, BN, 2, 1, 1, NS>(k, grid, lds, s, a, probe_only, &hit);   \
  if (hit) return e;
#define QL_TD_S(BM, BN, NS) QL_TD(0, BM, BN, NS) QL_TD(1, BM, BN, NS)
#define QL_TT_P(SW, BM, BN, WM_, AP) \
  QL_TT(SW, BM, BN, WM_, 1, AP) QL_TT(SW, BM, BN, WM_, 2, AP) QL_TT(SW, BM, BN, WM_, 4, AP)
  // (row-major W, row-major A), (packed W, row-major A), (packed W, packed A)
#define QL_TT_W(SW, BM, BN) QL_TT_P(SW, BM, BN, 0, 0) QL_TT_P(SW, BM, BN, 2, 0) QL_TT_P(SW, BM, BN, 2, 1)
#define QL_TT_S(BM, BN) QL_TT_W(0, BM, BN) QL_TT_W(1, BM, BN)
  QL_TT_S(64, 128)
  QL_TT_S(64, 256)
  QL_TT_S(128, 128)
  QL_TT_S(128, 256)
  QL_TT_S(256, 128)
  QL_TD_S(128, 128, 2)
  QL_TD_S(128, 128, 3)
  QL_TD_S(128, 256, 2)
  QL_TD_S(128, 256, 3)
  QL_TD_S(256, 128, 2)
  QL_TD_S(256, 128, 3)
  QL_TD_S(256, 256, 2)
#undef QL_TD_S
#undef QL_TD
#undef QL_TT_S
#undef QL_TT_W
#undef QL_TT_P
#undef QL_TT
  return hipErrorInvalidDeviceFunction;
}

}  // namespace qlk
