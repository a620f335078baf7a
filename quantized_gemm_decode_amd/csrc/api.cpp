// C ABI of the quantized linear: argument validation, planning (sweep table,
// heuristic, explicit configs), launches and hipGraph capture helpers.
//
// Planning follows the pages' split between an offline per-shape search and
// a cheap runtime lookup ([Summary] "Hybrid dispatch addresses runtime
// overhead": token counts 1, 2, 4, 8, 16, 24, 32 tuned per GEMM shape, graph
// replay for num_tokens <= 32).  Plans are host objects; nothing here
// allocates device memory or synchronises.
//
// [Summary] = English summary of "Building a High-Performance and Portable
// vLLM Linear Backend with Helion" (yuxiaoba.github.io).
#include "../../include/qlinear.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <mutex>
#include <sstream>
#include <string>
#include <vector>

#include "decode_args.hpp"

namespace {

thread_local std::string g_err;

ql_status fail(ql_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ql_status hip_fail(hipError_t e, const char* what) {
  return fail(QL_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

// gfx950: LDS per workgroup (above 64 KB with the per-kernel opt-in), less
// room for the kernels' own static LDS variables
constexpr int64_t kLdsLimit = 160 * 1024 - 256;
// Fused quantization holds the workgroup's share of X in registers: 16384 bf16 values.
constexpr int64_t kFusedMaxValues = 16384;
constexpr int kBuckets[] = {1, 2, 4, 8, 16, 24, 32};

bool valid_fmt(int32_t f) { return f >= QL_FP8_DYNAMIC && f <= QL_MXFP4; }
bool is_mx(int32_t f) { return f == QL_MXFP8 || f == QL_MXFP4; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int kernel_fmt(int32_t f) {
  return f == QL_W8A8_INT8 ? qlk::FMT_INT8 : f == QL_BLOCK_FP8 ? qlk::FMT_BLOCK : f == QL_MXFP8 ? qlk::FMT_MX
       : f == QL_MXFP4 ? qlk::FMT_MX4 : qlk::FMT_FP8;
}

ql_status check_sizes(int32_t fmt, int64_t R, int64_t K, const char* rname) {
  if (!valid_fmt(fmt)) return fail(QL_E_INVALID, "unknown format %d", fmt);
  if (R < 0 || K < 0) return fail(QL_E_INVALID, "negative size (%s=%lld, K=%lld)", rname, (long long)R, (long long)K);
  if (K % 16) return fail(QL_E_INVALID, "K=%lld is not a multiple of 16", (long long)K);
  if (fmt == QL_BLOCK_FP8 && K % 128) return fail(QL_E_INVALID, "Block_FP8 needs K %% 128 == 0 (K=%lld)", (long long)K);
  if (is_mx(fmt) && K % 128) return fail(QL_E_INVALID, "MXFP8 / MXFP4 need K %% 128 == 0 (K=%lld)", (long long)K);
  if (R * K > (int64_t(1) << 30)) return fail(QL_E_UNSUPPORTED, "%s*K=%lld exceeds 2^30", rname, (long long)(R * K));
  return QL_OK;
}

// ------------------------------------------------------------------ table

struct TableEntry {
  int32_t fmt;
  int64_t M, N, K;
  ql_config cfg;
  double us;
  int us_class;  // 2: a forward-only entry (its time covers quantize + GEMM); 3: a SiLU-and-mul forward
                 // entry (qlinear_plan_glu); 4: a forward entry for inputs whose per-token amax is
                 // given (qlinear_forward_amax); else act_class(a_mode)
};

std::mutex g_table_mu;
std::vector<TableEntry> g_table;

int64_t bucket_of(int64_t M) {
  for (int b : kBuckets)
    if (M <= b) return b;
  return M;
}

// Activation class of a configuration: 0 row-major A_q (a_mode 0, 1), 1 packed
// A_q (2, 3), 2 forward-only plans (fused quantization, 4), 4 forward plans
// of an input whose per-token amax is given (5).  A class-2 table entry is
// the best plan for quantize + GEMM, fused or not; a class-4 entry the best
// for the same with the amax given (a_mode 5, or a packed-A plan).
int act_class(int32_t a_mode) { return a_mode == 5 ? 4 : a_mode == 4 ? 2 : (a_mode >= 2 ? 1 : 0); }

bool table_lookup(int32_t fmt, int32_t layout, int a_class, int64_t M, int64_t N, int64_t K, ql_config* out) {
  std::lock_guard<std::mutex> lk(g_table_mu);
  const int64_t want = bucket_of(M);
  const TableEntry* best = nullptr;
  const TableEntry* largest = nullptr;
  for (const TableEntry& e : g_table) {
    if (e.fmt != fmt || e.N != N || e.K != K || e.cfg.w_layout != layout) continue;
    if (a_class >= 2 ? e.us_class != a_class : (e.us_class >= 2 || act_class(e.cfg.a_mode) != a_class)) continue;
    if (e.M >= want && (!best || e.M < best->M)) best = &e;
    if (!largest || e.M > largest->M) largest = &e;
  }
  if (!best && M > 32) best = largest;  // beyond every tuned M: the largest tuned one
  if (!best) return false;
  if ((M <= 32) != (best->M <= 32)) return false;  // never mix the decode and tiled regimes
  *out = best->cfg;
  return true;
}

}  // namespace

// ------------------------------------------------------------------ plan object

struct ql_plan_s {
  int32_t fmt;
  int64_t M, N, K;
  ql_config cfg;
  int32_t source;
  // derived
  int G, chunk_kb, chunks, mt, n_tiles, bn, tiles_n;
  int64_t lds, ws_bytes, ws_acc_bytes;
  bool tiled;
  bool glu;  // merged gate/up weight, SiLU-and-mul epilogue, output [M, N/2]
  qlk::DecodeKey key;
  qlk::TiledKey tkey;
};

struct ql_graph_s {
  hipGraph_t graph;
  hipGraphExec_t exec;
};

namespace {

// The last-resort tiled plan (M > 32): tile rows follow M, 128 weight rows
// per tile; split K only while the tiles alone cannot give every CU two
// workgroups.
ql_config heuristic_tiled(int32_t layout, bool a_packed, int64_t M, int64_t N, int64_t K) {
  ql_config c{};
  c.algo = QL_ALGO_TILED;
  c.w_layout = layout;
  c.a_mode = a_packed ? 2 : 0;
  c.swap_ab = 1;
  c.waves_n = 4;
  c.waves_k = 1;
  c.rows_per_wave = 16;
  c.prefetch = 2;
  c.tile_m = M <= 64 ? 64 : (M <= 128 ? 128 : 256);
  c.tile_n = 128;
  c.prefetch = c.tile_m == 64 ? 4 : (c.tile_m == 128 ? 2 : 1);
  const int64_t G = (K + 127) / 128;
  const int64_t tiles = ((M + c.tile_m - 1) / c.tile_m) * ((N + c.tile_n - 1) / c.tile_n);
  int64_t split = 1;
  while (tiles * split < 256 && split * 2 <= 256 && G / (split * 2) >= 8) split *= 2;
  c.split_k = (int32_t)split;
  return c;
}

// The last-resort decode plan: 4 waves side by side on N, split-K up to about
// 1024 workgroups (instantiated for every format and operand layout).
ql_config heuristic_config(int32_t fmt, int32_t layout, bool a_packed, int64_t M, int64_t N, int64_t K) {
  // the MX formats' decode kernel serves up to 64 tokens
  if (M > 32 && !(is_mx(fmt) && M <= 64)) return heuristic_tiled(layout, a_packed, M, N, K);
  ql_config c{};
  c.w_layout = layout;
  c.algo = QL_ALGO_DECODE;
  c.swap_ab = 1;
  c.waves_n = 4;
  c.waves_k = 1;
  c.rows_per_wave = 16;
  c.prefetch = 2;
  const int64_t G = (K + 127) / 128;
  const int64_t bn = 64;
  const int64_t tiles = (N + bn - 1) / bn;
  int64_t split = 1;
  while (tiles * split < 1024 && split * 2 <= 256 && (G + split * 2 - 1) / (split * 2) >= 2) split *= 2;
  c.split_k = (int32_t)split;
  const int64_t chunk_kb = (G + split - 1) / split;
  const int64_t mt = M <= 16 ? 1 : 2;
  c.a_mode = a_packed ? 2 : (chunk_kb * mt * 2048 <= kLdsLimit ? 1 : 0);
  c.w_lds = 0;
  (void)fmt;
  return c;
}

// Tiled plans without a table entry, in order of preference.  Over the
// probed shapes the fastest tile is the largest of 256 x 256 (2-stage LDS-DMA
// ring), 128 x 256, 128 x 128 and 64 x 128 that still gives about 200 tiles
// or more; below that the 64 x 128 tile, with split-K 4 when there are at
// most 64 tiles and split 2 at most 128 tiles over a K of 64 or more blocks.
// Block_FP8 applies its scales inside the K loop and keeps more registers
// live: it runs best with 1-block batches on 128 x 128 (Swap-AB) from about
// 400 such tiles, else on 64 x 128 (1-block batches from 400 tiles, 2 below,
// split-K 4 up to 64 tiles and 2 up to 128, or 4 over a K of 64 or more
// blocks).  Tiles a format or operand layout does not instantiate (the ring
// needs packed operands; MXFP8 runs neither the ring nor 256 x 256) are
// skipped by the caller, down to heuristic_tiled's plan.
std::vector<ql_config> tiled_candidates(int32_t fmt, int32_t layout, bool a_packed, int64_t M, int64_t N,
                                        int64_t K) {
  struct Tile {
    int bm, bn, pf, ring;
  };
  static const Tile kTiles[] = {{256, 256, 2, 1}, {128, 256, 1, 0}, {128, 128, 2, 0}, {64, 128, 2, 0}};
  const int64_t G = (K + 127) / 128;
  std::vector<ql_config> out;
  auto make = [&](int bm, int bn, int pf, int ring, int swap, int64_t split) {
    ql_config c{};
    c.algo = QL_ALGO_TILED;
    c.w_layout = layout;
    c.a_mode = a_packed ? 2 : 0;
    c.swap_ab = swap;
    c.waves_n = 4;
    c.waves_k = 1;
    c.rows_per_wave = 16;
    c.tile_m = bm;
    c.tile_n = bn;
    c.prefetch = pf;
    c.w_lds = ring;
    while (split > 1 && G / split < 4) split /= 2;
    c.split_k = (int32_t)split;
    return c;
  };
  auto count = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
  if (fmt == QL_BLOCK_FP8) {
    const int64_t t64 = count(64, 128);
    const int64_t split = t64 <= 64 ? 4 : (t64 <= 128 ? (G >= 64 ? 4 : 2) : 1);
    const ql_config small = make(64, 128, t64 >= 400 ? 1 : 2, 0, 0, split);
    if (M >= 64 && count(128, 128) >= 400) out.push_back(make(128, 128, 1, 0, 1, 1));
    out.push_back(small);
    out.push_back(heuristic_tiled(layout, a_packed, M, N, K));
    return out;
  }
  bool chosen = false;
  for (const Tile& t : kTiles) {
    if (t.bm > 64 && t.bm > 2 * M) continue;   // mostly padding rows
    const int64_t tiles = ((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const bool last = t.bm == 64;
    if (!chosen && tiles < 200 && !last) continue;
    int64_t split = 1;
    if (t.bm == 64 && tiles <= 64) split = 4;
    else if (t.bm == 64 && tiles <= 128 && G >= 64) split = 2;
    out.push_back(make(t.bm, t.bn, t.pf, t.ring, 0, split));
    chosen = true;
  }
  out.push_back(heuristic_tiled(layout, a_packed, M, N, K));
  return out;
}

// Plans without a table entry, in order of preference (the caller takes the
// first one that is instantiated).  Over the tabulated shapes the sweep
// settles on one K range per workgroup (split 1), shared by the workgroup's
// waves, and on a wave shape that follows the number of 16-row groups: one
// group per 4-wave workgroup up to 256 groups (about one workgroup per
// compute unit), 2 x 2 waves up to 1024 (4 x 1 with Swap-AB beyond 512
// groups at M > 8), and 32 rows a wave beyond 1024 or when K spans 96 or
// more 128-wide blocks (for the MX formats only at M > 16).  Split-K adds
// three memory round trips (partial sums, arrival counter, read-back) to the
// launch, so it is used only when a few row groups stream a long K.  A
// forward plan at M <= 2 tries the quantizer fused into the GEMM first.  The
// last candidate is heuristic_config's, which every format instantiates.
std::vector<ql_config> heuristic_candidates(int32_t fmt, int32_t layout, int a_class, int64_t M, int64_t N,
                                            int64_t K) {
  std::vector<ql_config> out;
  const int64_t groups = (N + 15) / 16;
  if (M > 32 && !(is_mx(fmt) && M <= 64)) {
    // Up to 64 tokens the weight-streaming kernel with four token tiles beats
    // the tiled one while the weights are few enough rows (measured 0.71-0.95x
    // the tiled plan up to 448 row groups, even at 896, 1.4x at 1792);
    // Block_FP8 has no four-token-tile instantiation.
    std::vector<ql_config> out;
    if (M <= 64 && fmt != QL_BLOCK_FP8 && layout == 1 && groups <= 512) {
      ql_config d{};
      d.algo = QL_ALGO_DECODE;
      d.w_layout = 1;
      d.a_mode = a_class != 0 ? 2 : 0;
      d.swap_ab = 1;
      d.split_k = 1;
      d.rows_per_wave = 16;
      d.prefetch = 2;
      d.waves_n = groups <= 256 ? 1 : 2;
      d.waves_k = groups <= 256 ? 4 : 2;
      out.push_back(d);
    }
    for (const ql_config& c : tiled_candidates(fmt, layout, a_class != 0, M, N, K)) out.push_back(c);
    return out;
  }
  const int64_t G = (K + 127) / 128;
  ql_config b{};
  b.algo = QL_ALGO_DECODE;
  b.w_layout = layout;
  b.w_lds = layout == 0 ? 1 : 0;
  b.a_mode = a_class != 0 ? 2 : 0;
  int64_t split = 1;
  while (groups * split < 128 && split * 2 <= 256 && G / (split * 2) >= 64) split *= 2;
  b.split_k = (int32_t)split;
  b.rows_per_wave = 16;
  b.prefetch = 2;
  int first_swap = 0;
  if (groups <= 256) {
    b.waves_n = 1;
    b.waves_k = 4;
  } else if (groups > 1024 || (G >= 96 && (!is_mx(fmt) || M > 16))) {
    // many row groups, or a long K: 32 rows a wave halve the activation reads per weight byte
    // (MX formats, whose scale loads add to the per-block work, gain only from two token tiles)
    b.waves_n = 1;
    b.waves_k = 4;
    b.rows_per_wave = 32;
    b.prefetch = layout == 1 ? 1 : 2;   // row-major weights run 2- and 4-block batches only
  } else if (groups <= 512 || M <= 8) {
    b.waves_n = 2;
    b.waves_k = 2;
  } else {
    // 512..1024 groups and two token tiles' worth of activations: four waves on one K range
    b.waves_n = 4;
    b.waves_k = 1;
    first_swap = 1;
  }
  if (a_class == 4 && M <= 16 && K % 128 == 0 && layout == 1 && (fmt == QL_FP8_DYNAMIC || fmt == QL_W8A8_INT8)) {
    // the given amax lets a workgroup quantize just its K chunk: split so that
    // M x chunk stays within the 16384 values a workgroup holds
    ql_config f = b;
    int64_t sp = 1;
    while (M * ((G + sp - 1) / sp) * 128 > kFusedMaxValues && sp < 256) sp *= 2;
    f.a_mode = 5;
    f.split_k = (int32_t)sp;
    f.waves_n = 1;
    f.waves_k = groups <= 256 ? 16 : 4;
    f.rows_per_wave = 16;
    f.prefetch = 1;
    out.push_back(f);
  }
  if (a_class == 2 && M <= 2) {
    ql_config f = b;
    f.a_mode = 4;
    f.split_k = 1;
    f.waves_n = 1;
    f.waves_k = groups <= 256 ? 16 : 4;
    f.rows_per_wave = 16;
    f.prefetch = 1;
    out.push_back(f);
  }
  for (int i = 0; i < 2; ++i) {
    ql_config c = b;
    c.swap_ab = i ^ first_swap;
    out.push_back(c);
  }
  out.push_back(heuristic_config(fmt, layout, a_class != 0, M, N, K));
  return out;
}

constexpr int64_t kTiledLdsLimit = 160 * 1024 - 256;  // as kLdsLimit

ql_status build_tiled_plan(int32_t fmt, int64_t M, int64_t N, int64_t K, const ql_config& cfg, int32_t source,
                           ql_plan* out) {
  if (cfg.swap_ab != 0 && cfg.swap_ab != 1) return fail(QL_E_INVALID, "swap_ab must be 0 or 1");
  if (!is_pow2(cfg.split_k) || cfg.split_k > 256) return fail(QL_E_INVALID, "split_k must be a power of two in [1, 256]");
  if (cfg.tile_m != 64 && cfg.tile_m != 128 && cfg.tile_m != 256) return fail(QL_E_INVALID, "tile_m must be 64, 128 or 256");
  if (cfg.tile_n != 128 && cfg.tile_n != 256) return fail(QL_E_INVALID, "tile_n must be 128 or 256");
  if (cfg.w_lds != 0 && cfg.w_lds != 1) return fail(QL_E_INVALID, "w_lds must be 0 or 1");
  if (cfg.w_lds && (cfg.a_mode != 2 || cfg.w_layout != 1 || (cfg.prefetch != 2 && cfg.prefetch != 3)))
    return fail(QL_E_INVALID, "the LDS-DMA ring (w_lds=1) needs packed operands and prefetch = 2 or 3 stages");
  if (cfg.w_layout != 0 && cfg.w_layout != 1) return fail(QL_E_INVALID, "w_layout must be 0 or 1");
  if (!cfg.w_lds && cfg.prefetch != 1 && cfg.prefetch != 2 && cfg.prefetch != 4)
    return fail(QL_E_INVALID, "prefetch must be 1, 2 or 4");
  if (cfg.a_mode != 0 && cfg.a_mode != 2) return fail(QL_E_INVALID, "a_mode must be 0 or 2 for the tiled algorithm");
  if (cfg.a_mode == 2 && qlinear_packed_act_bytes(M, K) > (int64_t(1) << 30))
    return fail(QL_E_UNSUPPORTED, "packed activations exceed 2^30 bytes");
  ql_plan_s* p = new ql_plan_s();
  p->fmt = fmt;
  p->M = M;
  p->N = N;
  p->K = K;
  p->cfg = cfg;
  p->source = source;
  p->tiled = true;
  p->G = (int)((K + 127) / 128);
  const int split = std::max(1, std::min<int>(cfg.split_k, std::max(1, p->G)));
  p->chunk_kb = p->G > 0 ? (p->G + split - 1) / split : 0;
  p->chunks = p->G > 0 ? (p->G + p->chunk_kb - 1) / p->chunk_kb : 1;
  p->mt = 0;
  p->bn = cfg.tile_n;
  p->tiles_n = (int)((N + cfg.tile_n - 1) / cfg.tile_n);
  p->n_tiles = (int)((M + cfg.tile_m - 1) / cfg.tile_m) * p->tiles_n;
  // a stage: the A tile's tile_m rows and the B tile's tile_n rows of one K block (MXFP4: 64 bytes a row)
  p->lds = (cfg.w_lds ? cfg.prefetch : 2) * ((int64_t)cfg.tile_m * 128 + (int64_t)cfg.tile_n * (fmt == QL_MXFP4 ? 64 : 128));
  if (p->lds > kTiledLdsLimit) {
    delete p;
    return fail(QL_E_UNSUPPORTED, "tile needs more LDS than a workgroup has");
  }
  p->ws_acc_bytes = p->chunks > 1 ? ((M * N * 4 + 255) / 256) * 256 : 0;
  p->ws_bytes = p->chunks > 1 ? p->ws_acc_bytes + (int64_t)p->n_tiles * 4 : 0;
  p->key = qlk::DecodeKey{kernel_fmt(fmt), cfg.swap_ab, 0, 0, 4, 0, 0, 0};
  p->tkey = qlk::TiledKey{kernel_fmt(fmt), cfg.swap_ab, cfg.tile_m, cfg.tile_n,
                          cfg.w_layout ? qlk::W_PACKED : qlk::W_DIRECT, cfg.w_lds ? 1 : cfg.prefetch,
                          cfg.a_mode == 2 ? 1 : 0, cfg.w_lds ? cfg.prefetch : 0};
  qlk::DecodeArgs dummy{};
  hipError_t pe;
  switch (p->tkey.fmt) {
    case qlk::FMT_INT8: pe = qlk::tiled_dispatch_int8(p->tkey, dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    case qlk::FMT_MX: pe = qlk::tiled_dispatch_mx(p->tkey, dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    case qlk::FMT_MX4: pe = qlk::tiled_dispatch_mx4(p->tkey, dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    case qlk::FMT_BLOCK: pe = qlk::tiled_dispatch_block(p->tkey, dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    default: pe = qlk::tiled_dispatch_fp8(p->tkey, dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
  }
  if (pe == hipErrorInvalidDeviceFunction) {
    delete p;
    return fail(QL_E_UNSUPPORTED, "no tiled kernel instantiated for tile %dx%d", cfg.tile_m, cfg.tile_n);
  }
  // any other error: raising the LDS limit needs a GPU; the launch reports it if it matters
  *out = p;
  return QL_OK;
}

ql_status build_plan(int32_t fmt, int64_t M, int64_t N, int64_t K, const ql_config& cfg, int32_t source,
                     ql_plan* out, bool glu = false) {
  if (!out) return fail(QL_E_INVALID, "out_plan is NULL");
  *out = nullptr;
  ql_status st = check_sizes(fmt, M, K, "M");
  if (st != QL_OK) return st;
  if ((st = check_sizes(fmt, N, K, "N")) != QL_OK) return st;
  if (M * N >= (int64_t(1) << 31)) return fail(QL_E_UNSUPPORTED, "M*N exceeds 2^31");
  if (cfg.w_layout == 1 && qlinear_packed_weight_bytes(N, K) > (int64_t(1) << 30))
    return fail(QL_E_UNSUPPORTED, "packed weights exceed 2^30 bytes");
  if (glu) {
    if (cfg.algo != QL_ALGO_DECODE || M > 32)
      return fail(QL_E_UNSUPPORTED, "the SiLU-and-mul epilogue runs on the decode algorithm (M <= 32)");
    if (N % 32) return fail(QL_E_INVALID, "SiLU-and-mul needs N (gate + up rows) a multiple of 32 (N=%lld)",
                            (long long)N);
    if (cfg.w_layout != 1 || cfg.rows_per_wave != 32 || (cfg.a_mode != 2 && cfg.a_mode != 4))
      return fail(QL_E_UNSUPPORTED, "SiLU-and-mul plans need packed weights, rows_per_wave 32 and a_mode 2 or 4");
  }
  if (is_mx(fmt)) {
    if (glu) return fail(QL_E_UNSUPPORTED, "MXFP8 / MXFP4 plans have no SiLU-and-mul epilogue");
    if (cfg.algo == QL_ALGO_TILED && cfg.w_lds)
      return fail(QL_E_UNSUPPORTED, "MXFP8 / MXFP4 tiled plans run the register ring (w_lds 0)");
    if (cfg.w_layout != 1 || (cfg.a_mode != 2 && cfg.a_mode != 3))
      return fail(QL_E_UNSUPPORTED, "MXFP8 / MXFP4 plans need packed weights and packed activations (a_mode 2 or 3)");
  }
  if (cfg.algo == QL_ALGO_TILED) return build_tiled_plan(fmt, M, N, K, cfg, source, out);
  if (cfg.algo != QL_ALGO_DECODE) return fail(QL_E_INVALID, "unknown algo %d", cfg.algo);
  if (M > 64) return fail(QL_E_UNSUPPORTED, "the decode algorithm serves M <= 64 (M=%lld)", (long long)M);
  if (cfg.swap_ab != 0 && cfg.swap_ab != 1) return fail(QL_E_INVALID, "swap_ab must be 0 or 1");
  if (!is_pow2(cfg.split_k) || cfg.split_k > 256) return fail(QL_E_INVALID, "split_k must be a power of two in [1, 256]");
  const int nw = cfg.waves_n * cfg.waves_k;
  if (cfg.waves_k < 1 || cfg.waves_n < 1 || (nw != 4 && nw != 8 && nw != 16))
    return fail(QL_E_INVALID, "waves_n * waves_k must be 4, 8 or 16");
  if (cfg.rows_per_wave != 16 && cfg.rows_per_wave != 32 && cfg.rows_per_wave != 64)
    return fail(QL_E_INVALID, "rows_per_wave must be 16, 32 or 64");
  if (cfg.prefetch != 1 && cfg.prefetch != 2 && cfg.prefetch != 4) return fail(QL_E_INVALID, "prefetch must be 1, 2 or 4");
  if (cfg.a_mode < 0 || cfg.a_mode > 5) return fail(QL_E_INVALID, "a_mode must be 0, 1, 2, 3, 4 or 5");
  if (cfg.a_mode == 5 && (fmt != QL_FP8_DYNAMIC && fmt != QL_W8A8_INT8))
    return fail(QL_E_UNSUPPORTED, "a_mode 5 (per-token amax given) serves FP8_Dynamic and W8A8_INT8");
  if (cfg.a_mode == 5 && (glu || M > 16 || K % 128))
    return fail(QL_E_UNSUPPORTED, "a_mode 5 needs M <= 16, K %% 128 == 0 and a plain (not SiLU-and-mul) epilogue");
  if (cfg.a_mode >= 2 && !cfg.w_layout) return fail(QL_E_UNSUPPORTED, "packed activations need packed weights");
  if (cfg.a_mode == 4 && fmt != QL_BLOCK_FP8 && (M > 16 || M * K > kFusedMaxValues || K % 512))
    return fail(QL_E_UNSUPPORTED, "fused per-token quantization needs M <= 16, M*K <= %lld and K %% 512 == 0",
                (long long)kFusedMaxValues);
  if (cfg.a_mode >= 2 && qlinear_packed_act_bytes(M, K) > (int64_t(1) << 30))
    return fail(QL_E_UNSUPPORTED, "packed activations exceed 2^30 bytes");
  if (cfg.w_lds != 0 && cfg.w_lds != 1) return fail(QL_E_INVALID, "w_lds must be 0 or 1");
  if (cfg.w_layout != 0 && cfg.w_layout != 1) return fail(QL_E_INVALID, "w_layout must be 0 or 1");
  if (cfg.w_layout == 1 && cfg.w_lds) return fail(QL_E_INVALID, "w_lds applies to row-major weights only");
  // tile_n of a decode plan: the rows of N one workgroup owns, 0 = all its waves cover
  if (cfg.tile_n != 0) {
    if (cfg.tile_n < 8 || cfg.tile_n % 8 || cfg.tile_n > qlk::kRowTileMax ||
        cfg.tile_n > cfg.waves_n * cfg.rows_per_wave)
      return fail(QL_E_INVALID, "a decode row tile (tile_n) is a multiple of 8 in [8, %d] and at most "
                  "waves_n * rows_per_wave", qlk::kRowTileMax);
    if (glu || is_mx(fmt) || cfg.w_lds)
      return fail(QL_E_UNSUPPORTED, "decode row tiles serve FP8_Dynamic / W8A8_INT8 / Block_FP8 linears with "
                  "weights read directly (no SiLU-and-mul, no LDS transpose, no MX)");
  }

  ql_plan_s* p = new ql_plan_s();
  p->fmt = fmt;
  p->M = M;
  p->N = N;
  p->K = K;
  p->cfg = cfg;
  p->source = source;
  p->G = (int)((K + 127) / 128);
  const int split = std::max(1, std::min<int>(cfg.split_k, std::max(1, p->G)));
  p->chunk_kb = p->G > 0 ? (p->G + split - 1) / split : 0;
  p->chunks = p->G > 0 ? (p->G + p->chunk_kb - 1) / p->chunk_kb : 1;
  p->mt = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  if (p->chunk_kb >= qlk::kShapeChunkLimit) {
    delete p;
    return fail(QL_E_UNSUPPORTED, "a decode K chunk holds fewer than 2^14 blocks of 128 (raise split_k)");
  }
  // Block_FP8 fused quantization reads only its K chunk: M * chunk values
  if ((cfg.a_mode == 4 && fmt == QL_BLOCK_FP8 || cfg.a_mode == 5) && (M > 16 || M * p->chunk_kb * 128 > kFusedMaxValues)) {
    const long long chunk = (long long)p->chunk_kb * 128;
    delete p;
    return fail(QL_E_UNSUPPORTED, "fused group quantization needs M <= 16 and M * chunk <= %lld (chunk %lld)",
                (long long)kFusedMaxValues, chunk);
  }
  const int rg = cfg.rows_per_wave / 16;
  p->glu = glu;
  // GLU: a tile's waves side by side cover 16 output columns each
  p->bn = glu ? cfg.waves_n * 16 : (cfg.tile_n ? cfg.tile_n : cfg.waves_n * rg * 16);
  p->n_tiles = (int)(((glu ? N / 2 : N) + p->bn - 1) / p->bn);
  const int64_t lds_a = (cfg.a_mode == 1 || cfg.a_mode == 3) ? (int64_t)p->chunk_kb * p->mt * 2048
                       : cfg.a_mode >= 4 ? 512 + M * ((int64_t)p->chunk_kb * 128 + 64) +
                                               (fmt == QL_BLOCK_FP8 ? M * (int64_t)p->chunk_kb * 4 : 0)
                                         : 0;
  const int64_t lds_w = (cfg.w_lds && !cfg.w_layout) ? (int64_t)nw * 2 * rg * 2048 : 0;
  const int64_t lds_red = cfg.waves_k > 1 ? (int64_t)nw * rg * p->mt * 1024 : 0;
  p->lds = std::max(lds_a + lds_w, lds_red);
  if (p->lds > kLdsLimit) {
    const long long need = (long long)p->lds;
    delete p;
    return fail(QL_E_UNSUPPORTED, "config needs %lld bytes of LDS (limit %lld); use a_mode 0 or 2, or a larger split_k",
                need, (long long)kLdsLimit);
  }
  p->ws_acc_bytes = p->chunks > 1 ? ((M * N * 4 + 255) / 256) * 256 : 0;
  p->ws_bytes = p->chunks > 1 ? p->ws_acc_bytes + (int64_t)p->n_tiles * 4 : 0;
  const int wm = cfg.w_layout ? qlk::W_PACKED : (cfg.w_lds ? qlk::W_LDS_TRANSPOSE : qlk::W_DIRECT);
  p->key = qlk::DecodeKey{kernel_fmt(fmt), cfg.swap_ab, p->mt, rg, nw, cfg.prefetch, cfg.a_mode, wm, glu ? 1 : 0};
  qlk::DecodeArgs dummy{};
  hipError_t pe;
  switch (p->key.fmt) {
    case qlk::FMT_INT8: pe = qlk::decode_dispatch_int8(p->key, dim3(1), dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    case qlk::FMT_BLOCK: pe = qlk::decode_dispatch_block(p->key, dim3(1), dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    case qlk::FMT_MX: pe = qlk::decode_dispatch_mx(p->key, dim3(1), dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    case qlk::FMT_MX4: pe = qlk::decode_dispatch_mx4(p->key, dim3(1), dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
    default: pe = qlk::decode_dispatch_fp8(p->key, dim3(1), dim3(1), (size_t)p->lds, nullptr, dummy, true); break;
  }
  if (pe == hipErrorInvalidDeviceFunction) {
    delete p;
    return fail(QL_E_UNSUPPORTED, "no kernel instantiated for this configuration");
  }
  // any other error: raising the LDS limit needs a GPU; the launch reports it if it matters
  *out = p;
  return QL_OK;
}

bool parse_force(ql_config* c) {
  const char* s = std::getenv("QLINEAR_FORCE");
  if (!s || !*s) return false;
  int v[12];
  if (std::sscanf(s, "%d,%d,%d,%d,%d,%d,%d,%d,%d,%d,%d,%d", &v[0], &v[1], &v[2], &v[3], &v[4], &v[5], &v[6], &v[7],
                  &v[8], &v[9], &v[10], &v[11]) != 12)
    return false;
  *c = ql_config{v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7], v[8], v[9], v[10], v[11]};
  return true;
}

// x / aq_out / sa_out: the fused plans' input X and their quantizer outputs
// (a_q and a_scale are then unused).
// amax: the per-token amax words of X and their counter (activation mode 5,
// required), or the SiLU-and-mul epilogue's amax output (optional).
ql_status launch_gemm(const ql_plan_s* p, const void* a_q, const void* a_scale, const void* w_q,
                      const void* w_scale, void* y, void* workspace, void* acc_out, hipStream_t s,
                      bool from_forward = false, const void* x = nullptr, void* aq_out = nullptr,
                      float* sa_out = nullptr, uint32_t* amax = nullptr) {
  const bool fused = !p->tiled && (p->cfg.a_mode == 4 || p->cfg.a_mode == 5);
  if (fused && !from_forward) return fail(QL_E_INVALID, "a fused-quantization plan runs through qlinear_forward");
  if (!p->tiled && p->cfg.a_mode == 5 && !amax)
    return fail(QL_E_INVALID, "an a_mode 5 plan runs through qlinear_forward_amax (it reads the given amax)");
  if (amax && !aligned16(amax)) return fail(QL_E_ALIGN, "amax is not 16-byte aligned");
  if (p->glu && acc_out) return fail(QL_E_UNSUPPORTED, "raw accumulators are not kept by a SiLU-and-mul plan");
  if (p->M == 0 || p->N == 0) return QL_OK;
  if (!y) return fail(QL_E_INVALID, "y is NULL");
  if (!aligned16(y)) return fail(QL_E_ALIGN, "y is not 16-byte aligned");
  if (p->K == 0) {   // Y = 0 (SiLU-and-mul plans: silu(0) * 0 over the [M, N/2] output)
    hipError_t e = qlk::launch_fill_zero_bf16(y, p->M * (p->glu ? p->N / 2 : p->N), s);
    return e == hipSuccess ? QL_OK : hip_fail(e, "zero fill");
  }
  if (fused) {
    if (!x || !aq_out || !sa_out || !w_q || !w_scale) return fail(QL_E_INVALID, "NULL operand pointer");
    if (!aligned16(x) || !aligned16(aq_out) || !aligned16(sa_out) || !aligned16(w_q) || !aligned16(w_scale))
      return fail(QL_E_ALIGN, "operand pointers must be 16-byte aligned");
  } else {
    if (!a_q || !a_scale || !w_q || !w_scale) return fail(QL_E_INVALID, "NULL operand pointer");
    if (!aligned16(a_q) || !aligned16(w_q) || !aligned16(a_scale) || !aligned16(w_scale))
      return fail(QL_E_ALIGN, "operand pointers must be 16-byte aligned");
  }
  if (p->ws_bytes > 0 && !workspace) return fail(QL_E_INVALID, "split-K plan needs a workspace");
  if (workspace && !aligned16(workspace)) return fail(QL_E_ALIGN, "workspace is not 16-byte aligned");
  if (acc_out && !aligned16(acc_out)) return fail(QL_E_ALIGN, "acc_out is not 16-byte aligned");

  qlk::DecodeArgs a{};
  a.a = static_cast<const uint8_t*>(a_q);
  a.sa = static_cast<const float*>(a_scale);   // MXFP8: E8M0 bytes, read as such by the kernel
  a.w = static_cast<const uint8_t*>(w_q);
  a.sw = static_cast<const float*>(w_scale);
  a.y = static_cast<uint16_t*>(y);
  a.ws = workspace;
  a.counters = p->ws_bytes > 0
                   ? reinterpret_cast<unsigned*>(static_cast<char*>(workspace) + p->ws_acc_bytes)
                   : nullptr;
  a.acc_out = acc_out;
  a.x = static_cast<const uint16_t*>(x);
  a.aq_out = static_cast<uint8_t*>(aq_out);
  a.sa_out = sa_out;
  a.amax = amax;
  a.M = (int)p->M;
  a.N = (int)p->N;
  a.K = (int)p->K;
  a.G = p->G;
  a.split = p->chunks;
  a.chunk_kb = p->chunk_kb;
  a.waves_k = p->cfg.waves_k;
  a.n_tiles = p->n_tiles;
  a.tiles_n = p->tiles_n;
  a.row_tile = p->tiled ? 0 : p->cfg.tile_n;
  hipError_t e;
  if (p->tiled) {
    const dim3 tgrid((unsigned)(p->n_tiles * p->chunks));
    switch (p->tkey.fmt) {
      case qlk::FMT_INT8: e = qlk::tiled_dispatch_int8(p->tkey, tgrid, (size_t)p->lds, s, a, false); break;
      case qlk::FMT_MX: e = qlk::tiled_dispatch_mx(p->tkey, tgrid, (size_t)p->lds, s, a, false); break;
      case qlk::FMT_MX4: e = qlk::tiled_dispatch_mx4(p->tkey, tgrid, (size_t)p->lds, s, a, false); break;
      case qlk::FMT_BLOCK: e = qlk::tiled_dispatch_block(p->tkey, tgrid, (size_t)p->lds, s, a, false); break;
      default: e = qlk::tiled_dispatch_fp8(p->tkey, tgrid, (size_t)p->lds, s, a, false); break;
    }
    return e == hipSuccess ? QL_OK : hip_fail(e, "tiled GEMM launch");
  }
  const dim3 grid((unsigned)(p->n_tiles * p->chunks)), block((unsigned)p->key.nw * 64u);
  switch (p->key.fmt) {
    case qlk::FMT_INT8: e = qlk::decode_dispatch_int8(p->key, grid, block, (size_t)p->lds, s, a, false); break;
    case qlk::FMT_BLOCK: e = qlk::decode_dispatch_block(p->key, grid, block, (size_t)p->lds, s, a, false); break;
    case qlk::FMT_MX: e = qlk::decode_dispatch_mx(p->key, grid, block, (size_t)p->lds, s, a, false); break;
    case qlk::FMT_MX4: e = qlk::decode_dispatch_mx4(p->key, grid, block, (size_t)p->lds, s, a, false); break;
    default: e = qlk::decode_dispatch_fp8(p->key, grid, block, (size_t)p->lds, s, a, false); break;
  }
  return e == hipSuccess ? QL_OK : hip_fail(e, "decode GEMM launch");
}

ql_status quantize_act(int32_t fmt, const void* x_bf16, int64_t M, int64_t K, void* a_q, void* a_scale,
                       bool packed, void* stream) {
  ql_status st = check_sizes(fmt, M, K, "M");
  if (st != QL_OK) return st;
  if (packed && qlinear_packed_act_bytes(M, K) > (int64_t(1) << 30))
    return fail(QL_E_UNSUPPORTED, "packed activations exceed 2^30 bytes");
  if (M == 0 || K == 0) return QL_OK;
  if (!x_bf16 || !a_q || !a_scale) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(x_bf16) || !aligned16(a_q) || !aligned16(a_scale)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (is_mx(fmt))   // MXFP4 plans take MXFP8 activations
    e = qlk::launch_quant_mx(x_bf16, M, K, a_q, static_cast<uint8_t*>(a_scale), packed, s);
  else if (fmt == QL_BLOCK_FP8)
    e = qlk::launch_quant_groups(x_bf16, M, K, a_q, static_cast<float*>(a_scale), packed, s);
  else
    e = qlk::launch_quant_rows(kernel_fmt(fmt), x_bf16, M, K, a_q, static_cast<float*>(a_scale), packed, s);
  return e == hipSuccess ? QL_OK : hip_fail(e, "activation quantizer launch");
}

// Split-K workspace for callers that cannot allocate (qlinear_forward_noalloc):
// one array per GPU, held until the process ends, shared by every such call
// on that GPU.  In host code `scratch` names a host-side stand-in; the
// device address comes from hipGetSymbolAddress, once per device.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address; on the first call on a device the
// array is also cleared on `s` (a fill kernel, so a graph being captured
// records an ordinary node) -- the kernels leave it all-zero after each run.
ql_status device_scratch(hipStream_t s, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(QL_E_UNSUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    e = qlk::launch_fill_zero_bf16(ptr, kScratchBytes / 2, s);
    if (e != hipSuccess) return hip_fail(e, "scratch clear");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QL_OK;
}

ql_status forward_impl(ql_plan p, const void* x_bf16, void* a_q, void* a_scale, const void* w_q,
                       const void* w_scale, void* y, void* workspace, void* stream, uint32_t* amax = nullptr) {
  if (!p->tiled && (p->cfg.a_mode == 4 || p->cfg.a_mode == 5))
    return launch_gemm(p, nullptr, nullptr, w_q, w_scale, y, workspace, nullptr, static_cast<hipStream_t>(stream),
                       true, x_bf16, a_q, static_cast<float*>(a_scale), amax);
  ql_status st = quantize_act(p->fmt, x_bf16, p->M, p->K, a_q, a_scale, p->cfg.a_mode >= 2, stream);
  if (st != QL_OK) return st;
  return launch_gemm(p, a_q, a_scale, w_q, w_scale, y, workspace, nullptr, static_cast<hipStream_t>(stream), false,
                     nullptr, nullptr, nullptr, amax);
}

}  // namespace

extern "C" {

int32_t qlinear_version(void) { return 100; }

const char* qlinear_status_string(int32_t s) {
  switch (s) {
    case QL_OK: return "QL_OK";
    case QL_E_INVALID: return "QL_E_INVALID";
    case QL_E_UNSUPPORTED: return "QL_E_UNSUPPORTED";
    case QL_E_NO_TABLE_ENTRY: return "QL_E_NO_TABLE_ENTRY";
    case QL_E_HIP: return "QL_E_HIP";
    case QL_E_ALIGN: return "QL_E_ALIGN";
    case QL_E_TABLE: return "QL_E_TABLE";
    default: return "QL_E_UNKNOWN";
  }
}

const char* qlinear_last_error(void) { return g_err.c_str(); }

ql_status qlinear_quantize_act(int32_t fmt, const void* x_bf16, int64_t M, int64_t K, void* a_q,
                               void* a_scale, void* stream) {
  return quantize_act(fmt, x_bf16, M, K, a_q, a_scale, false, stream);
}

int64_t qlinear_packed_act_bytes(int64_t M, int64_t K) {
  if (M < 0 || K < 0) return 0;
  return ((M + 15) / 16) * ((K + 127) / 128) * 2048;
}

ql_status qlinear_quantize_act_packed(int32_t fmt, const void* x_bf16, int64_t M, int64_t K, void* a_packed,
                                      void* a_scale, void* stream) {
  return quantize_act(fmt, x_bf16, M, K, a_packed, a_scale, true, stream);
}

ql_status qlinear_quantize_weight(int32_t fmt, const void* w_bf16, int64_t N, int64_t K, void* w_q,
                                  void* w_scale, void* stream) {
  ql_status st = check_sizes(fmt, N, K, "N");
  if (st != QL_OK) return st;
  if (N == 0 || K == 0) return QL_OK;
  if (!w_bf16 || !w_q || !w_scale) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(w_bf16) || !aligned16(w_q) || !aligned16(w_scale)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fmt == QL_MXFP8)
    e = qlk::launch_quant_mx(w_bf16, N, K, w_q, static_cast<uint8_t*>(w_scale), false, s);
  else if (fmt == QL_MXFP4)
    e = qlk::launch_quant_mx4(w_bf16, N, K, w_q, static_cast<uint8_t*>(w_scale), s);
  else if (fmt == QL_BLOCK_FP8)
    e = qlk::launch_quant_wblocks(w_bf16, N, K, w_q, static_cast<float*>(w_scale), s);
  else
    e = qlk::launch_quant_rows(kernel_fmt(fmt), w_bf16, N, K, w_q, static_cast<float*>(w_scale), false, s);
  return e == hipSuccess ? QL_OK : hip_fail(e, "weight quantizer launch");
}

int64_t qlinear_packed_weight_bytes_fp4(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return ((N + 15) / 16) * (K / 128) * 1024;
}

ql_status qlinear_pack_weight_fp4(const void* w_q, int64_t N, int64_t K, void* w_packed, void* stream) {
  ql_status st = check_sizes(QL_MXFP4, N, K, "N");
  if (st != QL_OK) return st;
  if (N == 0 || K == 0) return QL_OK;
  if (!w_q || !w_packed) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(w_q) || !aligned16(w_packed)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipError_t e = qlk::launch_pack_weight_fp4(w_q, N, K, w_packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "MXFP4 weight packing launch");
}

int64_t qlinear_packed_mx_scale_bytes(int64_t R, int64_t K) {
  if (R < 0 || K < 0) return 0;
  return ((R + 15) / 16) * (K / 128) * 64;
}

ql_status qlinear_pack_mx_scales(const void* scales, int64_t R, int64_t K, void* packed, void* stream) {
  ql_status st = check_sizes(QL_MXFP8, R, K, "R");
  if (st != QL_OK) return st;
  if (R == 0 || K == 0) return QL_OK;
  if (!scales || !packed) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(scales) || !aligned16(packed)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipError_t e = qlk::launch_pack_mx_scales(scales, R, K, packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "MXFP8 scale packing launch");
}

ql_status qlinear_table_load(const char* path, int64_t* n_entries) {
  if (!path) return fail(QL_E_INVALID, "path is NULL");
  std::ifstream f(path);
  if (!f) return fail(QL_E_TABLE, "cannot open table %s", path);
  std::vector<TableEntry> rows;
  std::string line;
  int lineno = 0;
  while (std::getline(f, line)) {
    ++lineno;
    const size_t hash = line.find('#');
    if (hash != std::string::npos) line.resize(hash);
    std::istringstream is(line);
    TableEntry e{};
    long long M, N, K;
    if (!(is >> e.fmt)) continue;  // blank or comment line
    if (!(is >> M >> N >> K >> e.cfg.algo >> e.cfg.swap_ab >> e.cfg.split_k >> e.cfg.waves_n >> e.cfg.waves_k >>
          e.cfg.rows_per_wave >> e.cfg.prefetch >> e.cfg.a_mode >> e.cfg.w_lds >> e.cfg.w_layout >> e.cfg.tile_m >>
          e.cfg.tile_n))
      return fail(QL_E_TABLE, "%s:%d: malformed entry", path, lineno);
    if (!(is >> e.us)) e.us = 0;
    std::string kind;
    e.us_class = act_class(e.cfg.a_mode);
    if (is >> kind) {
      if (kind != "fwd" && kind != "glu" && kind != "amx")
        return fail(QL_E_TABLE, "%s:%d: unknown entry kind '%s'", path, lineno, kind.c_str());
      e.us_class = kind == "glu" ? 3 : kind == "amx" ? 4 : 2;
    }
    if (!valid_fmt(e.fmt) || M < 1 || N < 1 || K < 1) return fail(QL_E_TABLE, "%s:%d: bad key", path, lineno);
    e.M = M;
    e.N = N;
    e.K = K;
    rows.push_back(e);
  }
  {
    std::lock_guard<std::mutex> lk(g_table_mu);
    g_table.swap(rows);
    if (n_entries) *n_entries = (int64_t)g_table.size();
  }
  return QL_OK;
}

void qlinear_table_clear(void) {
  std::lock_guard<std::mutex> lk(g_table_mu);
  g_table.clear();
}

static ql_status plan_for_layout(int32_t fmt, int32_t layout, int a_class, int64_t M, int64_t N, int64_t K,
                                 ql_plan* out_plan) {
  if (layout != 0 && layout != 1) return fail(QL_E_INVALID, "w_layout must be 0 or 1");
  ql_config c;
  if (parse_force(&c)) {
    const int fc = act_class(c.a_mode);
    const bool ok = a_class == 2 ? (fc == 1 || fc == 2) : a_class == 4 ? (fc == 1 || fc == 4) : fc == a_class;
    if (c.w_layout != layout || !ok) return fail(QL_E_INVALID, "QLINEAR_FORCE names other operand layouts");
    return build_plan(fmt, M, N, K, c, QL_SRC_CUSTOM, out_plan);
  }
  // a table entry that no longer builds (an instantiation removed since the
  // sweep) falls through to the heuristic instead of failing the plan
  if (table_lookup(fmt, layout, a_class, M, N, K, &c) && build_plan(fmt, M, N, K, c, QL_SRC_TABLE, out_plan) == QL_OK)
    return QL_OK;
  ql_status st = QL_E_UNSUPPORTED;
  // a given-amax forward plan without its own entry: a_mode 5 by the heuristic, else the packed-A plan
  if (a_class == 4) {
    for (const ql_config& h : heuristic_candidates(fmt, layout, 4, M, N, K))
      if (h.a_mode == 5 && build_plan(fmt, M, N, K, h, QL_SRC_HEURISTIC, out_plan) == QL_OK) return QL_OK;
    a_class = 1;
    if (table_lookup(fmt, layout, 1, M, N, K, &c) && build_plan(fmt, M, N, K, c, QL_SRC_TABLE, out_plan) == QL_OK)
      return QL_OK;
  }
  // a forward plan without its own entry: the packed-activation plan
  if (a_class == 2 && table_lookup(fmt, layout, 1, M, N, K, &c) &&
      build_plan(fmt, M, N, K, c, QL_SRC_TABLE, out_plan) == QL_OK)
    return QL_OK;
  for (const ql_config& h : heuristic_candidates(fmt, layout, a_class, M, N, K))
    if ((st = build_plan(fmt, M, N, K, h, QL_SRC_HEURISTIC, out_plan)) == QL_OK) break;
  return st;
}

ql_status qlinear_plan(int32_t fmt, int64_t M, int64_t N, int64_t K, ql_plan* out_plan) {
  return plan_for_layout(fmt, 0, 0, M, N, K, out_plan);
}

ql_status qlinear_plan_packed(int32_t fmt, int64_t M, int64_t N, int64_t K, ql_plan* out_plan) {
  return plan_for_layout(fmt, 1, 0, M, N, K, out_plan);
}

ql_status qlinear_plan_layouts(int32_t fmt, int64_t M, int64_t N, int64_t K, int32_t w_layout, int32_t a_packed,
                               ql_plan* out_plan) {
  if (a_packed < 0 || a_packed > 3) return fail(QL_E_INVALID, "a_packed must be 0, 1, 2 or 3");
  if (a_packed && !w_layout) return fail(QL_E_UNSUPPORTED, "packed activations need packed weights");
  if (a_packed == 3 && fmt != QL_FP8_DYNAMIC && fmt != QL_W8A8_INT8)
    return fail(QL_E_UNSUPPORTED, "given-amax forward plans serve FP8_Dynamic and W8A8_INT8");
  return plan_for_layout(fmt, w_layout, a_packed == 3 ? 4 : a_packed, M, N, K, out_plan);
}

ql_status qlinear_encode_e4m3(const float* x, int64_t n, void* codes, void* stream) {
  if (n < 0 || n > (int64_t(1) << 30)) return fail(QL_E_INVALID, "n=%lld outside [0, 2^30]", (long long)n);
  if (n == 0) return QL_OK;
  if (!x || !codes) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(x) || !aligned16(codes)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipError_t e = qlk::launch_encode_e4m3(x, n, codes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "E4M3 encoder launch");
}

ql_status qlinear_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t loads_in_flight,
                              int32_t check, void* sink, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes > (int64_t(1) << 36))
    return fail(QL_E_INVALID, "bytes=%lld must be a multiple of 16 in [0, 2^36]", (long long)bytes);
  if (workgroups == 0) workgroups = 1024;
  if (workgroups < 1 || workgroups > 65536) return fail(QL_E_INVALID, "workgroups=%d outside [1, 65536]", workgroups);
  if (loads_in_flight == 0) loads_in_flight = 8;
  if (loads_in_flight != 4 && loads_in_flight != 8)
    return fail(QL_E_INVALID, "loads_in_flight=%d must be 4 or 8", loads_in_flight);
  if (!src || !sink) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(src) || !aligned16(sink)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipError_t e = qlk::launch_stream_read(src, (uint64_t)bytes, workgroups, loads_in_flight, check != 0,
                                         static_cast<uint32_t*>(sink),
                                         static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "stream read launch");
}

ql_status qlinear_stream_read_bcast(const void* src, int64_t bytes, const void* bcast, int64_t bcast_bytes,
                                    int32_t workgroups, int32_t threads, int32_t loads_in_flight, int32_t check,
                                    void* sink, void* stream) {
  if (bytes < 0 || bytes % 16 || bytes > (int64_t(1) << 36))
    return fail(QL_E_INVALID, "bytes=%lld must be a multiple of 16 in [0, 2^36]", (long long)bytes);
  if (bcast_bytes < 0 || bcast_bytes % 16 || bcast_bytes > (int64_t(1) << 30))
    return fail(QL_E_INVALID, "bcast_bytes=%lld must be a multiple of 16 in [0, 2^30]", (long long)bcast_bytes);
  if (workgroups == 0) workgroups = 256;
  if (workgroups < 1 || workgroups > 65536) return fail(QL_E_INVALID, "workgroups=%d outside [1, 65536]", workgroups);
  if (threads == 0) threads = 1024;
  if (threads != 256 && threads != 512 && threads != 1024)
    return fail(QL_E_INVALID, "threads=%d must be 256, 512 or 1024", threads);
  if (loads_in_flight == 0) loads_in_flight = 4;
  if (loads_in_flight != 2 && loads_in_flight != 4)
    return fail(QL_E_INVALID, "loads_in_flight=%d must be 2 or 4", loads_in_flight);
  if (!src || !sink || (bcast_bytes && !bcast)) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(src) || !aligned16(sink) || (bcast && !aligned16(bcast)))
    return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipError_t e = qlk::launch_stream_read_bcast(src, (uint64_t)bytes, bcast, (uint64_t)bcast_bytes, workgroups,
                                               threads, loads_in_flight, check != 0, static_cast<uint32_t*>(sink),
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "broadcast read launch");
}

int64_t qlinear_packed_weight_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0) return 0;
  return ((N + 15) / 16) * ((K + 127) / 128) * 2048;
}

ql_status qlinear_pack_weight(const void* w_q, int64_t N, int64_t K, void* w_packed, void* stream) {
  if (N < 0 || K < 0 || K % 16) return fail(QL_E_INVALID, "bad shape (N=%lld, K=%lld)", (long long)N, (long long)K);
  if (qlinear_packed_weight_bytes(N, K) > (int64_t(1) << 30)) return fail(QL_E_UNSUPPORTED, "packed weights exceed 2^30 bytes");
  if (N == 0 || K == 0) return QL_OK;
  if (!w_q || !w_packed) return fail(QL_E_INVALID, "NULL pointer");
  if (!aligned16(w_q) || !aligned16(w_packed)) return fail(QL_E_ALIGN, "pointers must be 16-byte aligned");
  hipError_t e = qlk::launch_pack_weight(w_q, N, K, w_packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "weight packing launch");
}

ql_status qlinear_plan_from_table(int32_t fmt, int64_t M, int64_t N, int64_t K, ql_plan* out_plan) {
  if (out_plan) *out_plan = nullptr;
  ql_config c;
  if (!table_lookup(fmt, 0, 0, M, N, K, &c))
    return fail(QL_E_NO_TABLE_ENTRY, "no table entry for fmt=%d M=%lld N=%lld K=%lld", fmt, (long long)M,
                (long long)N, (long long)K);
  return build_plan(fmt, M, N, K, c, QL_SRC_TABLE, out_plan);
}

ql_status qlinear_plan_with_config(int32_t fmt, int64_t M, int64_t N, int64_t K, const ql_config* cfg,
                                   ql_plan* out_plan) {
  if (!cfg) return fail(QL_E_INVALID, "cfg is NULL");
  return build_plan(fmt, M, N, K, *cfg, QL_SRC_CUSTOM, out_plan);
}

ql_status qlinear_plan_glu_with_config(int32_t fmt, int64_t M, int64_t N, int64_t K, const ql_config* cfg,
                                       ql_plan* out_plan) {
  if (!cfg) return fail(QL_E_INVALID, "cfg is NULL");
  return build_plan(fmt, M, N, K, *cfg, QL_SRC_CUSTOM, out_plan, true);
}

ql_status qlinear_plan_glu(int32_t fmt, int64_t M, int64_t N, int64_t K, int32_t a_packed, ql_plan* out_plan) {
  if (out_plan) *out_plan = nullptr;
  if (a_packed != 1 && a_packed != 2) return fail(QL_E_INVALID, "a_packed must be 1 or 2 for SiLU-and-mul plans");
  // a swept SiLU-and-mul entry first (timed as a forward)
  ql_config tc;
  if (!std::getenv("QLINEAR_FORCE") && table_lookup(fmt, 1, 3, M, N, K, &tc)) {
    if (a_packed == 1 && tc.a_mode == 4) tc.a_mode = 2;   // qlinear_run takes quantized activations
    if (build_plan(fmt, M, N, K, tc, QL_SRC_TABLE, out_plan, true) == QL_OK) return QL_OK;
  }
  // else the merged linear's own plan (table or heuristic), keeping the
  // fields the SiLU-and-mul kernels are instantiated for
  ql_plan base = nullptr;
  ql_status st = plan_for_layout(fmt, 1, a_packed, M, N, K, &base);
  if (st != QL_OK) return st;
  ql_config c = base->cfg;
  const int32_t source = base->source;
  delete base;
  if (c.algo != QL_ALGO_DECODE) return fail(QL_E_UNSUPPORTED, "the SiLU-and-mul epilogue serves M <= 32");
  c.rows_per_wave = 32;
  const int nw = c.waves_n * c.waves_k;
  if (nw != 4 && nw != 8) {
    c.waves_n = 1;
    c.waves_k = 4;
  }
  if (c.prefetch > 2) c.prefetch = 2;
  if (c.a_mode == 3) c.a_mode = 2;
  st = build_plan(fmt, M, N, K, c, source, out_plan, true);
  if (st == QL_E_UNSUPPORTED) {     // that shape is not instantiated: the plain one is
    c.swap_ab = 0;
    c.waves_n = 1;
    c.waves_k = 4;
    c.prefetch = 1;
    st = build_plan(fmt, M, N, K, c, source, out_plan, true);
  }
  return st;
}

ql_status qlinear_plan_info(ql_plan p, ql_config* cfg, ql_plan_facts* facts) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  if (cfg) {
    *cfg = p->cfg;
    cfg->split_k = p->chunks;
  }
  if (facts) {
    facts->source = p->source;
    facts->chunks = p->chunks;
    facts->chunk_k = p->chunk_kb * 128;
    facts->workgroups = p->n_tiles * p->chunks;
    facts->threads = p->tiled ? ((p->fmt != QL_BLOCK_FP8 || p->cfg.tile_m * p->cfg.tile_n >= 128 * 256) ? 512 : 256)
                              : p->key.nw * 64;
    facts->lds_bytes = (int32_t)p->lds;
    facts->workspace_bytes = p->ws_bytes;
    facts->epilogue = p->glu ? 1 : 0;
  }
  return QL_OK;
}

int64_t qlinear_workspace_bytes(ql_plan p) { return p ? p->ws_bytes : 0; }

void qlinear_plan_destroy(ql_plan p) { delete p; }

ql_status qlinear_run(ql_plan p, const void* a_q, const void* a_scale, const void* w_q, const void* w_scale,
                      void* y, void* workspace, void* stream) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  return launch_gemm(p, a_q, a_scale, w_q, w_scale, y, workspace, nullptr, static_cast<hipStream_t>(stream));
}

ql_status qlinear_run_debug_acc(ql_plan p, const void* a_q, const void* a_scale, const void* w_q,
                                const void* w_scale, void* y, void* workspace, void* acc_out, void* stream) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  if (!acc_out && p->M > 0 && p->N > 0 && p->K > 0) return fail(QL_E_INVALID, "acc_out is NULL");
  return launch_gemm(p, a_q, a_scale, w_q, w_scale, y, workspace, acc_out, static_cast<hipStream_t>(stream));
}

ql_status qlinear_forward(ql_plan p, const void* x_bf16, void* a_q, void* a_scale, const void* w_q,
                          const void* w_scale, void* y, void* workspace, void* stream) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  return forward_impl(p, x_bf16, a_q, a_scale, w_q, w_scale, y, workspace, stream);
}

ql_status qlinear_forward_glu_amax(ql_plan p, const void* x_bf16, void* a_q, void* a_scale, const void* w_q,
                                   const void* w_scale, void* h_bf16, void* h_amax, void* workspace, void* stream) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  if (!p->glu) return fail(QL_E_INVALID, "qlinear_forward_glu_amax takes a SiLU-and-mul plan");
  if (p->fmt != QL_FP8_DYNAMIC && p->fmt != QL_W8A8_INT8)
    return fail(QL_E_UNSUPPORTED, "the per-token amax of H serves FP8_Dynamic and W8A8_INT8");
  if (!h_amax && p->M > 0 && p->N > 0 && p->K > 0) return fail(QL_E_INVALID, "h_amax is NULL");
  if (p->K == 0) return fail(QL_E_UNSUPPORTED, "K = 0: H is zero, its amax is not accumulated");
  return forward_impl(p, x_bf16, a_q, a_scale, w_q, w_scale, h_bf16, workspace, stream, static_cast<uint32_t*>(h_amax));
}

ql_status qlinear_forward_amax(ql_plan p, const void* x_bf16, void* x_amax, void* a_q, void* a_scale, const void* w_q,
                               const void* w_scale, void* y, void* workspace, void* stream) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  if (p->glu) return fail(QL_E_INVALID, "qlinear_forward_amax takes a plain (not SiLU-and-mul) plan");
  if (p->fmt != QL_FP8_DYNAMIC && p->fmt != QL_W8A8_INT8)
    return fail(QL_E_UNSUPPORTED, "the given per-token amax serves FP8_Dynamic and W8A8_INT8");
  if (p->M == 0) return QL_OK;
  if (!x_amax) return fail(QL_E_INVALID, "x_amax is NULL");
  if (!aligned16(x_amax)) return fail(QL_E_ALIGN, "x_amax is not 16-byte aligned");
  // a decode plan with work to do takes the buffer: a_mode 5 reads it, any
  // other finds the amax itself and its first workgroup clears the buffer
  if (!p->tiled && p->N > 0 && p->K > 0)
    return forward_impl(p, x_bf16, a_q, a_scale, w_q, w_scale, y, workspace, stream, static_cast<uint32_t*>(x_amax));
  ql_status st = forward_impl(p, x_bf16, a_q, a_scale, w_q, w_scale, y, workspace, stream);
  if (st != QL_OK) return st;
  hipError_t e = qlk::launch_fill_zero_bf16(x_amax, qlk::AMAX_WORDS * 2, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "amax clear");
}

ql_status qlinear_forward_noalloc(ql_plan p, const void* x_bf16, void* a_q, void* a_scale, const void* w_q,
                                  const void* w_scale, void* y, void* stream) {
  if (!p) return fail(QL_E_INVALID, "plan is NULL");
  void* ws = nullptr;
  if (p->ws_bytes > 0) {
    if (p->ws_bytes > kScratchBytes)
      return fail(QL_E_UNSUPPORTED, "plan needs %lld bytes of split-K workspace; the no-allocation scratch holds %lld",
                  (long long)p->ws_bytes, (long long)kScratchBytes);
    ql_status st = device_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != QL_OK) return st;
  }
  return forward_impl(p, x_bf16, a_q, a_scale, w_q, w_scale, y, ws, stream);
}

ql_status qlinear_graph_begin(void* stream) {
  if (!stream) return fail(QL_E_INVALID, "cannot capture the default stream");
  hipError_t e = hipStreamBeginCapture(static_cast<hipStream_t>(stream), hipStreamCaptureModeThreadLocal);
  return e == hipSuccess ? QL_OK : hip_fail(e, "hipStreamBeginCapture");
}

ql_status qlinear_graph_end(void* stream, ql_graph* out_graph) {
  if (!stream || !out_graph) return fail(QL_E_INVALID, "NULL argument");
  *out_graph = nullptr;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(static_cast<hipStream_t>(stream), &g);
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t x = nullptr;
  e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    (void)hipGraphDestroy(g);
    return hip_fail(e, "hipGraphInstantiate");
  }
  *out_graph = new ql_graph_s{g, x};
  return QL_OK;
}

ql_status qlinear_graph_launch(ql_graph g, void* stream) {
  if (!g) return fail(QL_E_INVALID, "graph is NULL");
  hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QL_OK : hip_fail(e, "hipGraphLaunch");
}

void qlinear_graph_destroy(ql_graph g) {
  if (!g) return;
  (void)hipGraphExecDestroy(g->exec);
  (void)hipGraphDestroy(g->graph);
  delete g;
}

}  // extern "C"
