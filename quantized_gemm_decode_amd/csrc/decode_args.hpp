// Launch arguments of the decode (M <= 64) quantized GEMM kernel, shared by
// the host dispatcher and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlk {

// The per-token amax buffer (32-bit words).  Device-scope atomics on one
// cache line serialize, and every wave of a SiLU-and-mul grid folds its
// tokens' maxima into the buffer, so the maxima are spread over
// AMAX_REPLICAS lines of AMAX_LINE words (token m of replica r at word
// r * AMAX_LINE + m, M <= 32): a producer wave picks one replica, a
// consumer takes the maximum over all of them.  The consumer's arrival
// counters follow, one line each: AMAX_GROUPS group counters (workgroup b
// counts in group b % AMAX_GROUPS), then the counter of completed groups.
constexpr uint32_t AMAX_LINE = 32;
constexpr uint32_t AMAX_REPLICAS = 64;
constexpr uint32_t AMAX_GROUPS = 16;
constexpr uint32_t AMAX_CTR0 = AMAX_REPLICAS * AMAX_LINE;
constexpr uint32_t AMAX_TOP = AMAX_CTR0 + AMAX_GROUPS * AMAX_LINE;
constexpr uint32_t AMAX_WORDS = AMAX_TOP + AMAX_LINE;

// Format selector of the kernels (matches ql_format's order).  FMT_MX:
// MXFP8, E4M3 codes with one E8M0 scale byte per 32 values along K.
// FMT_MX4: MXFP4 weights (E2M1, two a byte) with MXFP8 activations.
enum { FMT_FP8 = 0, FMT_INT8 = 1, FMT_BLOCK = 2, FMT_MX = 3, FMT_MX4 = 4 };

// How the decode kernel reads the weights.
enum {
  W_DIRECT = 0,         // row-major W_q[N,K], loads in matrix-core operand order
  W_LDS_TRANSPOSE = 1,  // row-major W_q[N,K], coalesced loads + LDS transpose
  W_PACKED = 2          // packed 2 KB tiles (see launch_pack_weight)
};

struct DecodeArgs {
  const uint8_t* a;    // A_q [M, K] codes
  const float* sa;     // s_a [M] or [M, G]; MXFP8: E8M0 bytes in lane order, 64 per (16 rows, K block)
  const uint8_t* w;    // W_q [N, K] codes
  const float* sw;     // s_w [N] or [ceil(N/128), G]; MXFP8: as s_a, over the weight rows
  uint16_t* y;         // Y [M, N] bf16
  void* ws;            // split-K partial sums [M, N] (int32 or fp32), all-zero between runs
  unsigned* counters;  // split-K arrival counters [n_tiles], all-zero between runs
  void* acc_out;       // optional raw accumulators [M, N] (test hook), may be null
  // fused quantization (decode activation mode 4): the kernel reads X and
  // writes the codes (packed layout) and scales it computed, if non-null
  const uint16_t* x;   // X [M, K] bf16
  uint8_t* aq_out;     // packed A_q, ceil(M/16) x G tiles of 2 KB
  float* sa_out;       // s_a [M]
  // per-token amax buffer of X (layout below): written by a SiLU-and-mul
  // plan's epilogue (atomic max over its output H) when non-null; read --
  // and reset to zero by the last workgroup -- by an activation-mode-5 plan;
  // cleared by any other decode plan that is given it
  uint32_t* amax;
  int M, N, K;
  int G;               // number of 128-wide K blocks, ceil(K / 128)
  int split;           // number of K chunks (workgroups per output tile)
  int chunk_kb;        // K blocks per chunk; chunk c covers [c*chunk_kb, min(G, (c+1)*chunk_kb))
  int waves_k;         // waves of a workgroup that share one K chunk
  int n_tiles;         // output tiles along N (decode) / all output tiles (tiled)
  int tiles_n;         // tiled kernel: output tiles along N
  int row_tile;        // decode: rows of N a workgroup owns (a multiple of 8, <= 120), 0 = what its waves cover
};

// The decode kernel's packed launch word: waves_k (5 bits), split (9 bits),
// chunk_kb (14 bits), row_tile / 8 (4 bits); the planner keeps every decode
// plan inside these ranges (waves_k <= 16, split <= 256, chunk_kb < 2^14,
// row_tile a multiple of 8 up to 120).
constexpr int kShapeChunkLimit = 1 << 14;
constexpr int kRowTileMax = 120;
inline int decode_shape_word(const DecodeArgs& a) {
  const unsigned w = (unsigned)(a.waves_k & 31) | ((unsigned)(a.split & 511) << 5) |
                     ((unsigned)(a.chunk_kb & 16383) << 14) | ((unsigned)((a.row_tile / 8) & 15) << 28);
  return (int)w;
}

// Compile-time shape of one decode kernel instantiation.
struct DecodeKey {
  int fmt;   // FMT_FP8 / FMT_INT8 / FMT_BLOCK
  int swap;  // weights as the matrix core's first operand
  int mt;    // 16-wide token tiles (1: M <= 16, 2: M <= 32, 4: M <= 64)
  int rg;    // 16-row groups per wave (1, 2 or 4)
  int nw;    // waves per workgroup (4, 8 or 16)
  int pf;    // K blocks per prefetch batch
  int alds;  // activations: 0 row-major from L2, 1 row-major staged in LDS, 2 packed from L2,
             // 3 packed staged in LDS, 4 quantized from X inside the kernel (fused), 5 the same
             // with the per-token amax given (each workgroup reads only its K chunk of X)
  int wm;    // weight mode: W_DIRECT / W_LDS_TRANSPOSE / W_PACKED
  int glu;   // 1: merged gate/up weight, SiLU-and-mul epilogue, output [M, N/2]
};

// Compile-time shape of one tiled (M > 32) kernel instantiation.
struct TiledKey {
  int fmt;   // FMT_FP8 / FMT_INT8 / FMT_BLOCK / FMT_MX / FMT_MX4
  int swap;  // weights as the matrix core's first operand
  int bm;    // output tile rows (tokens): 64, 128 or 256
  int bn;    // output tile columns (weight rows): 128 or 256
  int wm;    // weight layout: W_DIRECT (row-major) or W_PACKED
  int pf;    // K blocks in flight in the register ring: 1, 2 or 4
  int ap;    // activations packed (1) or row-major (0)
  int ns;    // 0: register ring; 2 or 3: LDS-DMA ring of that many stages (packed operands)
};

// Launch an instantiated kernel; returns hipErrorInvalidDeviceFunction when
// the key has no instantiation.  `probe_only` checks without launching.
hipError_t decode_dispatch_fp8(const DecodeKey& k, dim3 grid, dim3 block, size_t lds,
                               hipStream_t s, const DecodeArgs& a, bool probe_only);
hipError_t decode_dispatch_int8(const DecodeKey& k, dim3 grid, dim3 block, size_t lds,
                                hipStream_t s, const DecodeArgs& a, bool probe_only);
hipError_t decode_dispatch_block(const DecodeKey& k, dim3 grid, dim3 block, size_t lds,
                                 hipStream_t s, const DecodeArgs& a, bool probe_only);
hipError_t decode_dispatch_mx(const DecodeKey& k, dim3 grid, dim3 block, size_t lds,
                              hipStream_t s, const DecodeArgs& a, bool probe_only);
hipError_t decode_dispatch_mx4(const DecodeKey& k, dim3 grid, dim3 block, size_t lds,
                               hipStream_t s, const DecodeArgs& a, bool probe_only);

// Tiled kernel launchers (tiled_*.hip); `probe_only` also raises the
// kernel's dynamic LDS limit to `lds`.
hipError_t tiled_dispatch_fp8(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                              bool probe_only);
hipError_t tiled_dispatch_int8(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                               bool probe_only);
hipError_t tiled_dispatch_block(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                                bool probe_only);
hipError_t tiled_dispatch_mx(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                             bool probe_only);
hipError_t tiled_dispatch_mx4(const TiledKey& k, dim3 grid, size_t lds, hipStream_t s, const DecodeArgs& a,
                              bool probe_only);

// Quantizer launchers (quant.hip).
// `packed`: codes in the packed activation layout (2 KB tiles of 16 rows x
// 128 K in matrix-core operand order, zero padding), else row-major [R, C].
hipError_t launch_quant_rows(int fmt, const void* x, int64_t R, int64_t C, void* q, float* s, bool packed,
                             hipStream_t st);
hipError_t launch_quant_groups(const void* x, int64_t M, int64_t K, void* q, float* s, bool packed,
                               hipStream_t st);
hipError_t launch_quant_wblocks(const void* w, int64_t N, int64_t K, void* q, float* s,
                                hipStream_t st);
hipError_t launch_fill_zero_bf16(void* y, int64_t count, hipStream_t st);
// plain streaming read of `bytes` (a multiple of 16), a contiguous slice per workgroup with `unroll`
// (4 or 8) loads in flight per lane; `check`: one 32-bit word sum per workgroup into sink
hipError_t launch_stream_read(const void* src, uint64_t bytes, int workgroups, int unroll, bool check,
                              uint32_t* sink, hipStream_t s);
// the same slices of `src` plus, interleaved, all of `bcast` in every workgroup; `threads` 256, 512
// or 1024, `unroll` (2 or 4) loads of each stream in flight per lane
hipError_t launch_stream_read_bcast(const void* src, uint64_t bytes, const void* bcast, uint64_t bcast_bytes,
                                    int workgroups, int threads, int unroll, bool check, uint32_t* sink,
                                    hipStream_t s);
// MXFP8 rows: x bf16 [R, C] (C % 32 == 0) -> E4M3 codes (row-major [R, C],
// or packed tiles when `packed`) and E8M0 scale bytes [R, C/32].
hipError_t launch_quant_mx(const void* x, int64_t R, int64_t C, void* q, uint8_t* s, bool packed,
                           hipStream_t st);
// MXFP8 scales [R, K/32] -> lane order: 64 bytes per (16-row group t, K
// block kb) at (t*G + kb)*64, byte l = s[16t + l%16][4kb + l/16], 0 past R.
hipError_t launch_pack_mx_scales(const void* s, int64_t R, int64_t K, void* packed, hipStream_t st);
// MXFP4 weights: w bf16 [N, K] -> E2M1 codes two a byte (low nibble = even K),
// row-major [N, K/2], and E8M0 scale bytes [N, K/32].
hipError_t launch_quant_mx4(const void* w, int64_t N, int64_t K, void* q, uint8_t* s, hipStream_t st);
// Row-major E2M1 bytes [N, K/2] -> 1 KB tiles per (16-row group t, 128-wide
// K block kb) at (t*G + kb)*1024; lane l's 16 bytes at l*16 are row
// 16t + l%16, K [128kb + 32(l/16), +32), zero past N.
hipError_t launch_pack_weight_fp4(const void* w_q, int64_t N, int64_t K, void* w_packed, hipStream_t st);
// codes[i] = E4M3 code of x[i] clamped to [-448, 448], round to nearest even.
hipError_t launch_encode_e4m3(const float* x, int64_t n, void* q, hipStream_t st);
// Row-major W_q[N,K] -> packed 2 KB tiles (zero padding to 16 rows / 128 K).
hipError_t launch_pack_weight(const void* w_q, int64_t N, int64_t K, void* w_packed, hipStream_t st);

}  // namespace qlk
