/*
 * qlinear.h -- C ABI of the MI355X (gfx950) scaled quantized linear.
 *
 *   Y[M,N] = s_a[m] * s_w[n] * (A_q[M,K] . W_q[N,K]^T)      bf16 output
 *
 * plus the dynamic activation quantizer that produces (A_q, s_a) and the
 * offline weight quantizer that produces (W_q, s_w).
 *
 * Sources.  The operation and its variants are described on five web pages
 * about the article "Building a High-Performance and Portable vLLM Linear
 * Backend with Helion" (PyTorch blog).  Cited here as:
 *   [Summary]  English summary, yuxiaoba.github.io/tech/en/helion-linear/
 *   [Noticias] "Helion entra al backend lineal de vLLM y supera a CUTLASS en
 *              Hopper", noticias.mechatronicstore.cl
 *   [Deep dive] "Optimizing vLLM Linear Backend Performance using Helion
 *              Kernel DSL", explore.n1n.ai
 *
 * Formats ([Summary] "Put algorithm selection inside the search space", last
 * paragraph; [Noticias] "El backend lineal de Helion / Alcance"):
 *   QL_FP8_DYNAMIC  OCP E4M3 activations scaled per token, weights per output channel
 *   QL_W8A8_INT8    int8 activations per token, weights per output channel
 *   QL_BLOCK_FP8    E4M3 with 1x128 activation groups and 128x128 weight blocks
 *   QL_MXFP8        E4M3 with one E8M0 (power-of-two) scale per 32 values along K,
 *                   activations and weights alike
 *   QL_MXFP4        MXFP4 weights (E2M1 values, two a byte, one E8M0 scale per 32)
 *                   with MXFP8 activations
 * Quantization rule (the pages give none; the plain reading): symmetric
 * absmax, s = fl(amax / Q) with Q = 127 (int8) or 448 (E4M3); code =
 * round-half-even(fl(x / s)) clamped to [-Q, Q]; an all-zero group gets s = 1.
 * MXFP8 ([Noticias] "¿Qué son vLLM y Helion?" lists block-scaled NVFP4 among
 * the formats linear backends serve; gfx950's counterpart is OCP
 * microscaling, whose v1.0 rule is taken here): per block of 32 values
 * e = floor(log2(amax)) - 8 clamped to [-127, 127] (-127 for an all-zero
 * block), scale byte e + 127, code = E4M3 round-to-nearest-even of
 * x * 2^-e clamped to [-448, 448].  The matrix core applies the scales inside
 * the product: Y = bf16(sum_k 2^(ea+ew) a_k w_k), no scale epilogue.  MXFP4
 * weights: the same rule with E2M1 elements (values 0, 0.5, 1, 1.5, 2, 3, 4,
 * 6; e = floor(log2(amax)) - 2, clamp to [-6, 6], round to nearest, ties to
 * the even code); W_q holds them two a byte, low nibble = even K, [N, K/2].
 *
 * Data layouts (all row-major, caller-owned device memory):
 *   X      bf16   [M, K]                 activations (input of the quantizer)
 *   A_q    1 byte [M, K]                 int8 or E4M3 codes
 *   s_a    fp32   [M]  or [M, K/128]     (Block_FP8: one scale per 1x128 group)
 *          uint8  [M, K/32]              (MXFP8: E8M0 bytes; every scale pointer of
 *                                        this header is void* for that reason)
 *   W      bf16   [N, K]                 weights (input of the weight quantizer)
 *   W_q    1 byte [N, K]                 row n = output channel n, K contiguous
 *   s_w    fp32   [N]  or [ceil(N/128), K/128];  MXFP8: uint8 [N, K/32]
 *   Y      bf16   [M, N]
 *
 * Argument rules checked on the host before any launch (QL_E_INVALID /
 * QL_E_ALIGN / QL_E_UNSUPPORTED otherwise):
 *   M, N, K >= 0; K % 16 == 0 (rows are 16-byte aligned); Block_FP8 and
 *   MXFP8 need K % 128 == 0; N * K and M * K at most 2^30; device pointers 16-byte
 *   aligned and non-null whenever the sizes make them used.
 *   M == 0 or N == 0 is a successful no-op.  K == 0 gives Y == 0.
 *
 * Streams: every `stream` argument is a hipStream_t passed as void* (NULL =
 * the default stream).  Calls only enqueue work: no synchronisation, no
 * device allocation, no memset nodes, so sequences of calls can be captured
 * into a hipGraph (see qlinear_graph_begin).
 *
 * Errors: every call returns a ql_status; nothing throws or aborts across the
 * ABI.  qlinear_last_error() returns a thread-local description of the last
 * failure.  A failing HIP launch is reported as QL_E_HIP.
 *
 * Threading: plans are immutable after creation and may be shared between
 * threads and streams; concurrent runs of split-K plans need distinct
 * workspaces.  The sweep table is process-global; load it before creating
 * plans from several threads.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QL_FP8_DYNAMIC = 0,
  QL_W8A8_INT8 = 1,
  QL_BLOCK_FP8 = 2,
  QL_MXFP8 = 3,
  QL_MXFP4 = 4
} ql_format;

typedef enum {
  QL_OK = 0,
  QL_E_INVALID = 1,        /* bad size, format, null pointer or config */
  QL_E_UNSUPPORTED = 2,    /* valid request the library does not serve */
  QL_E_NO_TABLE_ENTRY = 3, /* qlinear_plan_from_table: no sweep-table entry */
  QL_E_HIP = 4,            /* a HIP runtime call or kernel launch failed */
  QL_E_ALIGN = 5,          /* pointer not 16-byte aligned */
  QL_E_TABLE = 6           /* sweep table file unreadable or malformed */
} ql_status;

/* Algorithm family of a plan. */
typedef enum {
  QL_ALGO_DECODE = 0, /* weight-streaming kernel for M <= 64 (decode token counts; the planner's
                          heuristic uses it up to 32 -- 64 for the MX formats -- and the sweep
                          table may pick it up to 64) */
  QL_ALGO_TILED = 1   /* LDS-tiled matrix-core GEMM for larger M */
} ql_algo;

/* Where a plan's configuration came from. */
typedef enum {
  QL_SRC_TABLE = 0,     /* the offline sweep table */
  QL_SRC_HEURISTIC = 1, /* built-in rule (no table entry) */
  QL_SRC_CUSTOM = 2     /* qlinear_plan_with_config or QLINEAR_FORCE */
} ql_source;

/*
 * Tunable configuration of one GEMM launch.  The two algorithmic choices of
 * the pages are `split_k` (powers of two 1..256) and `swap_ab` (boolean)
 * ([Summary] "Put algorithm selection inside the search space"; [Noticias]
 * "¿Cómo se implementa el kernel?"); the rest are the low-level tile
 * parameters searched alongside them.
 *   Standard GEMM = split_k 1, swap_ab 0; Split-K = split_k > 1;
 *   Swap-AB = swap_ab 1 (the weights become the matrix core's first operand).
 */
typedef struct {
  int32_t algo;          /* ql_algo */
  int32_t swap_ab;       /* 0 or 1 */
  int32_t split_k;       /* 1,2,4,...,256; clamped to the number of 128-wide K blocks */
  int32_t waves_n;       /* DECODE: waves of a workgroup side by side along N;
                            waves_n * waves_k = 4, 8 or 16 (8 and 16: packed weights) */
  int32_t waves_k;       /* DECODE: waves of a workgroup sharing its K chunk */
  int32_t rows_per_wave; /* DECODE: 16, 32 or 64 weight rows per wave */
  int32_t prefetch;      /* DECODE: 128-wide K blocks per wave and batch, two batches in flight (1, 2 or 4);
                            TILED: 128-wide K blocks in flight per workgroup (1, 2 or 4) */
  int32_t a_mode;        /* activations: 0 = row-major A_q read per K block; 1 (DECODE) = row-major
                            A_q chunk staged in LDS; 2 = packed A_q (qlinear_quantize_act_packed)
                            read per K block; 3 (DECODE) = packed A_q chunk staged in LDS and
                            shared by the workgroup's waves; 4 (DECODE) = fused quantization:
                            every workgroup quantizes the bf16 rows of X itself (row or
                            1x128-group amax, then the codes of its K chunk into LDS) and the
                            plan runs only through qlinear_forward, which then writes a_q
                            (packed) and a_scale from inside the GEMM launch -- M <= 16;
                            per-token formats: M*K <= 16384, K % 512 == 0; Block_FP8:
                            M * (K chunk) <= 16384.  2..4 need packed weights */
  int32_t w_lds;         /* DECODE, row-major weights: 1 = coalesced weight loads (8 rows x 128 B
                            per instruction) transposed to the matrix-core layout through LDS;
                            0 = direct loads in operand order.  TILED, packed weights and
                            activations: 1 = both operands go straight to an LDS ring of
                            `prefetch` (2 or 3) stages by LDS-DMA loads; 0 = register ring */
  int32_t w_layout;      /* weight layout the plan reads: 0 = row-major W_q[N,K];
                            1 = packed tiles (qlinear_pack_weight) */
  int32_t tile_m;        /* TILED: workgroup tile rows (tokens): 64, 128 or 256 */
  int32_t tile_n;        /* TILED: workgroup tile columns (weight rows): 128 or 256;
                            every tile runs 8 waves (Block_FP8 below 128 x 256: 4); 256 x 256
                            needs packed operands, the LDS-DMA ring of 2 stages and a
                            per-token format.  TILED reads swap_ab, split_k,
                            a_mode (0 or 2), w_layout, w_lds, prefetch and the tile; the
                            other fields are ignored.
                            DECODE: 0, or the rows of N one workgroup owns -- a multiple of 8
                            in [8, 120], at most waves_n * rows_per_wave -- so that N can be
                            spread evenly over the compute units (N = 6144: 256 workgroups of
                            24 rows instead of 192 of 32); the rows of a workgroup's last row
                            group beyond its tile are neither loaded nor stored.  FP8_Dynamic,
                            W8A8_INT8 and Block_FP8 linears with weights read directly (w_lds
                            0), not SiLU-and-mul plans */
} ql_config;

/* Derived launch facts of a plan (read-only). */
typedef struct {
  int32_t source;          /* ql_source */
  int32_t chunks;          /* effective number of K chunks */
  int32_t chunk_k;         /* K elements per chunk (last chunk may be shorter) */
  int32_t workgroups;      /* grid size */
  int32_t threads;         /* threads per workgroup */
  int32_t lds_bytes;       /* dynamic LDS per workgroup */
  int64_t workspace_bytes; /* see qlinear_workspace_bytes */
  int32_t epilogue;        /* 0 = Y [M, N]; 1 = SiLU-and-mul of a merged gate/up weight, Y [M, N/2] */
} ql_plan_facts;

typedef struct ql_plan_s* ql_plan;
typedef struct ql_graph_s* ql_graph;

/* Library version (major*10000 + minor*100 + patch). */
int32_t qlinear_version(void);
/* Static string naming a status code; never NULL. */
const char* qlinear_status_string(int32_t status);
/* Thread-local description of the last failure on this thread ("" if none). */
const char* qlinear_last_error(void);

/*
 * Dynamic activation quantizer ([Summary] last paragraph of "Put algorithm
 * selection inside the search space": per-token or 1x128 activation scaling).
 *   x_bf16  [M, K] bf16 in;  a_q [M, K] codes out;  a_scale fp32 [M] or [M, K/128]
 *   out (MXFP8: E8M0 bytes [M, K/32]).
 * Bit-exact contract: amax exact in fp32, IEEE division, round-half-even,
 * clamp, E4M3 round-to-nearest-even, fp32 subnormals kept (MXFP8: the
 * shared exponent from amax's bits, an exact power-of-two scaling, E4M3
 * round-to-nearest-even).  An all-zero row (or group) gets scale 1 and zero
 * codes (MXFP8: E8M0 byte 0).  X must be finite: for a row (or group)
 * holding an infinity or NaN the scale and codes are outside the contract;
 * the other rows are unaffected.
 */
ql_status qlinear_quantize_act(int32_t fmt, const void* x_bf16, int64_t M, int64_t K,
                               void* a_q, void* a_scale, void* stream);

/*
 * The same quantizer writing the packed activation layout that plans with
 * a_mode = 2 read: the weight packing below applied to A_q, i.e. 2 KB tiles
 * (t, kb) of 16 tokens x 128 K at byte (t * ceil(K/128) + kb) * 2048, tile
 * byte h*1024 + l*16 + j = A_q[16t + l%16][128kb + 64h + 16*(l/16) + j], zero
 * for tokens >= M and K beyond K.  Every activation load of the GEMM then
 * reads one contiguous kilobyte.  a_packed holds qlinear_packed_act_bytes(M, K)
 * bytes; a_scale is as for qlinear_quantize_act -- except MXFP8, whose scales
 * are then written in the lane-order layout of qlinear_pack_mx_scales
 * (qlinear_packed_mx_scale_bytes(M, K) bytes).  Same codes, same scales.
 */
int64_t qlinear_packed_act_bytes(int64_t M, int64_t K);
ql_status qlinear_quantize_act_packed(int32_t fmt, const void* x_bf16, int64_t M, int64_t K,
                                      void* a_packed, void* a_scale, void* stream);

/*
 * The E4M3 encoder every FP8 quantizer of the library applies to its
 * quotients, on its own: codes[i] = OCP E4M3 code of x[i] clamped to
 * [-448, 448], rounded to nearest even (signed zeros kept, subnormal codes
 * produced).  x: n binary32 values, codes: n bytes, both device memory,
 * 16-byte aligned; n <= 2^30.  NaN inputs are outside the contract.  Used to
 * check the encoder against the format definition.  Enqueue-only.
 */
ql_status qlinear_encode_e4m3(const float* x, int64_t n, void* codes, void* stream);

/*
 * Measurement aid, not part of the linear: read `bytes` bytes of device
 * memory at `src` once with 16-byte nontemporal loads -- workgroup w of
 * `workgroups` (256 threads each; 0 = 1024) reads the w-th contiguous slice,
 * `loads_in_flight` (4 or 8; 0 = 8) loads per lane in flight.  Its time for
 * a buffer the size of a GEMM's operands is the streaming-read ceiling a
 * weight-streaming kernel is held against on this device (launch and ramp
 * included, as for the GEMM).  With `check` nonzero every workgroup also
 * writes the wrapping 32-bit sum of the words it read to sink[w] (a test of
 * the read); with `check` zero the kernel writes nothing in practice (a lane
 * writes its sum to sink[w] only if it equals a fixed constant, which keeps
 * the loads from being elided).  bytes % 16 == 0 and bytes <= 2^36; src and
 * sink device memory, 16-byte aligned; sink holds 4 * workgroups bytes.
 * Enqueue-only.
 */
ql_status qlinear_stream_read(const void* src, int64_t bytes, int32_t workgroups, int32_t loads_in_flight,
                              int32_t check, void* sink, void* stream);

/*
 * Measurement aid for the same purpose, one level finer: the ceiling of a
 * weight-streaming decomposition without a K split, in which every
 * workgroup owns a share of the weight rows over all of K and therefore
 * multiplies them with every token's activations.  Workgroup w (of
 * `workgroups`, 0 = 256, i.e. one per compute unit; `threads` 256, 512 or
 * 1024, 0 = 1024) reads the w-th contiguous slice of src, as
 * qlinear_stream_read does, and, interleaved with it, all bcast_bytes of
 * bcast -- the activation block every such workgroup must load (from L2
 * once one workgroup has brought it in).  `loads_in_flight` (2 or 4; 0 = 4)
 * pieces of each stream per lane.  `check` as for qlinear_stream_read: then
 * sink[w] = wrapping 32-bit sum of the words of slice w plus those of
 * bcast.  bytes % 16 == 0 and bytes <= 2^36; bcast_bytes % 16 == 0 and
 * bcast_bytes <= 2^30; device pointers, 16-byte aligned (bcast may be NULL
 * when bcast_bytes is 0); sink holds 4 * workgroups bytes.  Enqueue-only.
 */
ql_status qlinear_stream_read_bcast(const void* src, int64_t bytes, const void* bcast, int64_t bcast_bytes,
                                    int32_t workgroups, int32_t threads, int32_t loads_in_flight, int32_t check,
                                    void* sink, void* stream);

/*
 * Offline weight quantizer: per output channel (rows of W) or per 128x128
 * block for Block_FP8 (the last block row may be ragged).
 *   w_bf16 [N, K] in;  w_q [N, K] out;  w_scale fp32 [N] or [ceil(N/128), K/128]
 *   out (MXFP8: E8M0 bytes [N, K/32], the activation rule applied to rows of W;
 *   MXFP4: w_q is [N, K/2] bytes of E2M1 pairs, w_scale E8M0 bytes [N, K/32]).
 * Same rounding contract as the activation quantizer.
 */
ql_status qlinear_quantize_weight(int32_t fmt, const void* w_bf16, int64_t N, int64_t K,
                                  void* w_q, void* w_scale, void* stream);

/*
 * Offline weight packing (optional, for the packed-weight plans).  The
 * packed layout stores each 16-row x 128-K block of W_q as 2 KB in the order
 * the matrix core consumes it, with a row group's blocks adjacent, so the
 * decode kernel streams whole contiguous kilobytes per load instruction:
 *   tile (t, kb) at byte (t * ceil(K/128) + kb) * 2048; tile byte
 *   h*1024 + l*16 + j = W_q[16t + l%16][128kb + 64h + 16*(l/16) + j],
 *   zero outside N x K (h in {0,1}, l in [0,64), j in [0,16)).
 * The scales are unchanged.  qlinear_pack_weight reads w_q [N, K] (1-byte
 * codes, row-major) and writes qlinear_packed_weight_bytes(N, K) bytes.
 */
int64_t qlinear_packed_weight_bytes(int64_t N, int64_t K);
ql_status qlinear_pack_weight(const void* w_q, int64_t N, int64_t K, void* w_packed, void* stream);

/*
 * MXFP8 scales in lane order, the layout MXFP8 plans read for weights and
 * activations alike: the E8M0 bytes of 16 rows x one 128-wide K block take
 * 64 bytes at (t * K/128 + kb) * 64, byte l = s[16t + l%16][4kb + l/16] (the
 * scale byte lane l hands the matrix core with that K block; see QL_MXFP8),
 * 0 for rows >= R.  One wave then reads a K block's scales as 64 contiguous
 * bytes.  qlinear_pack_mx_scales reads row-major scales [R, K/32] (as
 * qlinear_quantize_weight writes them; K % 128 == 0) and writes
 * qlinear_packed_mx_scale_bytes(R, K) bytes; the packed MXFP8 activation
 * quantizer writes this layout directly.  Enqueue-only.
 */
int64_t qlinear_packed_mx_scale_bytes(int64_t R, int64_t K);

/*
 * MXFP4 weight packing: 1 KB per (16-row group t, 128-wide K block kb) at
 * (t * K/128 + kb) * 1024; lane l's 16 bytes at l*16 hold row 16t + l%16, K
 * [128kb + 32*(l/16), +32) as E2M1 pairs (low nibble first) -- the 32 values
 * lane l hands the scaled matrix core as its E2M1 operand, which pairs them
 * with the same K of the E4M3 operand's packed pieces.  Reads w_q [N, K/2]
 * (K % 128 == 0), writes qlinear_packed_weight_bytes_fp4(N, K) bytes, zero
 * past N.  The scales are packed with qlinear_pack_mx_scales.  Enqueue-only.
 */
int64_t qlinear_packed_weight_bytes_fp4(int64_t N, int64_t K);
ql_status qlinear_pack_weight_fp4(const void* w_q, int64_t N, int64_t K, void* w_packed, void* stream);
ql_status qlinear_pack_mx_scales(const void* scales, int64_t R, int64_t K, void* packed, void* stream);

/*
 * Offline sweep table ([Summary] "Hybrid dispatch addresses runtime
 * overhead": per-shape, per-token-count tuned configurations).  Text file,
 * one entry per line: fmt M N K algo swap_ab split_k waves_n waves_k
 * rows_per_wave prefetch a_mode w_lds w_layout tile_m tile_n [time_us [fwd]];
 * '#' starts a comment.  Entries are looked up for the operand layouts asked
 * for (w_layout; row-major A_q = a_mode 0/1, packed A_q = a_mode 2/3).  An
 * entry marked "fwd" (and every a_mode 4 entry) is a forward plan: the best
 * configuration for quantize + GEMM together, fused or not, and its time
 * covers both.  An entry marked "glu" is the same for a SiLU-and-mul plan
 * (qlinear_plan_glu) of the merged gate/up weight [N, K].
 * Loading replaces the in-process table.  Returns the entry count via n_entries.
 */
ql_status qlinear_table_load(const char* path, int64_t* n_entries);
void qlinear_table_clear(void);

/*
 * Plan one GEMM shape: the runtime half of the pages' hybrid dispatch -- a
 * per-shape configuration searched offline, with the algorithmic switches
 * (split_k, swap_ab) inside the search space, and looked up per token-count
 * bucket at run time ([Summary] "Put algorithm selection inside the search
 * space" and "Hybrid dispatch addresses runtime overhead": token counts 1, 2,
 * 4, 8, 16, 24, 32 tuned separately).  Looks up the sweep table with M rounded
 * up to the next tuned token bucket {1,2,4,8,16,24,32} (M > 32: the nearest
 * tuned M at or above, else the largest); without an entry a built-in heuristic is used
 * (facts.source tells which).  The environment variable QLINEAR_FORCE =
 * "algo,swap,split,wn,wk,rows,prefetch,amode,wlds,wlayout,tile_m,tile_n"
 * overrides both (its operand layouts must match the call).  Without a table
 * entry M <= 32 plans use the DECODE algorithm and M > 32 the TILED one; the
 * table may choose DECODE up to M = 64 (four 16-token tiles, packed weights).  qlinear_plan: row-major
 * W_q and A_q.
 * Host-only: nothing is enqueued and nothing is allocated (a TILED plan
 * raises its kernel's dynamic LDS limit with hipFuncSetAttribute).
 */
ql_status qlinear_plan(int32_t fmt, int64_t M, int64_t N, int64_t K, ql_plan* out_plan);
/* Like qlinear_plan, for weights packed with qlinear_pack_weight (row-major A_q). */
ql_status qlinear_plan_packed(int32_t fmt, int64_t M, int64_t N, int64_t K, ql_plan* out_plan);
/*
 * Like qlinear_plan for any operand layouts: w_layout 0 = row-major W_q,
 * 1 = packed weights; a_packed 0 = row-major A_q (qlinear_quantize_act),
 * 1 = packed A_q (qlinear_quantize_act_packed; the plan's a_mode is 2 or 3),
 * 2 = a forward plan for packed weights (the table's "fwd" entry, else the
 * packed-A_q plan): a_mode 2, 3 or 4, to be run with qlinear_forward only;
 * 3 = a forward plan for an input whose per-token amax is given (FP8_Dynamic
 * and W8A8_INT8, packed weights; the table's "amx" entry, else a_mode 5 when
 * M <= 16 and K % 128 == 0, else the packed-A_q plan), to be run with
 * qlinear_forward_amax.
 */
ql_status qlinear_plan_layouts(int32_t fmt, int64_t M, int64_t N, int64_t K, int32_t w_layout,
                               int32_t a_packed, ql_plan* out_plan);
/* Like qlinear_plan (row-major weights) but only from the table; QL_E_NO_TABLE_ENTRY when absent. */
ql_status qlinear_plan_from_table(int32_t fmt, int64_t M, int64_t N, int64_t K, ql_plan* out_plan);
/* Plan with an explicit configuration (validated; QL_E_INVALID / QL_E_UNSUPPORTED on a bad one). */
ql_status qlinear_plan_with_config(int32_t fmt, int64_t M, int64_t N, int64_t K,
                                   const ql_config* cfg, ql_plan* out_plan);
/*
 * SiLU-and-mul epilogue ([Deep dive] "Understanding Helion": activations
 * such as SiLU fused into the GEMM's write-back).  The weight [N, K] is a
 * merged gate/up projection -- rows [0, N/2) gate, rows [N/2, N) up -- and
 * the plan's runs write, instead of the linear's output, the [M, N/2] bf16
 * tensor H[m, i] = bf16(silu(g) * u) with g, u the binary32 epilogue values
 * of output columns i and N/2 + i (after the scales, before any rounding),
 * silu(g) = g / (1 + exp(-g)).  Decode algorithm only (M <= 32), packed
 * weights, N % 32 == 0; qlinear_run (a_packed 1) or qlinear_forward
 * (a_packed 2: the quantizer may be fused as well) drive it as usual with
 * y_bf16 [M, N/2].  qlinear_plan_glu takes the table's "glu" entry, else the
 * merged linear's planned configuration (table or heuristic) with 32 rows a
 * wave (a gate and an up group); qlinear_run_debug_acc rejects these plans.
 */
ql_status qlinear_plan_glu(int32_t fmt, int64_t M, int64_t N, int64_t K, int32_t a_packed, ql_plan* out_plan);
ql_status qlinear_plan_glu_with_config(int32_t fmt, int64_t M, int64_t N, int64_t K, const ql_config* cfg,
                                       ql_plan* out_plan);
/* Effective configuration and launch facts of a plan (either pointer may be NULL). */
ql_status qlinear_plan_info(ql_plan plan, ql_config* cfg, ql_plan_facts* facts);
/*
 * Bytes of device workspace a run needs (0 for split_k == 1).  Split-K plans
 * accumulate partial sums (int32 for INT8, fp32 for FP8) plus one arrival
 * counter per output tile.  The caller allocates it and zeroes it ONCE; every
 * run leaves it all-zero again (the last-arriving workgroup of a tile clears
 * its part), so it can be reused by later runs and graph replays.
 */
int64_t qlinear_workspace_bytes(ql_plan plan);
void qlinear_plan_destroy(ql_plan plan);

/*
 * The scaled quantized GEMM: Y = epilogue(A_q . W_q^T) with the scales fused
 * into the epilogue ([Summary] "Put algorithm selection inside the search
 * space": split-K combines partial results; quantized variants add scaling).
 * Epilogue op order (fixed): INT8 y = bf16(fl(fl(f32(acc) * s_a[m]) * s_w[n]))
 * with an exact int32 accumulator; FP8_Dynamic the same on the fp32
 * accumulator; Block_FP8 applies s_a[m,g] * s_w[n/128,g] to every 128-wide K
 * group's partial inside the K loop and rounds the fp32 sum to bf16; MXFP8
 * hands the E8M0 bytes to the scaled matrix-core instruction, which applies
 * them to every 32-wide block of products, and rounds the fp32 sum to bf16.
 * MXFP8 and MXFP4 plans read packed weights (MXFP4: qlinear_pack_weight_fp4)
 * and packed activations (a_mode 2 or 3; the tiled algorithm a_mode 2), and
 * both scales in the lane order of qlinear_pack_mx_scales.  MXFP4 runs on
 * the decode algorithm (M <= 64); MXFP8 also on the tiled one with the
 * register ring (w_lds 0; no 256 x 256 tile).
 * MXFP4 plans take MXFP8 activations (qlinear_quantize_act_packed with
 * fmt = QL_MXFP4 writes them).
 * a_q is in the plan's activation layout: row-major [M, K], or packed when
 * the plan's a_mode is 2 or 3; w_q in the plan's weight layout (w_layout).
 * Enqueue-only; workspace may be NULL when qlinear_workspace_bytes is 0.
 */
ql_status qlinear_run(ql_plan plan, const void* a_q, const void* a_scale,
                      const void* w_q, const void* w_scale, void* y_bf16,
                      void* workspace, void* stream);

/*
 * Test hook: same launch as qlinear_run, and additionally stores the raw
 * accumulator per output element into acc_out [M, N] (int32 for INT8, fp32
 * for FP8_Dynamic, the scaled fp32 sum for Block_FP8 and MXFP8) before the bf16 rounding.
 */
ql_status qlinear_run_debug_acc(ql_plan plan, const void* a_q, const void* a_scale,
                                const void* w_q, const void* w_scale, void* y_bf16,
                                void* workspace, void* acc_out, void* stream);

/*
 * Quantize the activations, then run the GEMM: the whole decode step of one
 * linear layer.  a_q / a_scale are caller-owned staging buffers; a_q is
 * written in the plan's activation layout (qlinear_packed_act_bytes(M, K)
 * bytes when a_mode is 2, 3 or 4, else M*K).  With a_mode 4 this is one
 * launch: the GEMM kernel quantizes X itself and also writes a_q / a_scale
 * (identical to what qlinear_quantize_act_packed writes).  qlinear_run
 * rejects an a_mode 4 plan with QL_E_INVALID.
 */
ql_status qlinear_forward(ql_plan plan, const void* x_bf16, void* a_q, void* a_scale,
                          const void* w_q, const void* w_scale, void* y_bf16,
                          void* workspace, void* stream);

/*
 * The gated MLP of a decode step as a chain: gate_up with the SiLU-and-mul
 * epilogue, then down, whose input H must be quantized per token.  The
 * deep-dive page lists fused epilogues -- activations, and quantization of the
 * output for the next layer -- among what a GEMM's write-back can carry
 * ([Deep dive] "Understanding Helion").  A per-token scale needs the whole
 * row's amax, which no single workgroup of gate_up sees; so the SiLU-and-mul
 * epilogue folds max |bf16(h)| of each token into a small buffer with atomic
 * maxima (exact: a maximum does not depend on the order), and down's
 * workgroups each quantize only their own K chunk of H with the rule of
 * qlinear_quantize_act (s = fl(amax / Q), code = round(fl(h / s)), the same
 * codes and scales bit for bit), in the GEMM launch itself: no separate
 * quantizer launch and no second pass over H.
 *
 * h_amax / x_amax: QL_AMAX_BUFFER_BYTES bytes (any M <= 32), 16-byte
 * aligned, caller-owned, all zero before the first producer runs.  Atomics
 * on one cache line serialize, so the maxima are spread over 64 replicas of
 * one 128-byte line each: word 32 r + m holds the binary32 bit pattern of
 * the largest |h| of token m among the producer waves that chose replica r
 * (the token's amax is the maximum over r); the consumer's arrival counters
 * follow (16 group counters and one counter of groups, a line each).  The
 * consumer (qlinear_forward_amax) leaves the whole buffer zero again, so one
 * buffer serves every layer in turn; a producer must be followed by exactly
 * one consumer before the next producer, and the two run in stream order.
 *
 * qlinear_forward_glu_amax: qlinear_forward of a SiLU-and-mul plan
 * (qlinear_plan_glu, FP8_Dynamic or W8A8_INT8) that also accumulates the
 * per-token amax of its output H [M, N/2] into h_amax.  K must be > 0.
 * qlinear_forward_amax: qlinear_forward of a plan from qlinear_plan_layouts
 * (..., a_packed = 3) for X whose amax words are x_amax.  An a_mode 5 plan is
 * one launch that reads X (bf16, the whole of it across the grid, each
 * workgroup its K chunk) and writes a_q / a_scale as qlinear_quantize_act_packed
 * would; any other decode plan runs the quantizer and the GEMM, whose first
 * workgroup clears the buffer (a large-M plan adds a fill launch).  Either
 * way x_amax is all zero afterwards.  Enqueue-only.
 */
#define QL_AMAX_BUFFER_BYTES 10368

ql_status qlinear_forward_glu_amax(ql_plan plan, const void* x_bf16, void* a_q, void* a_scale,
                                   const void* w_q, const void* w_scale, void* h_bf16, void* h_amax,
                                   void* workspace, void* stream);
ql_status qlinear_forward_amax(ql_plan plan, const void* x_bf16, void* x_amax, void* a_q, void* a_scale,
                               const void* w_q, const void* w_scale, void* y_bf16, void* workspace,
                               void* stream);

/*
 * For callers that cannot allocate device memory -- code running under
 * hipGraph capture, tight serving loops, harnesses that forbid hipMalloc:
 * qlinear_forward without the workspace argument.  A split-K plan's partial
 * sums and arrival counters live in a scratch array inside the library, one
 * per GPU (16 MiB = 16777216 bytes, held until the process
 * ends); nothing is allocated by this call, or by the library for it.  The
 * first call on a GPU clears that GPU's array with a fill kernel on `stream`
 * (make it outside graph capture, or capture it: the fill is an ordinary
 * node); every run leaves the array all-zero again.  All such calls on one
 * GPU share its array, so calls that overlap in time on one GPU (concurrent
 * streams, or graph replays in flight on two streams) race and must not be
 * made.  A plan whose workspace (qlinear_workspace_bytes) exceeds the scratch
 * is rejected with QL_E_UNSUPPORTED before anything is enqueued.  Otherwise
 * arguments, results and errors are those of qlinear_forward.
 */
ql_status qlinear_forward_noalloc(ql_plan plan, const void* x_bf16, void* a_q, void* a_scale,
                                  const void* w_q, const void* w_scale, void* y_bf16,
                                  void* stream);

/*
 * hipGraph dispatch for the small-M path ([Summary] "Hybrid dispatch
 * addresses runtime overhead": the tuned kernels run only under graph
 * replay, which removes the host launch cost).  qlinear_graph_begin starts
 * capturing `stream` (thread-local capture mode; `stream` must not be the
 * default stream); every qlinear_* call enqueued on it until
 * qlinear_graph_end is recorded into one executable graph.  The graph binds
 * the pointers given at capture time.  Replays are stream-ordered.
 */
ql_status qlinear_graph_begin(void* stream);
ql_status qlinear_graph_end(void* stream, ql_graph* out_graph);
ql_status qlinear_graph_launch(ql_graph graph, void* stream);
void qlinear_graph_destroy(ql_graph graph);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
