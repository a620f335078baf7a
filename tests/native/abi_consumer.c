/*
 * A plain C99 consumer of the library's C ABI (include/qlinear.h): no C++,
 * no Python, no torch.  Test infrastructure.
 *
 *   abi_consumer host <table>            calls that need no GPU: version,
 *                                        status strings, table, plans, sizes
 *   abi_consumer gpu <in.bin> <out.bin>  one linear on the GPU: quantize the
 *                                        weights and activations, plan, run,
 *                                        then the same two launches captured
 *                                        into a graph and replayed twice
 *
 * in.bin: int64 fmt, M, N, K, then X as bf16 bits [M, K] and W as bf16 bits
 * [N, K].  out.bin: Y as bf16 bits [M, N] from the eager run.  Exit status 0
 * on success; every failure prints what failed.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qlinear.h"

#define CHECK(cond, what)                                                   \
  do {                                                                      \
    if (!(cond)) {                                                          \
      fprintf(stderr, "FAILED: %s (%s)\n", what, qlinear_last_error());     \
      return 1;                                                             \
    }                                                                       \
  } while (0)
#define HIPCHECK(call)                                                      \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "FAILED: %s -> %d\n", #call, (int)e_);                \
      return 1;                                                             \
    }                                                                       \
  } while (0)

static int host_mode(const char* table) {
  int64_t n = 0;
  ql_plan plan = NULL;
  ql_config cfg;
  ql_plan_facts facts;
  CHECK(qlinear_version() > 0, "qlinear_version");
  CHECK(qlinear_status_string(QL_OK) != NULL && qlinear_status_string(12345) != NULL, "qlinear_status_string");
  CHECK(qlinear_table_load(table, &n) == QL_OK && n > 0, "qlinear_table_load");
  CHECK(qlinear_plan(QL_FP8_DYNAMIC, 8, 4096, 4096, &plan) == QL_OK && plan != NULL, "qlinear_plan");
  CHECK(qlinear_plan_info(plan, &cfg, &facts) == QL_OK, "qlinear_plan_info");
  CHECK(facts.source == QL_SRC_TABLE && facts.workgroups > 0 && facts.threads > 0, "plan facts");
  CHECK(qlinear_workspace_bytes(plan) == facts.workspace_bytes, "qlinear_workspace_bytes");
  qlinear_plan_destroy(plan);
  plan = NULL;
  CHECK(qlinear_plan(QL_FP8_DYNAMIC, 8, 4096, 100, &plan) == QL_E_INVALID && plan == NULL, "K % 16 rejected");
  CHECK(strlen(qlinear_last_error()) > 0, "qlinear_last_error after a failure");
  CHECK(qlinear_plan(7, 8, 4096, 4096, &plan) == QL_E_INVALID, "unknown format rejected");
  CHECK(qlinear_packed_weight_bytes(4096, 4096) == 4096 * 4096, "qlinear_packed_weight_bytes");
  CHECK(qlinear_packed_act_bytes(5, 256) == 2 * 2048, "qlinear_packed_act_bytes");
  printf("host ok: version %d, %lld table entries, plan %d workgroups x %d threads\n", qlinear_version(),
         (long long)n, facts.workgroups, facts.threads);
  return 0;
}

static int gpu_mode(const char* in_path, const char* out_path) {
  int64_t hdr[4];
  FILE* f = fopen(in_path, "rb");
  CHECK(f != NULL, "open input");
  CHECK(fread(hdr, sizeof(int64_t), 4, f) == 4, "read header");
  const int32_t fmt = (int32_t)hdr[0];
  const int64_t M = hdr[1], N = hdr[2], K = hdr[3];
  CHECK(M > 0 && N > 0 && K > 0 && K % 128 == 0 && M * K <= (1 << 24) && N * K <= (1 << 26), "input shape");
  uint16_t* hx = (uint16_t*)malloc((size_t)(M * K) * 2);
  uint16_t* hw = (uint16_t*)malloc((size_t)(N * K) * 2);
  uint16_t* hy = (uint16_t*)malloc((size_t)(M * N) * 2);
  uint16_t* hy2 = (uint16_t*)malloc((size_t)(M * N) * 2);
  CHECK(hx && hw && hy && hy2, "host buffers");
  CHECK(fread(hx, 2, (size_t)(M * K), f) == (size_t)(M * K), "read X");
  CHECK(fread(hw, 2, (size_t)(N * K), f) == (size_t)(N * K), "read W");
  fclose(f);

  /* scale buffer sizes: per token / per channel, or Block_FP8 groups and blocks */
  const int64_t sa_n = fmt == QL_BLOCK_FP8 ? M * (K / 128) : M;
  const int64_t sw_n = fmt == QL_BLOCK_FP8 ? ((N + 127) / 128) * (K / 128) : N;
  void *x, *w, *wq, *ws, *aq, *as, *y, *work = NULL;
  HIPCHECK(hipMalloc(&x, (size_t)(M * K) * 2));
  HIPCHECK(hipMalloc(&w, (size_t)(N * K) * 2));
  HIPCHECK(hipMalloc(&wq, (size_t)(N * K)));
  HIPCHECK(hipMalloc(&ws, (size_t)sw_n * 4));
  HIPCHECK(hipMalloc(&aq, (size_t)(M * K)));
  HIPCHECK(hipMalloc(&as, (size_t)sa_n * 4));
  HIPCHECK(hipMalloc(&y, (size_t)(M * N) * 2));
  HIPCHECK(hipMemcpy(x, hx, (size_t)(M * K) * 2, hipMemcpyHostToDevice));
  HIPCHECK(hipMemcpy(w, hw, (size_t)(N * K) * 2, hipMemcpyHostToDevice));

  ql_plan plan = NULL;
  CHECK(qlinear_quantize_weight(fmt, w, N, K, wq, ws, NULL) == QL_OK, "qlinear_quantize_weight");
  CHECK(qlinear_plan(fmt, M, N, K, &plan) == QL_OK, "qlinear_plan");
  const int64_t wsb = qlinear_workspace_bytes(plan);
  if (wsb > 0) {
    HIPCHECK(hipMalloc(&work, (size_t)wsb));
    HIPCHECK(hipMemset(work, 0, (size_t)wsb));   /* zeroed once; runs leave it zero */
  }
  CHECK(qlinear_quantize_act(fmt, x, M, K, aq, as, NULL) == QL_OK, "qlinear_quantize_act");
  CHECK(qlinear_run(plan, aq, as, wq, ws, y, work, NULL) == QL_OK, "qlinear_run");
  HIPCHECK(hipDeviceSynchronize());
  HIPCHECK(hipMemcpy(hy, y, (size_t)(M * N) * 2, hipMemcpyDeviceToHost));

  /* the same quantize + GEMM captured into a graph, replayed twice */
  hipStream_t s;
  ql_graph g = NULL;
  HIPCHECK(hipStreamCreate(&s));
  CHECK(qlinear_graph_begin(s) == QL_OK, "qlinear_graph_begin");
  CHECK(qlinear_quantize_act(fmt, x, M, K, aq, as, s) == QL_OK, "captured qlinear_quantize_act");
  CHECK(qlinear_run(plan, aq, as, wq, ws, y, work, s) == QL_OK, "captured qlinear_run");
  CHECK(qlinear_graph_end(s, &g) == QL_OK && g != NULL, "qlinear_graph_end");
  for (int rep = 0; rep < 2; ++rep) {
    HIPCHECK(hipMemsetAsync(y, 0, (size_t)(M * N) * 2, s));   /* eager, outside the graph */
    CHECK(qlinear_graph_launch(g, s) == QL_OK, "qlinear_graph_launch");
    HIPCHECK(hipStreamSynchronize(s));
    HIPCHECK(hipMemcpy(hy2, y, (size_t)(M * N) * 2, hipMemcpyDeviceToHost));
    CHECK(memcmp(hy, hy2, (size_t)(M * N) * 2) == 0, "graph replay equals the eager run");
  }
  qlinear_graph_destroy(g);
  qlinear_plan_destroy(plan);
  HIPCHECK(hipStreamDestroy(s));

  f = fopen(out_path, "wb");
  CHECK(f != NULL, "open output");
  CHECK(fwrite(hy, 2, (size_t)(M * N), f) == (size_t)(M * N), "write Y");
  fclose(f);
  hipFree(x);
  hipFree(w);
  hipFree(wq);
  hipFree(ws);
  hipFree(aq);
  hipFree(as);
  hipFree(y);
  if (work) hipFree(work);
  free(hx);
  free(hw);
  free(hy);
  free(hy2);
  printf("gpu ok: fmt %d, M %lld N %lld K %lld, eager run and 2 graph replays\n", fmt, (long long)M,
         (long long)N, (long long)K);
  return 0;
}

int main(int argc, char** argv) {
  if (argc == 3 && strcmp(argv[1], "host") == 0) return host_mode(argv[2]);
  if (argc == 4 && strcmp(argv[1], "gpu") == 0) return gpu_mode(argv[2], argv[3]);
  fprintf(stderr, "usage: %s host <table> | gpu <in.bin> <out.bin>\n", argv[0]);
  return 2;
}
