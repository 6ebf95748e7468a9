// Host-side argument validation of libmscan under AddressSanitizer and
// UndefinedBehaviorSanitizer. Built by tests/test_host_sanitizers.py from the
// library's own sources, with the host code instrumented and the device code
// built as usual. Every call below is refused on the host before any HIP call
// (no GPU is needed or touched); the driver checks each returned status and
// the sanitizers check every host access the validation makes.
#include <stdint.h>
#include <stdio.h>

#include "mscan.h"

static int g_fail = 0;
static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
    g_fail = 1;
  }
}

int main() {
  float* F = (float*)(uintptr_t)(1u << 20);  // aligned, never dereferenced
  void* V = (void*)F;
  const int32_t cu_host[3] = {0, 50, 100};  // only its address is checked on the host
  mscan_problem ok = {8, 100, 100, nullptr, 1, 0};

  // problem shapes
  mscan_problem bad[] = {
      {0, 100, 100, nullptr, 1, 0},   {8, 0, 0, nullptr, 1, 0},       {8, 100, 50, nullptr, 1, 0},
      {8, 100, 100, nullptr, 2, 0},   {8, 100, 100, nullptr, 1, 2},   {8, 100, 100, nullptr, 0, 0},
      {8, 1ll << 31, 1ll << 31, nullptr, 1, 0}, {8, 100, 100, (const int32_t*)((uintptr_t)cu_host + 1), 2, 0},
  };
  for (const mscan_problem& p : bad) {
    expect("scan_fwd bad problem", scan_fwd(&p, 0, V, V, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_INVALID);
    expect("scan_bwd bad problem", scan_bwd(&p, 0, V, F, F, nullptr, F, F, nullptr, nullptr, 0, nullptr),
           MSCAN_ERR_INVALID);
    expect("log fwd bad problem", scan_log_fwd(&p, F, F, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_INVALID);
    expect("matrix bad problem", matrix_affine_scan_fwd(&p, 4, 4, F, F, nullptr, F, V, 1 << 20, nullptr),
           MSCAN_ERR_INVALID);
    expect("noalloc bad problem", scan_fwd_noalloc(&p, 0, V, V, nullptr, F, nullptr), MSCAN_ERR_INVALID);
    expect("workspace bytes of a bad problem", (int)mscan_workspace_bytes(&p, MSCAN_OP_SCAN_FWD, 1, 1), 0);
  }
  expect("null problem", scan_fwd(nullptr, 0, V, V, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_INVALID);

  // pointers and dtypes
  expect("null g", scan_fwd(&ok, 0, nullptr, V, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_INVALID);
  expect("misaligned g", scan_fwd(&ok, 0, (char*)V + 4, V, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_INVALID);
  expect("misaligned h0", scan_fwd(&ok, 0, V, V, (float*)((char*)V + 2), F, nullptr, 0, nullptr), MSCAN_ERR_INVALID);
  expect("dtype", scan_fwd(&ok, 7, V, V, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_UNSUPPORTED);
  expect("bwd null dx", scan_bwd(&ok, 0, V, F, F, nullptr, nullptr, F, nullptr, nullptr, 0, nullptr),
         MSCAN_ERR_INVALID);
  expect("bwd misaligned dh0", scan_bwd(&ok, 0, V, F, F, nullptr, F, F, (float*)((char*)V + 1), nullptr, 0, nullptr),
         MSCAN_ERR_INVALID);
  expect("log bwd null log_b",
         scan_log_bwd(&ok, F, nullptr, F, F, nullptr, F, F, nullptr, nullptr, 0, nullptr), MSCAN_ERR_INVALID);

  // workspaces
  mscan_problem longp = {4, 20000, 20000, nullptr, 1, 0};
  const size_t need = mscan_workspace_bytes(&longp, MSCAN_OP_SCAN_FWD, 1, 1);
  expect("workspace needed", need > 128, 1);
  expect("no workspace", scan_fwd(&longp, 0, V, V, nullptr, F, nullptr, 0, nullptr), MSCAN_ERR_WORKSPACE);
  expect("small workspace", scan_fwd(&longp, 0, V, V, nullptr, F, V, need - 8, nullptr), MSCAN_ERR_WORKSPACE);
  mscan_problem huge = {12288, 1 << 20, 1 << 20, nullptr, 1, 0};
  expect("noalloc beyond its scratch", scan_fwd_noalloc(&huge, 0, V, V, nullptr, F, nullptr), MSCAN_ERR_WORKSPACE);
  expect("matrix-core without workspace", matrix_affine_scan_fwd(&ok, 16, 16, F, F, nullptr, F, nullptr, 0, nullptr),
         MSCAN_ERR_WORKSPACE);

  // envelope and gates
  const int kvs[][2] = {{3, 3}, {16, 32}, {0, 1}, {4, 0}, {-2, 2}, {8, 6}};
  for (const auto& kv : kvs) {
    expect("outside the envelope", matrix_affine_scan_fwd(&ok, kv[0], kv[1], F, F, nullptr, F, V, 1 << 20, nullptr),
           MSCAN_ERR_UNSUPPORTED);
    expect("outside the envelope (bwd)",
           matrix_affine_scan_bwd(&ok, kv[0], kv[1], F, F, F, nullptr, F, F, nullptr, V, 1 << 20, nullptr),
           MSCAN_ERR_UNSUPPORTED);
  }
  expect("gate kind", scan_fwd_gated(&ok, 0, MSCAN_GATE_NEG_SOFTPLUS, V, V, nullptr, F, nullptr, 0, nullptr),
         MSCAN_ERR_UNSUPPORTED);
  expect("log gate kind", scan_log_fwd_gated(&ok, MSCAN_GATE_SIGMOID, F, F, nullptr, F, nullptr, 0, nullptr),
         MSCAN_ERR_UNSUPPORTED);
  mscan_problem grid = {1 << 20, 1 << 16, 1 << 16, nullptr, 1, 0};
  expect("grid beyond one launch", scan_fwd(&grid, 0, V, V, nullptr, F, V, (size_t)1 << 40, nullptr),
         MSCAN_ERR_UNSUPPORTED);

  // diagnostics and test hooks
  expect("error word: null ws", mscan_workspace_error(nullptr, 4096, (int32_t*)V, nullptr), MSCAN_ERR_INVALID);
  expect("error word: small ws", mscan_workspace_error(V, 64, (int32_t*)V, nullptr), MSCAN_ERR_INVALID);
  expect("partial launch: one tile per row",
         mscan_debug_partial_fwd(&ok, 1, 1, F, F, F, V, 1 << 30, 0, 1, 100, nullptr), MSCAN_ERR_UNSUPPORTED);
  mscan_problem three = {8, 3 * 4096, 3 * 4096, nullptr, 1, 0};
  expect("partial launch past the grid",
         mscan_debug_partial_fwd(&three, 1, 1, F, F, F, V, 1 << 30, 23, 2, 100, nullptr), MSCAN_ERR_INVALID);
  const float* srcs[2] = {F, F};
  float* dsts[1] = {F};
  expect("stream mix", mscan_stream_ceiling(srcs, 2, dsts, 1, 6, nullptr), MSCAN_ERR_INVALID);  // n % 4
  float* dsts3[3] = {F, nullptr, F};
  expect("stream null destination", mscan_stream_ceiling(srcs, 1, dsts3, 3, 8, nullptr), MSCAN_ERR_INVALID);
  expect("stream mix 1:3", mscan_stream_ceiling(srcs, 1, dsts, 4, 8, nullptr), MSCAN_ERR_INVALID);  // > 3 writes
  for (int s = 0; s <= 6; ++s) expect("status string", mscan_status_string(s) != nullptr, 1);
  expect("abi version", mscan_abi_version(), MSCAN_ABI_VERSION);

  if (!g_fail) printf("host checks ok\n");
  return g_fail;
}
