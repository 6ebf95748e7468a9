// C ABI of libmscan: host-side validation, workspace sizing and dispatch.
// Every check runs before any HIP call; nothing is enqueued on an error.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "mscan.h"
#include "mscan_device.hpp"
#include "mscan_launch.hpp"

namespace {

thread_local char g_last_hip_error[256] = "";

mscan_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MSCAN_OK;
  strncpy(g_last_hip_error, hipGetErrorString(e), sizeof(g_last_hip_error) - 1);
  g_last_hip_error[sizeof(g_last_hip_error) - 1] = '\0';
  return MSCAN_ERR_HIP;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Problem shape checks shared by every op.
mscan_status check_problem(const mscan_problem* p) {
  if (!p) return MSCAN_ERR_INVALID;
  if (p->rows < 1 || p->T < 1 || p->row_stride < p->T) return MSCAN_ERR_INVALID;
  if (p->T > (int64_t)INT32_MAX) return MSCAN_ERR_INVALID;  // cu_seqlens offsets are int32
  if (p->nseg < 1) return MSCAN_ERR_INVALID;
  if (!p->cu_seqlens && p->nseg != 1) return MSCAN_ERR_INVALID;
  if (p->cu_seqlens && ((uintptr_t)p->cu_seqlens & 3u)) return MSCAN_ERR_INVALID;
  if (p->reverse != 0 && p->reverse != 1) return MSCAN_ERR_INVALID;
  return MSCAN_OK;
}

// Tiles per row of the linear scalar kernels for one input type.
int64_t scalar_tiles_for(const mscan_problem* p, int in_dtype) {
  return mscan::scalar_tiles(p->T, p->row_stride, mscan::scalar_vec(in_dtype),
                             mscan::scalar_tile_elems(in_dtype, p->T));
}
// Tiles per row of the log-space kernels (forward and backward).
int64_t log_tiles_for(const mscan_problem* p) {
  return mscan::scalar_tiles(p->T, p->row_stride, 4, mscan::log_tile_elems(p->T));
}

enum class ScalarOp { Linear, LinearF32, Log };

// Workspace for a scalar-layout op: header, then (only when rows are chained by
// look-back) `words` descriptor words per tile (3 for the linear scan, 5 for
// the log-space scan). Linear: every input type (the size does not depend on
// the call's dtype); LinearF32: fp32 inputs only.
size_t scalar_ws_bytes(const mscan_problem* p, int words, ScalarOp op) {
  int64_t nt = 0;
  if (op == ScalarOp::Log) {
    const int64_t n = log_tiles_for(p);
    if (mscan::scalar_uses_lookback(p->rows, n)) nt = n;
  } else {
    for (int dt = MSCAN_F32; dt <= (op == ScalarOp::LinearF32 ? MSCAN_F32 : MSCAN_F16); ++dt) {
      const int64_t n = scalar_tiles_for(p, dt);
      if (mscan::scalar_uses_lookback(p->rows, n) && n > nt) nt = n;
    }
  }
  if (nt == 0) return mscan::kWsHeaderBytes;
  return mscan::ws_desc_offset() + (size_t)p->rows * (size_t)nt * (size_t)words * sizeof(uint64_t);
}

// A launch's grid counts work-items in 32 bits: with up to 256 threads per
// workgroup, at most 2^24 - 1 workgroups. (Every problem whose arrays fit in
// HBM stays far below that.)
mscan_status check_grid(const mscan_problem* p, int64_t tiles_per_row) {
  const double blocks = (double)p->rows * (double)tiles_per_row;
  if (blocks * 256.0 > 4294967295.0) return MSCAN_ERR_UNSUPPORTED;
  return MSCAN_OK;
}

// Workspace of a matrix op: header, then (look-back only) k*k + 2*k*v
// descriptor words per tile.
size_t matrix_ws_bytes(const mscan_problem* p, int k, int v) {
  if (mscan::matrix_core_shape(k, v)) return mscan::matrix_core_ws_bytes(p->rows, p->T, k, v);
  int64_t nt = 0;
  for (int b = 0; b < 2; ++b) {
    const int64_t n = mscan::matrix_tiles(p->T, k, v, b == 1);
    if (mscan::scalar_uses_lookback(p->rows, n) && n > nt) nt = n;
  }
  if (nt == 0) return mscan::kWsHeaderBytes;
  return mscan::ws_desc_offset() + (size_t)p->rows * (size_t)nt * (size_t)(k * k + 2 * k * v) * sizeof(uint64_t);
}

// The envelope k, v in {1, 2, 4, 8, 16}: (1, 1) is the scalar scan, four small
// shapes have VALU kernels, the rest run on the matrix cores.
bool matrix_shape_ok(int k, int v) {
  return (k == 1 && v == 1) || mscan::matrix_valu_shape(k, v) || mscan::matrix_core_shape(k, v);
}

// Whether a matrix call chains its row through the workspace (the matrix-core
// path always does).
bool matrix_needs_ws(const mscan_problem* p, int k, int v, int64_t nt) {
  return mscan::matrix_core_shape(k, v) || mscan::scalar_uses_lookback(p->rows, nt);
}

}  // namespace

extern "C" {

size_t mscan_workspace_bytes(const mscan_problem* prob, int op, int k, int v) {
  if (check_problem(prob) != MSCAN_OK) return 0;
  switch (op) {
    case MSCAN_OP_SCAN_FWD:
    case MSCAN_OP_SCAN_BWD:
      return scalar_ws_bytes(prob, 3, ScalarOp::Linear);
    case MSCAN_OP_SCAN_LOG_FWD:
      return scalar_ws_bytes(prob, 5, ScalarOp::Log);
    case MSCAN_OP_SCAN_LOG_BWD:
      return scalar_ws_bytes(prob, 3, ScalarOp::Log);
    case MSCAN_OP_MATRIX_FWD:
    case MSCAN_OP_MATRIX_BWD:
      if (!matrix_shape_ok(k, v)) return 0;
      if (k == 1 && v == 1) return scalar_ws_bytes(prob, 3, ScalarOp::LinearF32);
      return matrix_ws_bytes(prob, k, v);
    default:
      return 0;
  }
}

mscan_status mscan_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (!ws || !aligned16(ws) || ws_bytes < mscan::kWsHeaderBytes) return MSCAN_ERR_INVALID;
  return hip_status(mscan::launch_zero(ws, ws_bytes, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// gate: MSCAN_GATE_NONE (g holds gates) or MSCAN_GATE_SIGMOID (g holds logits)
mscan_status scalar_fwd_impl(const mscan_problem* prob, int in_dtype, int gate, const void* g, const void* x,
                             const float* h0, float* h, void* ws, size_t ws_bytes, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (in_dtype != MSCAN_F32 && in_dtype != MSCAN_BF16 && in_dtype != MSCAN_F16) return MSCAN_ERR_UNSUPPORTED;
  if (!g || !x || !h) return MSCAN_ERR_INVALID;
  if (!aligned16(g) || !aligned16(x) || !aligned16(h) || (h0 && ((uintptr_t)h0 & 3u))) return MSCAN_ERR_INVALID;
  const int64_t nt = scalar_tiles_for(prob, in_dtype);
  if ((s = check_grid(prob, nt)) != MSCAN_OK) return s;
  if (mscan::scalar_uses_lookback(prob->rows, nt) && (!ws || !aligned16(ws) || ws_bytes < scalar_ws_bytes(prob, 3, ScalarOp::Linear)))
    return MSCAN_ERR_WORKSPACE;
  mscan::ScalarArgs a{};
  a.g = g;
  a.b = x;
  a.h0 = h0;
  a.out0 = h;
  a.cu = prob->cu_seqlens;
  a.nseg = prob->nseg;
  a.rev = prob->reverse;
  a.rows = prob->rows;
  a.T = prob->T;
  a.stride = prob->row_stride;
  a.ws = ws;
  return hip_status(gate == MSCAN_GATE_SIGMOID ? mscan::launch_scalar_sigmoid(a, in_dtype, false, (hipStream_t)stream)
                                               : mscan::launch_scalar(a, in_dtype, false, (hipStream_t)stream));
}

mscan_status scalar_bwd_impl(const mscan_problem* prob, int in_dtype, int gate, const void* g, const float* h,
                             const float* dy, const float* h0, float* dx, float* dg, float* dh0, void* ws,
                             size_t ws_bytes, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (in_dtype != MSCAN_F32 && in_dtype != MSCAN_BF16 && in_dtype != MSCAN_F16) return MSCAN_ERR_UNSUPPORTED;
  if (!g || !h || !dy || !dx || !dg) return MSCAN_ERR_INVALID;
  if (!aligned16(g) || !aligned16(h) || !aligned16(dy) || !aligned16(dx) || !aligned16(dg))
    return MSCAN_ERR_INVALID;
  if ((h0 && ((uintptr_t)h0 & 3u)) || (dh0 && ((uintptr_t)dh0 & 3u))) return MSCAN_ERR_INVALID;
  const int64_t nt = scalar_tiles_for(prob, in_dtype);
  if ((s = check_grid(prob, nt)) != MSCAN_OK) return s;
  if (mscan::scalar_uses_lookback(prob->rows, nt) && (!ws || !aligned16(ws) || ws_bytes < scalar_ws_bytes(prob, 3, ScalarOp::Linear)))
    return MSCAN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (dh0 && prob->cu_seqlens) {
    // empty sequences have no element to write their (zero) gradient
    const mscan_status z = hip_status(mscan::launch_zero(dh0, (size_t)prob->nseg * (size_t)prob->rows * 4u, st));
    if (z != MSCAN_OK) return z;
  }
  mscan::ScalarArgs a{};
  a.g = g;
  a.b = dy;
  a.hs = h;
  a.h0 = h0;
  a.out0 = dx;
  a.out1 = dg;
  a.dh0 = dh0;
  a.cu = prob->cu_seqlens;
  a.nseg = prob->nseg;
  a.rev = prob->reverse ? 0 : 1;  // the adjoint runs against the forward's order
  a.rows = prob->rows;
  a.T = prob->T;
  a.stride = prob->row_stride;
  a.ws = ws;
  return hip_status(gate == MSCAN_GATE_SIGMOID ? mscan::launch_scalar_sigmoid(a, in_dtype, true, st)
                                               : mscan::launch_scalar(a, in_dtype, true, st));
}

// gate: MSCAN_GATE_NONE (log_a holds log a) or MSCAN_GATE_NEG_SOFTPLUS (logits)
mscan_status log_fwd_impl(const mscan_problem* prob, int gate, const float* log_a, const float* log_b,
                          const float* log_h0, float* h, void* ws, size_t ws_bytes, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (!log_a || !log_b || !h) return MSCAN_ERR_INVALID;
  if (!aligned16(log_a) || !aligned16(log_b) || !aligned16(h) || (log_h0 && ((uintptr_t)log_h0 & 3u)))
    return MSCAN_ERR_INVALID;
  const int64_t nt = log_tiles_for(prob);
  if ((s = check_grid(prob, nt)) != MSCAN_OK) return s;
  if (mscan::scalar_uses_lookback(prob->rows, nt) && (!ws || !aligned16(ws) || ws_bytes < scalar_ws_bytes(prob, 5, ScalarOp::Log)))
    return MSCAN_ERR_WORKSPACE;
  mscan::ScalarArgs a{};
  a.g = log_a;
  a.b = log_b;
  a.h0 = log_h0;
  a.out0 = h;
  a.cu = prob->cu_seqlens;
  a.nseg = prob->nseg;
  a.rev = prob->reverse;
  a.rows = prob->rows;
  a.T = prob->T;
  a.stride = prob->row_stride;
  a.ws = ws;
  return hip_status(gate == MSCAN_GATE_NEG_SOFTPLUS ? mscan::launch_log_softplus(a, false, (hipStream_t)stream)
                                                    : mscan::launch_log(a, (hipStream_t)stream));
}

mscan_status log_bwd_impl(const mscan_problem* prob, int gate, const float* log_a, const float* log_b,
                          const float* h, const float* dy, const float* log_h0, float* dlog_a, float* dlog_b,
                          float* dlog_h0, void* ws, size_t ws_bytes, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (!log_a || !log_b || !h || !dy || !dlog_a || !dlog_b) return MSCAN_ERR_INVALID;
  if (!aligned16(log_a) || !aligned16(log_b) || !aligned16(h) || !aligned16(dy) || !aligned16(dlog_a) ||
      !aligned16(dlog_b))
    return MSCAN_ERR_INVALID;
  if ((log_h0 && ((uintptr_t)log_h0 & 3u)) || (dlog_h0 && ((uintptr_t)dlog_h0 & 3u))) return MSCAN_ERR_INVALID;
  const int64_t nt = log_tiles_for(prob);
  if ((s = check_grid(prob, nt)) != MSCAN_OK) return s;
  if (mscan::scalar_uses_lookback(prob->rows, nt) && (!ws || !aligned16(ws) || ws_bytes < scalar_ws_bytes(prob, 3, ScalarOp::Log)))
    return MSCAN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (dlog_h0 && prob->cu_seqlens) {
    // empty sequences have no element to write their (zero) gradient
    const mscan_status z = hip_status(mscan::launch_zero(dlog_h0, (size_t)prob->nseg * (size_t)prob->rows * 4u, st));
    if (z != MSCAN_OK) return z;
  }
  mscan::ScalarArgs a{};
  a.g = log_a;
  a.lb = log_b;
  a.b = dy;
  a.hs = h;
  a.h0 = log_h0;
  a.out0 = dlog_b;
  a.out1 = dlog_a;
  a.dh0 = dlog_h0;
  a.cu = prob->cu_seqlens;
  a.nseg = prob->nseg;
  a.rev = prob->reverse ? 0 : 1;  // the adjoint runs against the forward's order
  a.rows = prob->rows;
  a.T = prob->T;
  a.stride = prob->row_stride;
  a.ws = ws;
  return hip_status(gate == MSCAN_GATE_NEG_SOFTPLUS ? mscan::launch_log_softplus(a, true, st)
                                                    : mscan::launch_log_bwd(a, st));
}

}  // namespace

extern "C" {

mscan_status scan_fwd(const mscan_problem* prob, int in_dtype, const void* g, const void* x,
                      const float* h0, float* h, void* ws, size_t ws_bytes, void* stream) {
  return scalar_fwd_impl(prob, in_dtype, MSCAN_GATE_NONE, g, x, h0, h, ws, ws_bytes, stream);
}

mscan_status scan_bwd(const mscan_problem* prob, int in_dtype, const void* g, const float* h,
                      const float* dy, const float* h0, float* dx, float* dg, float* dh0, void* ws,
                      size_t ws_bytes, void* stream) {
  return scalar_bwd_impl(prob, in_dtype, MSCAN_GATE_NONE, g, h, dy, h0, dx, dg, dh0, ws, ws_bytes, stream);
}

mscan_status scan_log_fwd(const mscan_problem* prob, const float* log_a, const float* log_b,
                          const float* log_h0, float* h, void* ws, size_t ws_bytes, void* stream) {
  return log_fwd_impl(prob, MSCAN_GATE_NONE, log_a, log_b, log_h0, h, ws, ws_bytes, stream);
}

mscan_status scan_log_bwd(const mscan_problem* prob, const float* log_a, const float* log_b, const float* h,
                          const float* dy, const float* log_h0, float* dlog_a, float* dlog_b, float* dlog_h0,
                          void* ws, size_t ws_bytes, void* stream) {
  return log_bwd_impl(prob, MSCAN_GATE_NONE, log_a, log_b, h, dy, log_h0, dlog_a, dlog_b, dlog_h0, ws, ws_bytes,
                      stream);
}

mscan_status scan_fwd_gated(const mscan_problem* prob, int in_dtype, int gate, const void* z, const void* x,
                            const float* h0, float* h, void* ws, size_t ws_bytes, void* stream) {
  if (gate != MSCAN_GATE_SIGMOID) return MSCAN_ERR_UNSUPPORTED;
  return scalar_fwd_impl(prob, in_dtype, gate, z, x, h0, h, ws, ws_bytes, stream);
}

mscan_status scan_bwd_gated(const mscan_problem* prob, int in_dtype, int gate, const void* z, const float* h,
                            const float* dy, const float* h0, float* dx, float* dz, float* dh0, void* ws,
                            size_t ws_bytes, void* stream) {
  if (gate != MSCAN_GATE_SIGMOID) return MSCAN_ERR_UNSUPPORTED;
  return scalar_bwd_impl(prob, in_dtype, gate, z, h, dy, h0, dx, dz, dh0, ws, ws_bytes, stream);
}

mscan_status scan_log_fwd_gated(const mscan_problem* prob, int gate, const float* z, const float* log_b,
                                const float* log_h0, float* h, void* ws, size_t ws_bytes, void* stream) {
  if (gate != MSCAN_GATE_NEG_SOFTPLUS) return MSCAN_ERR_UNSUPPORTED;
  return log_fwd_impl(prob, gate, z, log_b, log_h0, h, ws, ws_bytes, stream);
}

mscan_status scan_log_bwd_gated(const mscan_problem* prob, int gate, const float* z, const float* log_b,
                                const float* h, const float* dy, const float* log_h0, float* dz, float* dlog_b,
                                float* dlog_h0, void* ws, size_t ws_bytes, void* stream) {
  if (gate != MSCAN_GATE_NEG_SOFTPLUS) return MSCAN_ERR_UNSUPPORTED;
  return log_bwd_impl(prob, gate, z, log_b, h, dy, log_h0, dz, dlog_b, dlog_h0, ws, ws_bytes, stream);
}

mscan_status matrix_affine_scan_fwd(const mscan_problem* prob, int k, int v, const float* A,
                                    const float* B, const float* h0, float* h, void* ws,
                                    size_t ws_bytes, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (!matrix_shape_ok(k, v)) return MSCAN_ERR_UNSUPPORTED;
  if (k == 1 && v == 1) return scan_fwd(prob, MSCAN_F32, A, B, h0, h, ws, ws_bytes, stream);  // the scalar scan
  if (!A || !B || !h) return MSCAN_ERR_INVALID;
  if (!aligned16(A) || !aligned16(B) || !aligned16(h) || (h0 && !aligned16(h0))) return MSCAN_ERR_INVALID;
  const int64_t nt = mscan::matrix_tiles(prob->T, k, v, false);
  if ((s = check_grid(prob, nt)) != MSCAN_OK) return s;
  if (matrix_needs_ws(prob, k, v, nt) && (!ws || !aligned16(ws) || ws_bytes < matrix_ws_bytes(prob, k, v)))
    return MSCAN_ERR_WORKSPACE;
  mscan::MatArgs a{};
  a.A = A;
  a.B = B;
  a.h0 = h0;
  a.out0 = h;
  a.cu = prob->cu_seqlens;
  a.nseg = prob->nseg;
  a.rev = prob->reverse;
  a.rows = prob->rows;
  a.T = prob->T;
  a.stride = prob->row_stride;
  a.ws = ws;
  return hip_status(mscan::launch_matrix(a, k, v, false, (hipStream_t)stream));
}

mscan_status matrix_affine_scan_bwd(const mscan_problem* prob, int k, int v, const float* A,
                                    const float* h, const float* dy, const float* h0, float* dA,
                                    float* dB, float* dh0, void* ws, size_t ws_bytes, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (!matrix_shape_ok(k, v)) return MSCAN_ERR_UNSUPPORTED;
  if (k == 1 && v == 1) return scan_bwd(prob, MSCAN_F32, A, h, dy, h0, dB, dA, dh0, ws, ws_bytes, stream);
  if (!A || !h || !dy || !dA || !dB) return MSCAN_ERR_INVALID;
  if (!aligned16(A) || !aligned16(h) || !aligned16(dy) || !aligned16(dA) || !aligned16(dB)) return MSCAN_ERR_INVALID;
  if ((h0 && !aligned16(h0)) || (dh0 && ((uintptr_t)dh0 & 3u))) return MSCAN_ERR_INVALID;
  const int64_t nt = mscan::matrix_tiles(prob->T, k, v, true);
  if ((s = check_grid(prob, nt)) != MSCAN_OK) return s;
  if (matrix_needs_ws(prob, k, v, nt) && (!ws || !aligned16(ws) || ws_bytes < matrix_ws_bytes(prob, k, v)))
    return MSCAN_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (dh0 && prob->cu_seqlens) {
    const mscan_status z = hip_status(
        mscan::launch_zero(dh0, (size_t)prob->nseg * (size_t)prob->rows * (size_t)(k * v) * 4u, st));
    if (z != MSCAN_OK) return z;
  }
  mscan::MatArgs a{};
  a.A = A;
  a.B = dy;
  a.hs = h;
  a.h0 = h0;
  a.out0 = dB;
  a.out1 = dA;
  a.dh0 = dh0;
  a.cu = prob->cu_seqlens;
  a.nseg = prob->nseg;
  a.rev = prob->reverse ? 0 : 1;  // the adjoint runs against the forward's order
  a.rows = prob->rows;
  a.T = prob->T;
  a.stride = prob->row_stride;
  a.ws = ws;
  return hip_status(mscan::launch_matrix(a, k, v, true, st));
}

// ---------------------------------------------------------------------------
// scan_fwd_noalloc: scan_fwd with its look-back descriptors in a fixed array
// the library owns on each device, for callers that cannot allocate.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

// The fixed scratch array. Each device holds its own copy from the moment the
// library's code is loaded on it until the process ends. Host code must not
// use the name as an address (on the host it is only a stand-in for the
// symbol); every use goes through the per-device address resolved below.
static_assert(MSCAN_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) uint8_t scratch[MSCAN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device, resolved once per device
// (hipGetSymbolAddress with that device current) and cached.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

extern "C" {

mscan_status scan_fwd_noalloc(const mscan_problem* prob, int in_dtype, const void* g, const void* x,
                              const float* h0, float* h, void* stream) {
  // every host-side check of scan_fwd first (nothing is resolved or enqueued
  // for an invalid call), then the scratch size
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (in_dtype != MSCAN_F32 && in_dtype != MSCAN_BF16 && in_dtype != MSCAN_F16) return MSCAN_ERR_UNSUPPORTED;
  if (!g || !x || !h) return MSCAN_ERR_INVALID;
  if (!aligned16(g) || !aligned16(x) || !aligned16(h) || (h0 && ((uintptr_t)h0 & 3u))) return MSCAN_ERR_INVALID;
  if ((s = check_grid(prob, scalar_tiles_for(prob, in_dtype))) != MSCAN_OK) return s;
  if (scalar_ws_bytes(prob, 3, ScalarOp::Linear) > (size_t)MSCAN_NOALLOC_SCRATCH_BYTES) return MSCAN_ERR_WORKSPACE;
  void* ws = nullptr;
  const mscan_status r = hip_status(scratch_on_current_device(&ws));
  if (r != MSCAN_OK) return r;
  return scalar_fwd_impl(prob, in_dtype, MSCAN_GATE_NONE, g, x, h0, h, ws, MSCAN_NOALLOC_SCRATCH_BYTES, stream);
}

mscan_status mscan_stream_ceiling(const float* const* src, int nsrc, float* const* dst, int ndst, size_t n,
                                  void* stream) {
  if (!src || !dst || nsrc < 1 || nsrc > 4 || ndst < 1 || ndst > 3 || n == 0 || (n & 3u)) return MSCAN_ERR_INVALID;
  for (int i = 0; i < nsrc; ++i)
    if (!src[i] || !aligned16(src[i])) return MSCAN_ERR_INVALID;
  for (int i = 0; i < ndst; ++i)
    if (!dst[i] || !aligned16(dst[i])) return MSCAN_ERR_INVALID;
  const bool mix = (nsrc == 1 && ndst == 1) || (nsrc == 2 && ndst == 1) || (nsrc == 3 && ndst == 1) ||
                   (nsrc == 1 && ndst == 2) || (nsrc == 2 && ndst == 2) || (nsrc == 3 && ndst == 2) ||
                   (nsrc == 4 && ndst == 2) || (nsrc == 4 && ndst == 3);
  if (!mix) return MSCAN_ERR_UNSUPPORTED;
  return hip_status(mscan::launch_stream(src, nsrc, dst, ndst, n / 4, (hipStream_t)stream));
}

mscan_status mscan_workspace_error(const void* ws, size_t ws_bytes, int32_t* flag_out, void* stream) {
  if (!ws || !aligned16(ws) || ws_bytes < mscan::kWsHeaderBytes || !flag_out || ((uintptr_t)flag_out & 3u))
    return MSCAN_ERR_INVALID;
  return hip_status(mscan::launch_read_error(ws, flag_out, (hipStream_t)stream));
}

mscan_status mscan_debug_partial_fwd(const mscan_problem* prob, int k, int v, const float* a, const float* b,
                                     float* out, void* ws, size_t ws_bytes, int64_t first_block, int64_t nblocks,
                                     uint32_t spin_limit, void* stream) {
  mscan_status s = check_problem(prob);
  if (s != MSCAN_OK) return s;
  if (!matrix_shape_ok(k, v)) return MSCAN_ERR_UNSUPPORTED;
  if (!a || !b || !out || !aligned16(a) || !aligned16(b) || !aligned16(out)) return MSCAN_ERR_INVALID;
  if (!ws || !aligned16(ws)) return MSCAN_ERR_WORKSPACE;
  // the call's grid, which must chain tiles (else there is no wait to run out)
  const bool scalar = k == 1 && v == 1;
  int64_t per_row = 0;
  bool chained = false;
  size_t need = 0;
  if (scalar) {
    per_row = scalar_tiles_for(prob, MSCAN_F32);
    chained = !mscan::scalar_short_rows(prob->T, prob->row_stride) && mscan::scalar_uses_lookback(prob->rows, per_row);
    need = scalar_ws_bytes(prob, 3, ScalarOp::Linear);
  } else if (mscan::matrix_core_shape(k, v)) {
    per_row = mscan::matrix_core_chunks(prob->T, false, k, v);
    chained = true;
    need = matrix_ws_bytes(prob, k, v);
  } else {
    per_row = mscan::matrix_tiles(prob->T, k, v, false);
    chained = mscan::scalar_uses_lookback(prob->rows, per_row);
    need = matrix_ws_bytes(prob, k, v);
  }
  if (!chained) return MSCAN_ERR_UNSUPPORTED;
  if ((s = check_grid(prob, per_row)) != MSCAN_OK) return s;
  if (ws_bytes < need) return MSCAN_ERR_WORKSPACE;
  const int64_t total = prob->rows * per_row;
  if (first_block < 0 || nblocks < 1 || first_block + nblocks > total) return MSCAN_ERR_INVALID;
  hipStream_t st = (hipStream_t)stream;
  if (scalar) {
    mscan::ScalarArgs sa{};
    sa.g = a;
    sa.b = b;
    sa.out0 = out;
    sa.cu = prob->cu_seqlens;
    sa.nseg = prob->nseg;
    sa.rev = prob->reverse;
    sa.rows = prob->rows;
    sa.T = prob->T;
    sa.stride = prob->row_stride;
    sa.ws = ws;
    sa.blk0 = (uint32_t)first_block;
    sa.nblk = (uint32_t)nblocks;
    sa.spin = spin_limit;
    return hip_status(mscan::launch_scalar(sa, MSCAN_F32, false, st));
  }
  mscan::MatArgs ma{};
  ma.A = a;
  ma.B = b;
  ma.out0 = out;
  ma.cu = prob->cu_seqlens;
  ma.nseg = prob->nseg;
  ma.rev = prob->reverse;
  ma.rows = prob->rows;
  ma.T = prob->T;
  ma.stride = prob->row_stride;
  ma.ws = ws;
  ma.blk0 = (uint32_t)first_block;
  ma.nblk = (uint32_t)nblocks;
  ma.spin = spin_limit;
  return hip_status(mscan::launch_matrix(ma, k, v, false, st));
}

const char* mscan_status_string(int status) {
  switch (status) {
    case MSCAN_OK: return "ok";
    case MSCAN_ERR_INVALID: return "invalid argument";
    case MSCAN_ERR_UNSUPPORTED: return "unsupported configuration";
    case MSCAN_ERR_WORKSPACE: return "workspace missing or too small";
    case MSCAN_ERR_HIP: return "HIP launch error";
    case MSCAN_ERR_TIMEOUT: return "a look-back wait gave up (outputs that needed the missing carry are NaN)";
    default: return "unknown status";
  }
}

const char* mscan_last_hip_error(void) { return g_last_hip_error; }

int mscan_abi_version(void) { return MSCAN_ABI_VERSION; }

}  // extern "C"
