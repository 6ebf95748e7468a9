// Private interface between the C ABI (mscan_api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

// Arguments of the scalar forward / backward kernels (see scan_scalar.hip).
struct ScalarArgs {
  const void* g;        // gates, fp32 or bf16
  const void* b;        // forward: x (same type as g); backward: dy (fp32)
  const float* lb;      // log-space backward: log b (the gate g is log a)
  const float* hs;      // backward: forward states h
  const float* h0;      // [nseg][rows] or null
  float* out0;          // forward: h; backward: dx
  float* out1;          // backward: dg
  float* dh0;           // backward: [nseg][rows] or null
  const int32_t* cu;    // cu_seqlens or null
  int32_t nseg;
  int32_t rev;          // processing order runs from high t to low t
  int64_t rows, T, stride;
  int32_t ntiles;       // tiles per row (set by the launcher)
  void* ws;             // workspace (only used when ntiles > 1)
  // partial launches (a test hook; 0 in every normal call): run blocks
  // [blk0, blk0 + nblk) of the call's grid, with look-back waits giving up
  // after `spin` polls (0 = the default limit)
  uint32_t blk0, nblk, spin;
};

// Elements per tile of the scalar kernels, and tiles per row for a given T.
bool scalar_wide_tile(int in_dtype, int64_t T);       // linear scan: one 8192-element tile
int64_t scalar_tile_elems(int in_dtype, int64_t T);    // linear scans
bool log_wide_tile(int64_t T);                         // log-space scan: one 8192-element tile
int64_t log_tile_elems(int64_t T);                     // log-space scans
int64_t scalar_tiles(int64_t T, int64_t stride, int vec, int64_t tile);
int scalar_vec(int in_dtype);
// Whether a scalar call chains the tiles of a row by look-back (few long rows).
bool scalar_uses_lookback(int64_t rows, int64_t ntiles);
// rows that fit one tile of at most 2048 elements: a smaller workgroup per row
bool scalar_short_rows(int64_t T, int64_t stride);
hipError_t launch_scalar_short(const ScalarArgs& a, int in_dtype, int gate, bool bwd, hipStream_t st);
hipError_t launch_log_short(const ScalarArgs& a, int gate, bool bwd, hipStream_t st);
hipError_t launch_scalar(const ScalarArgs& a, int in_dtype, bool bwd, hipStream_t st);
// Log-space forward (g = log a, b = log b, h0 = log h0; fp32).
hipError_t launch_log(const ScalarArgs& a, hipStream_t st);
// Log-space backward (g = log a, lb = log b, b = dy, hs = h, h0 = log h0;
// out0 = dlog_b, out1 = dlog_a, dh0 = dlog_h0; fp32).
hipError_t launch_log_bwd(const ScalarArgs& a, hipStream_t st);
// Gate-logit variants: linear scan with g = sigmoid(z); log-space scan with
// log a = -softplus(z) (g holds z; the backward's out1 is dz).
hipError_t launch_scalar_sigmoid(const ScalarArgs& a, int in_dtype, bool bwd, hipStream_t st);
hipError_t launch_log_softplus(const ScalarArgs& a, bool bwd, hipStream_t st);

// Arguments of the matrix-affine kernels (see scan_matrix.hip). Strides and
// offsets count time steps; a step holds a k x k block of A and k x v blocks
// of B / h / dy.
struct MatArgs {
  const float* A;       // transitions [rows][T][k][k]
  const float* B;       // forward: injections B; backward: dy  ([rows][T][k][v])
  const float* hs;      // backward: forward states h
  const float* h0;      // [nseg][rows][k][v] or null
  float* out0;          // forward: h; backward: dB
  float* out1;          // backward: dA
  float* dh0;           // backward: [nseg][rows][k][v] or null
  const int32_t* cu;
  int32_t nseg;
  int32_t rev;          // processing order runs from high t to low t
  int64_t rows, T, stride;
  int32_t ntiles;
  void* ws;
  int32_t k, v;         // block sizes (read by the matrix-core kernels; the
                        // VALU kernels take them as template parameters)
  uint32_t blk0, nblk, spin;  // partial launches, as for ScalarArgs
};

// Grid of a chained call: the whole grid, or the part a partial launch asks for.
inline unsigned launch_blocks(uint64_t total, uint32_t nblk) { return (unsigned)(nblk ? nblk : total); }

// (k, v) served by the VALU kernels (scan_matrix.hip): (2,1), (2,2), (4,1).
bool matrix_valu_shape(int k, int v);
// (k, v) served by the matrix-core kernels (scan_matrix_cores.hip): every
// other pair of the envelope k, v in {1, 2, 4, 8, 16} except (1, 1), the
// scalar scan.
bool matrix_core_shape(int k, int v);
// Tiles per row of the matrix kernels for (k, v) (0 if unsupported).
int64_t matrix_tiles(int64_t T, int k, int v, bool bwd);
hipError_t launch_matrix(const MatArgs& a, int k, int v, bool bwd, hipStream_t st);
// Matrix-core kernels, blocks zero-padded to 4 x 4 (k, v <= 4) or 16 x 16:
// chunks per row, the workspace a call needs (always), and the launch
// (a.k, a.v in 1..16).
int64_t matrix_core_chunks(int64_t T, bool bwd, int k, int v);
size_t matrix_core_ws_bytes(int64_t rows, int64_t T, int k, int v);
hipError_t launch_matrix_core(const MatArgs& a, bool bwd, hipStream_t st);

// Fill n floats (or bytes / 4 words) with zero on `st` (no hipMemsetAsync, so
// callers may capture it in a graph).
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

// Workspace header bytes (control words) ahead of the per-tile descriptors,
// and the header word a kernel sets when one of its waits gives up.
constexpr size_t kWsHeaderBytes = 128;
constexpr int kHdrErrorWord = 3;
// Copy the error word as an mscan status (0 or 5) to *dst, on `st`.
hipError_t launch_read_error(const void* ws, int32_t* dst, hipStream_t st);
// Streaming diagnostic: read nsrc arrays, write ndst arrays of n4 16-byte
// units each ((nsrc, ndst) in {(1,1), (2,1), (3,1), (1,2), (2,2), (3,2),
// (4,2), (4,3)}).
hipError_t launch_stream(const float* const* src, int nsrc, float* const* dst, int ndst, size_t n4, hipStream_t st);

}  // namespace mscan
