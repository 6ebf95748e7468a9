// Scalar affine scan: host dispatch over tile shapes and input types (the
// kernel and its decomposition are described in scan_scalar_kernel.hpp).
#include "scan_scalar_kernel.hpp"

namespace mscan {

// Tile shape of the linear scans, every input type: 4 waves x 4 sub-chunks x
// 64 lanes x 4 elements (rows of at most 2048 elements take the smaller
// one-per-row shapes of scan_scalar_short.hip instead). Rows of 4097 to 8191
// elements (8192 for 16-bit inputs) take one tile of 8 waves (8192 elements)
// instead of two chained ones (a second, mostly empty tile and its look-back
// cost more than the wider workgroup). 12288 rows, flushed forward /
// backward: fp32 T = 5000 151 -> 130 / 258 -> 235 us, T = 8000 209 -> 193 /
// 368 -> 349 us; bf16 T = 5000 155 -> 98 / 235 -> 228 us, T = 8000 192 -> 136 /
// 344 -> 316 us, T = 8192 138 -> 132 / 309 -> 302 us (fp32 at T = 8192: the
// forward 2% slower, so it keeps two tiles).
// (8192-element tiles for the packed bf16 forward, 16 tiles per row, measured
// within run-to-run noise.)
bool scalar_wide_tile(int in_dtype, int64_t T) { return T > 4096 && T <= (in_dtype == 0 ? 8191 : 8192); }
int64_t scalar_tile_elems(int in_dtype, int64_t T) { return scalar_wide_tile(in_dtype, T) ? 8192 : 4096; }
// The log-space kernels: 4096-element tiles, and one 8192-element tile of 8
// waves for rows of 4097 to 8192 elements (8192 rows of T = 8192, flushed:
// forward 137 -> 135 us, backward 274 -> 266 us, plus the look-back's
// descriptor fill saved).
bool log_wide_tile(int64_t T) { return T > 4096 && T <= 8192; }
int64_t log_tile_elems(int64_t T) { return log_wide_tile(T) ? 8192 : 4096; }
int scalar_vec(int) { return 4; }

int64_t scalar_tiles(int64_t T, int64_t stride, int vec, int64_t tile) {
  // padded row length: rows all start aligned when the stride is a multiple of
  // the vector width; otherwise allow for the worst misalignment
  const int64_t umax = (stride % vec == 0) ? (T + vec - 1) / vec * vec : ((T - 1 + vec - 1) / vec + 1) * vec;
  return (umax + tile - 1) / tile;
}

// One workgroup per tile, chained by look-back, whenever a row spans several
// tiles: measured faster than walking rows in one workgroup (more bytes in
// flight per CU), at every row count of the benchmark workloads.
bool scalar_uses_lookback(int64_t rows, int64_t ntiles) {
  (void)rows;
  return ntiles > 1;
}

template <int GATE>
static hipError_t launch_scalar_gate(const ScalarArgs& a, int in_dtype, bool bwd, hipStream_t st) {
  if (scalar_short_rows(a.T, a.stride)) return launch_scalar_short(a, in_dtype, GATE, bwd, st);
  const bool rev = a.rev != 0;
  if (scalar_wide_tile(in_dtype, a.T)) {
    if (in_dtype == 0) {
      if (bwd) return rev ? launch_cfg<LinOps, float, true, true, 8, 4, 1, false, GATE>(a, st)
                          : launch_cfg<LinOps, float, true, false, 8, 4, 1, false, GATE>(a, st);
      return rev ? launch_cfg<LinOps, float, false, true, 8, 4, 1, false, GATE>(a, st)
                 : launch_cfg<LinOps, float, false, false, 8, 4, 1, false, GATE>(a, st);
    }
    if (in_dtype == 2) {
      if (bwd) return rev ? launch_cfg<LinOps, _Float16, true, true, 8, 4, 1, false, GATE>(a, st)
                          : launch_cfg<LinOps, _Float16, true, false, 8, 4, 1, false, GATE>(a, st);
      return rev ? launch_cfg<LinOps, _Float16, false, true, 8, 4, 1, false, GATE>(a, st)
                 : launch_cfg<LinOps, _Float16, false, false, 8, 4, 1, false, GATE>(a, st);
    }
    if (bwd) return rev ? launch_cfg<LinOps, uint16_t, true, true, 8, 4, 1, false, GATE>(a, st)
                        : launch_cfg<LinOps, uint16_t, true, false, 8, 4, 1, false, GATE>(a, st);
    return rev ? launch_cfg<LinOps, uint16_t, false, true, 8, 4, 1, false, GATE>(a, st)
               : launch_cfg<LinOps, uint16_t, false, false, 8, 4, 1, false, GATE>(a, st);
  }
  if (in_dtype == 0) {
    if (bwd) return rev ? launch_cfg<LinOps, float, true, true, 4, 4, 1, false, GATE>(a, st)
                        : launch_cfg<LinOps, float, true, false, 4, 4, 1, false, GATE>(a, st);
    // A forward row that fits one tile runs it as 8 waves of 2 sub-chunks
    // (B=8 C=1536 T=4096: 98.0 -> 95.3 us); the backward (165.9 vs 168.6 us)
    // and chained tiles (T = 65536 forward: 1.51 vs 1.59 ms) keep 4 x 4.
    if (scalar_tiles(a.T, a.stride, 4, 4096) == 1)
      return rev ? launch_cfg<LinOps, float, false, true, 8, 2, 1, false, GATE>(a, st)
                 : launch_cfg<LinOps, float, false, false, 8, 2, 1, false, GATE>(a, st);
    return rev ? launch_cfg<LinOps, float, false, true, 4, 4, 1, false, GATE>(a, st)
               : launch_cfg<LinOps, float, false, false, 4, 4, 1, false, GATE>(a, st);
  }
  if (in_dtype == 2) {
    if (bwd) return rev ? launch_cfg<LinOps, _Float16, true, true, 4, 4, 1, false, GATE>(a, st)
                        : launch_cfg<LinOps, _Float16, true, false, 4, 4, 1, false, GATE>(a, st);
    return rev ? launch_cfg<LinOps, _Float16, false, true, 4, 4, 1, false, GATE>(a, st)
               : launch_cfg<LinOps, _Float16, false, false, 4, 4, 1, false, GATE>(a, st);
  }
  if (bwd) return rev ? launch_cfg<LinOps, uint16_t, true, true, 4, 4, 1, false, GATE>(a, st)
                      : launch_cfg<LinOps, uint16_t, true, false, 4, 4, 1, false, GATE>(a, st);
  return rev ? launch_cfg<LinOps, uint16_t, false, true, 4, 4, 1, false, GATE>(a, st)
             : launch_cfg<LinOps, uint16_t, false, false, 4, 4, 1, false, GATE>(a, st);
}

hipError_t launch_scalar(const ScalarArgs& a, int in_dtype, bool bwd, hipStream_t st) {
  return launch_scalar_gate<kGateNone>(a, in_dtype, bwd, st);
}

// Linear scan with gates g = sigmoid(z) (z fp32 or bf16).
hipError_t launch_scalar_sigmoid(const ScalarArgs& a, int in_dtype, bool bwd, hipStream_t st) {
  return launch_scalar_gate<kGateSigmoid>(a, in_dtype, bwd, st);
}

// Log-space forward: fp32 (log a, log b), 4096-element tiles like the fp32
// scalar scan, with lanes owning 16 consecutive elements through LDS-staged
// windows: it carries the most VALU work per element (one exp per
// composition), and one DPP scan per wave instead of four measured 3% faster
// on dense rows and 13% on packed ones. (The memory-bound linear scans are
// 6-11% slower that way and keep 4-element lanes.)
hipError_t launch_log(const ScalarArgs& a, hipStream_t st) {
  if (scalar_short_rows(a.T, a.stride)) return launch_log_short(a, kGateNone, false, st);
  if (log_wide_tile(a.T))
    return a.rev ? launch_cfg<LogOps, float, false, true, 8, 1, 4, false, kGateNone, true>(a, st)
                 : launch_cfg<LogOps, float, false, false, 8, 1, 4, false, kGateNone, true>(a, st);
  return a.rev ? launch_cfg<LogOps, float, false, true, 4, 1, 4, false, kGateNone, true>(a, st)
               : launch_cfg<LogOps, float, false, false, 4, 1, 4, false, kGateNone, true>(a, st);
}

// Log-space backward: the fp32 adjoint scan with exponentiated gates.
hipError_t launch_log_bwd(const ScalarArgs& a, hipStream_t st) {
  if (scalar_short_rows(a.T, a.stride)) return launch_log_short(a, kGateNone, true, st);
  if (log_wide_tile(a.T))
    return a.rev ? launch_cfg<LinOps, float, true, true, 8, 4, 1, true>(a, st)
                 : launch_cfg<LinOps, float, true, false, 8, 4, 1, true>(a, st);
  return a.rev ? launch_cfg<LinOps, float, true, true, 4, 4, 1, true>(a, st)
               : launch_cfg<LinOps, float, true, false, 4, 4, 1, true>(a, st);
}

// Log-space scan with log a = -softplus(z): forward and backward.
hipError_t launch_log_softplus(const ScalarArgs& a, bool bwd, hipStream_t st) {
  if (scalar_short_rows(a.T, a.stride)) return launch_log_short(a, kGateNegSoftplus, bwd, st);
  if (log_wide_tile(a.T)) {
    if (bwd) return a.rev ? launch_cfg<LinOps, float, true, true, 8, 4, 1, true, kGateNegSoftplus>(a, st)
                          : launch_cfg<LinOps, float, true, false, 8, 4, 1, true, kGateNegSoftplus>(a, st);
    return a.rev ? launch_cfg<LogOps, float, false, true, 8, 1, 4, false, kGateNegSoftplus, true>(a, st)
                 : launch_cfg<LogOps, float, false, false, 8, 1, 4, false, kGateNegSoftplus, true>(a, st);
  }
  if (bwd) return a.rev ? launch_cfg<LinOps, float, true, true, 4, 4, 1, true, kGateNegSoftplus>(a, st)
                        : launch_cfg<LinOps, float, true, false, 4, 4, 1, true, kGateNegSoftplus>(a, st);
  return a.rev ? launch_cfg<LogOps, float, false, true, 4, 1, 4, false, kGateNegSoftplus, true>(a, st)
               : launch_cfg<LogOps, float, false, false, 4, 1, 4, false, kGateNegSoftplus, true>(a, st);
}

}  // namespace mscan
