// Scalar affine scan on short rows: rows that fit one tile of at most 2048
// elements run one workgroup per row with the smallest tile that holds the
// row, instead of a 4096-element tile that is mostly masked (the linear scan
// in every input type, and the log-space scan). Timing at 12288
// rows (fp32, forward / backward): T = 128 with 256-element tiles 7.9 / 9.6 us
// against 39 / 68 us; T = 1024 with 1024-element tiles 27 / 45 us against
// 36 / 70 us; T = 2048 with 2048-element tiles 50 / 87 us against 50 / 102 us.
#include "scan_scalar_kernel.hpp"

namespace mscan {
namespace {

// (waves, sub-chunks) of the short-row tiles: 256, 1024 and 2048 elements
constexpr int64_t kShortTiles[3] = {1 * 1 * 256, 2 * 2 * 256, 4 * 2 * 256};

int short_shape(int64_t T, int64_t stride) {
  for (int i = 0; i < 3; ++i)
    if (scalar_tiles(T, stride, 4, kShortTiles[i]) == 1) return i;
  return -1;
}

template <typename Tin, bool BWD, bool REV, int GATE, int WAVES, int SUBS>
hipError_t launch_row(const ScalarArgs& a0, hipStream_t st) {
  ScalarArgs a = a0;
  a.ntiles = 1;
  const dim3 grid((unsigned)a.rows), block(WAVES * 64);
  if (a.cu) hipLaunchKernelGGL((k_scalar<LinOps, Tin, BWD, REV, true, kRowLoop, WAVES, SUBS, 1, false, GATE>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_scalar<LinOps, Tin, BWD, REV, false, kRowLoop, WAVES, SUBS, 1, false, GATE>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <typename Tin, bool BWD, bool REV, int GATE>
hipError_t launch_shape(const ScalarArgs& a, int shape, hipStream_t st) {
  if (shape == 0) return launch_row<Tin, BWD, REV, GATE, 1, 1>(a, st);
  if (shape == 1) return launch_row<Tin, BWD, REV, GATE, 2, 2>(a, st);
  return launch_row<Tin, BWD, REV, GATE, 4, 2>(a, st);
}

// log space: forward on (m, s) carries, backward as the linear adjoint with
// exponentiated gates (LOGB); fp32 inputs
template <bool BWD, bool REV, int GATE, int WAVES, int SUBS>
hipError_t launch_log_row(const ScalarArgs& a0, hipStream_t st) {
  ScalarArgs a = a0;
  a.ntiles = 1;
  const dim3 grid((unsigned)a.rows), block(WAVES * 64);
  using Ops = typename std::conditional<BWD, LinOps, LogOps>::type;
  if (a.cu) hipLaunchKernelGGL((k_scalar<Ops, float, BWD, REV, true, kRowLoop, WAVES, SUBS, 1, BWD, GATE>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((k_scalar<Ops, float, BWD, REV, false, kRowLoop, WAVES, SUBS, 1, BWD, GATE>), grid, block, 0, st, a);
  return hipGetLastError();
}

template <bool BWD, bool REV, int GATE>
hipError_t launch_log_shape(const ScalarArgs& a, int shape, hipStream_t st) {
  if (shape == 0) return launch_log_row<BWD, REV, GATE, 1, 1>(a, st);
  if (shape == 1) return launch_log_row<BWD, REV, GATE, 2, 2>(a, st);
  return launch_log_row<BWD, REV, GATE, 4, 2>(a, st);
}

template <int GATE>
hipError_t launch_log_dir(const ScalarArgs& a, bool bwd, int shape, hipStream_t st) {
  const bool rev = a.rev != 0;
  if (bwd) return rev ? launch_log_shape<true, true, GATE>(a, shape, st) : launch_log_shape<true, false, GATE>(a, shape, st);
  return rev ? launch_log_shape<false, true, GATE>(a, shape, st) : launch_log_shape<false, false, GATE>(a, shape, st);
}

template <typename Tin, int GATE>
hipError_t launch_dir(const ScalarArgs& a, bool bwd, int shape, hipStream_t st) {
  const bool rev = a.rev != 0;
  if (bwd) return rev ? launch_shape<Tin, true, true, GATE>(a, shape, st) : launch_shape<Tin, true, false, GATE>(a, shape, st);
  return rev ? launch_shape<Tin, false, true, GATE>(a, shape, st) : launch_shape<Tin, false, false, GATE>(a, shape, st);
}

template <int GATE>
hipError_t launch_type(const ScalarArgs& a, int in_dtype, bool bwd, int shape, hipStream_t st) {
  if (in_dtype == 0) return launch_dir<float, GATE>(a, bwd, shape, st);
  if (in_dtype == 2) return launch_dir<_Float16, GATE>(a, bwd, shape, st);
  return launch_dir<uint16_t, GATE>(a, bwd, shape, st);
}

}  // namespace

bool scalar_short_rows(int64_t T, int64_t stride) { return short_shape(T, stride) >= 0; }

hipError_t launch_scalar_short(const ScalarArgs& a, int in_dtype, int gate, bool bwd, hipStream_t st) {
  const int shape = short_shape(a.T, a.stride);
  if (shape < 0) return hipErrorInvalidValue;
  return gate == kGateSigmoid ? launch_type<kGateSigmoid>(a, in_dtype, bwd, shape, st)
                              : launch_type<kGateNone>(a, in_dtype, bwd, shape, st);
}

hipError_t launch_log_short(const ScalarArgs& a, int gate, bool bwd, hipStream_t st) {
  const int shape = short_shape(a.T, a.stride);
  if (shape < 0) return hipErrorInvalidValue;
  return gate == kGateNegSoftplus ? launch_log_dir<kGateNegSoftplus>(a, bwd, shape, st)
                                  : launch_log_dir<kGateNone>(a, bwd, shape, st);
}

}  // namespace mscan
