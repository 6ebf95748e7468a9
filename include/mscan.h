/*
 * mscan.h -- C ABI of libmscan, the MI355X (gfx950) affine associative scan.
 *
 * The library computes first-order affine recurrences h_t = a_t * h_{t-1} + b_t
 * along the last (time) axis of row-major [rows][T] arrays, one independent
 * recurrence per row and per packed sequence, with hand-written HIP kernels.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Pointers.   Every array argument is a DEVICE pointer on the current HIP
 *              device. Base pointers must be 16-byte aligned. Outputs must not
 *              alias inputs. The caller owns every buffer, the workspace too;
 *              the library never allocates, frees or synchronises.
 *  Stream.     `stream` is a hipStream_t passed as void* (NULL = the null
 *              stream). Calls only enqueue work on it and return at once.
 *  Layout.     Element (r, t) of a scalar array sits at r*row_stride + t
 *              (elements). Matrix arrays hold a row-major k x k (transition) or
 *              k x v (injection / state) block per (r, t), with row_stride
 *              counted in time steps. Every array of one call shares rows, T
 *              and row_stride.
 *  Segments.   cu_seqlens (device, int32, nseg+1 entries, nondecreasing,
 *              cu[0] = 0, cu[nseg] = T) splits the time axis of every row into
 *              independent sequences, as in the flash-attn convention the
 *              associative-scan-triton README uses for packing ("how it works":
 *              each sequence is scanned on its own, no cross-document
 *              leakage). NULL means one sequence [0, T) and nseg must be 1.
 *              Empty sequences are allowed and do nothing. Sequence starts are
 *              hard boundaries: nothing, not even NaN, crosses them. The
 *              kernels do not validate the device contents of cu_seqlens;
 *              malformed offsets give unspecified values but every memory
 *              access stays inside the arrays described above.
 *  h0.         Optional initial state per (sequence, row): [nseg][rows] for
 *              scalars, [nseg][rows][k][v] for matrices; NULL means zero. The
 *              first step of a sequence multiplies it by its own transition:
 *              h_s = a_s * h0 + b_s ("Our RG-LRU GPU audit", "Strengthened
 *              fused path": nonzero initial state and its gradient).
 *  reverse.    0: causal, h_t = a_t h_{t-1} + b_t. 1: every sequence runs from
 *              its last element to its first, h_t = a_t h_{t+1} + b_t, with h0
 *              entering at the last element (the second, opposite-direction
 *              branch of the README's bidirectional scan).
 *  Precision.  Inputs are fp32, bf16 or fp16 (the scalar scan's g and x);
 *              bf16 and fp16 are widened exactly. All
 *              accumulation and every output is fp32 ("Triton scan kernels",
 *              "Kernel design": accumulation is fp32 regardless of input
 *              dtype).
 *  Workspace.  Calls that split a row into several tiles chain them through a
 *              small device workspace of mscan_workspace_bytes() bytes (about
 *              0.2% of the inputs; 2-4% for the matrix-core shapes). The call itself clears the part it uses,
 *              with a small fill kernel on `stream` before the scan kernel, so
 *              the contents between calls do not matter. Calls that overlap in
 *              time (different streams) must not share a workspace.
 *  Errors.     Arguments are validated on the host before any HIP call:
 *              MSCAN_ERR_INVALID (null required pointer, bad sizes, misaligned
 *              pointer, nseg inconsistent with cu_seqlens), MSCAN_ERR_UNSUPPORTED
 *              (dtype or matrix shape outside the supported envelope, or more
 *              than 2^24 - 1 tiles in one call; never silently masked, as the
 *              minGRU page's kernel envelope raises rather than
 *              miscomputes), MSCAN_ERR_WORKSPACE (ws_bytes too
 *              small), MSCAN_ERR_HIP (a launch failed; mscan_last_hip_error()
 *              gives the HIP error text). Nothing is enqueued on any error.
 *              There is no fallback path.
 */
#ifndef MSCAN_H_
#define MSCAN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSCAN_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define MSCAN_API __attribute__((visibility("default")))
#else
#define MSCAN_API
#endif

typedef enum {
  MSCAN_OK = 0,
  MSCAN_ERR_INVALID = 1,
  MSCAN_ERR_UNSUPPORTED = 2,
  MSCAN_ERR_WORKSPACE = 3,
  MSCAN_ERR_HIP = 4,
  MSCAN_ERR_TIMEOUT = 5 /* reported by mscan_workspace_error only (see there) */
} mscan_status;

typedef enum { MSCAN_F32 = 0, MSCAN_BF16 = 1, MSCAN_F16 = 2 } mscan_dtype;

/* Gate activation of the *_gated entry points, which take gate logits z and
 * compute the gate as they load it (no separate pointwise pass). */
typedef enum {
  MSCAN_GATE_NONE = 0,         /* (plain entry points) the operand is the gate itself */
  MSCAN_GATE_SIGMOID = 1,      /* linear scan: g = sigmoid(z)                          */
  MSCAN_GATE_NEG_SOFTPLUS = 2  /* log-space scan: log a = -softplus(z), a in (0, 1)    */
} mscan_gate;

/* Which computation a workspace is sized for. */
typedef enum {
  MSCAN_OP_SCAN_FWD = 0,
  MSCAN_OP_SCAN_BWD = 1,
  MSCAN_OP_SCAN_LOG_FWD = 2,
  MSCAN_OP_MATRIX_FWD = 3,
  MSCAN_OP_MATRIX_BWD = 4,
  MSCAN_OP_SCAN_LOG_BWD = 5
} mscan_op;

typedef struct {
  int64_t rows;               /* independent rows (e.g. B*C), >= 1                       */
  int64_t T;                  /* time steps per row (packed tokens for varlen),         *
                               * 1 <= T <= 2^31 - 1 (cu_seqlens offsets are int32)       */
  int64_t row_stride;         /* elements (steps for matrices) between rows, >= T       */
  const int32_t* cu_seqlens;  /* device, nseg+1 offsets; NULL = one sequence            */
  int32_t nseg;               /* number of sequences (1 when cu_seqlens is NULL)        */
  int32_t reverse;            /* 0 causal, 1 reverse-in-time                            */
} mscan_problem;

/* Workspace bytes `op` needs for `prob` (k, v are ignored for scalar ops).
 * Pure host function; returns 0 when the problem is invalid. */
MSCAN_API size_t mscan_workspace_bytes(const mscan_problem* prob, int op, int k, int v);

/* Zero-fill a workspace (one small fill kernel on `stream`). Optional: every
 * call clears the part of the workspace it uses. */
MSCAN_API mscan_status mscan_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Scalar forward scan (associative-scan-triton README, intro and quick start:
 * h[t] = g[t] * h[t-1] + x[t]; "how it works": chunked scan with a running
 * prefix carried across chunks).
 *   g, x : [rows][T] of in_dtype (MSCAN_F32, MSCAN_BF16 or MSCAN_F16), read only.
 *   h0   : fp32 [nseg][rows] or NULL.
 *   h    : fp32 [rows][T], written.                                          */
MSCAN_API mscan_status scan_fwd(const mscan_problem* prob, int in_dtype, const void* g, const void* x,
                      const float* h0, float* h, void* ws, size_t ws_bytes, void* stream);

/* Scalar backward: adjoint of scan_fwd given its output h (README, "how it
 * works": d_tokens is a reverse scan on shifted gates and d_gates = shifted
 * states * d_tokens; the fused kernel reads only the forward's inputs and
 * outputs, as the minGRU page's reversed-scan backward does).
 *   causal : lam_t = dy_t + g_{t+1} lam_{t+1} (no g past a sequence end),
 *            dx_t = lam_t, dg_t = lam_t h_{t-1} (h0 before a sequence start),
 *            dh0 = g_s lam_s at each sequence start s.
 *   reverse: the mirror image (g_{t-1}, h_{t+1}, dh0 at the last element).
 *   g    : [rows][T] of in_dtype; h, dy : fp32 [rows][T]; h0 : fp32 or NULL.
 *   dx, dg : fp32 [rows][T], written. dh0 : fp32 [nseg][rows] or NULL;
 *   an empty sequence gets dh0 = 0.                                          */
MSCAN_API mscan_status scan_bwd(const mscan_problem* prob, int in_dtype, const void* g, const float* h,
                      const float* dy, const float* h0, float* dx, float* dg, float* dh0,
                      void* ws, size_t ws_bytes, void* stream);

/* Log-space forward ("Triton scan kernels", "One associative-scan family":
 * parallel_scan_log carries h_t = a_t h_{t-1} + b_t in log space, a running
 * log-coefficient sum plus a max-shifted log-sum-exp, and writes h = exp(.)).
 *   log_a, log_b : fp32 [rows][T]; log_a = -inf (a = 0) is a reset.
 *   log_h0 : fp32 [nseg][rows] or NULL (h0 = 0).
 *   h : fp32 [rows][T] = exp(log h_t), written.                               */
MSCAN_API mscan_status scan_log_fwd(const mscan_problem* prob, const float* log_a, const float* log_b,
                          const float* log_h0, float* h, void* ws, size_t ws_bytes, void* stream);

/* Log-space backward: the adjoint of scan_log_fwd with respect to its log
 * inputs, for a loss L with dL/dh = dy ("Triton scan kernels", "One
 * associative-scan family": the log-space member is h_t = a_t h_{t-1} + b_t
 * with a = e^{log a}, b = e^{log b}; the page's own backward for it recomputes
 * through autograd, "Measured results"). Walking each sequence against the
 * forward's direction:
 *   lam_t    = dy_t + a_{t+1} lam_{t+1}  (no a past a sequence end)
 *   dlog_b_t = lam_t * b_t
 *   dlog_a_t = lam_t * a_t * h_{t-1}     (h0 = e^{log_h0} before a sequence start)
 *   dlog_h0  = lam_s * a_s * h0          at each sequence's first step s
 * (reverse: the mirror image, as for scan_bwd).
 *   log_a, log_b : fp32 [rows][T] (the forward's inputs);
 *   h : fp32 [rows][T], the forward's output; dy : fp32 [rows][T];
 *   log_h0 : fp32 [nseg][rows] or NULL.
 *   dlog_a, dlog_b : fp32 [rows][T], written. dlog_h0 : fp32 [nseg][rows] or
 *   NULL; an empty sequence gets 0.                                          */
MSCAN_API mscan_status scan_log_bwd(const mscan_problem* prob, const float* log_a, const float* log_b,
                          const float* h, const float* dy, const float* log_h0, float* dlog_a,
                          float* dlog_b, float* dlog_h0, void* ws, size_t ws_bytes, void* stream);

/* Scans that take gate logits z instead of gates. The activations are the ones
 * the pages' workloads draw their gates with: g = sigmoid(z) for the linear
 * scan (the associative-scan-triton README's benchmark gates), and
 * log a = -softplus(z) for the log-space scan (minGRU "One associative-scan
 * family": the base log-space member's coefficient is a positive scalar in
 * (0, 1)). Each computes exactly what the plain entry point computes on f(z);
 * the backward returns dz = dg * f'(z) in place of dg (resp. dlog_a):
 *   sigmoid      : dz = dg * g (1 - g)
 *   -softplus    : dz = dlog_a * (-sigmoid(z))
 * A reset in logit form is z = -inf for the sigmoid gate (g = 0) and
 * z = +inf for the -softplus gate (log a = -inf).
 * Arguments, layouts, workspace and errors are those of scan_fwd / scan_bwd /
 * scan_log_fwd / scan_log_bwd; z has the gate's type (fp32, bf16 or fp16
 * for the linear scan, fp32 for the log-space scan). A gate kind other than the one
 * listed for the entry point returns MSCAN_ERR_UNSUPPORTED.                 */
MSCAN_API mscan_status scan_fwd_gated(const mscan_problem* prob, int in_dtype, int gate /* MSCAN_GATE_SIGMOID */,
                            const void* z, const void* x, const float* h0, float* h, void* ws,
                            size_t ws_bytes, void* stream);
MSCAN_API mscan_status scan_bwd_gated(const mscan_problem* prob, int in_dtype, int gate /* MSCAN_GATE_SIGMOID */,
                            const void* z, const float* h, const float* dy, const float* h0, float* dx,
                            float* dz, float* dh0, void* ws, size_t ws_bytes, void* stream);
MSCAN_API mscan_status scan_log_fwd_gated(const mscan_problem* prob, int gate /* MSCAN_GATE_NEG_SOFTPLUS */,
                                const float* z, const float* log_b, const float* log_h0, float* h, void* ws,
                                size_t ws_bytes, void* stream);
MSCAN_API mscan_status scan_log_bwd_gated(const mscan_problem* prob, int gate /* MSCAN_GATE_NEG_SOFTPLUS */,
                                const float* z, const float* log_b, const float* h, const float* dy,
                                const float* log_h0, float* dz, float* dlog_b, float* dlog_h0, void* ws,
                                size_t ws_bytes, void* stream);

/* Matrix-affine forward ("Triton scan kernels", "One associative-scan family":
 * h_t = A_t h_{t-1} + B_t with A_t k x k, B_t and h_t k x v; matrix_scan is
 * k=2, v=1 and matrix_affine_scan is generic (k, v)). Supported: the page's
 * kernel envelope, k and v each in {1, 2, 4, 8, 16}, any T >= 1; any other
 * (k, v) returns MSCAN_ERR_UNSUPPORTED. (1, 1) is the scalar scan; (2,1),
 * (2,2) and (4,1) run on the vector ALUs; every other pair, (4,4) included,
 * runs its products on the matrix cores, zero-padded to 4 x 4 (k, v <= 4) or
 * 16 x 16, with fp32 operands and fp32 accumulation (the page's precision
 * guard at k = 16), and always needs the workspace (mscan_workspace_bytes:
 * per row, 2 KiB per chunk of 32 steps, or 128 bytes per chunk of 256 steps
 * when k, v <= 4). Its results are bit-reproducible from call to call.
 *   A : fp32 [rows][T][k][k]; B : fp32 [rows][T][k][v];
 *   h0 : fp32 [nseg][rows][k][v] or NULL; h : fp32 [rows][T][k][v], written. */
MSCAN_API mscan_status matrix_affine_scan_fwd(const mscan_problem* prob, int k, int v, const float* A,
                                    const float* B, const float* h0, float* h, void* ws,
                                    size_t ws_bytes, void* stream);

/* Matrix-affine backward (same page, "Autograd integration and the
 * reversed-scan backward": reverse-scan the output gradients with A_{t+1}^T and
 * form dA_t from the previous forward state).
 *   causal : lam_t = dy_t + A_{t+1}^T lam_{t+1}, dB_t = lam_t,
 *            dA_t = lam_t h_{t-1}^T (h0 before a sequence start),
 *            dh0 = A_s^T lam_s.   reverse: the mirror image.
 *   A : [rows][T][k][k]; h, dy : [rows][T][k][v]; h0 : [nseg][rows][k][v] or NULL.
 *   dA, dB written; dh0 : [nseg][rows][k][v] or NULL.                        */
MSCAN_API mscan_status matrix_affine_scan_bwd(const mscan_problem* prob, int k, int v, const float* A,
                                    const float* h, const float* dy, const float* h0, float* dA,
                                    float* dB, float* dh0, void* ws, size_t ws_bytes, void* stream);

/* Measurement aid (not part of the scan): the practical HBM ceiling for a
 * kernel that reads nsrc arrays and writes ndst arrays of n floats each. It
 * streams exactly those bytes with the scan kernels' access type
 * (non-temporal 16-byte loads and stores) and no other work, so a scan's
 * achieved bandwidth can be set against what the memory system delivers for
 * the same read:write mix (the associative-scan-triton README,
 * "performance", reports its kernels against device timings of the same
 * bytes). Each destination receives the elementwise sum of the sources.
 *   src : nsrc device pointers, dst : ndst device pointers, all 16-byte
 *         aligned, n floats each, n a multiple of 4.
 * Supported (nsrc, ndst): (1,1), (2,1), (3,1), (1,2), (2,2), (3,2), (4,2),
 * (4,3); other mixes return MSCAN_ERR_UNSUPPORTED, bad pointers or sizes
 * MSCAN_ERR_INVALID. Enqueues one kernel on `stream`. */
MSCAN_API mscan_status mscan_stream_ceiling(const float* const* src, int nsrc, float* const* dst, int ndst, size_t n,
                                            void* stream);

/* Whether the last call that chained tiles through `ws` had a look-back wait
 * give up ("The dispatch seam" of the minGRU page: a problem is reported,
 * never turned into a silent wrong result). A wait runs out only when a
 * predecessor never publishes (a workspace shared by calls that overlap in
 * time, or a partial launch below); the waiting tile then takes a NaN carry,
 * so every output that needed the missing value is NaN, and sets the
 * workspace's error word. This call enqueues a one-thread kernel on `stream`
 * that writes MSCAN_OK (0) or MSCAN_ERR_TIMEOUT (5) to *flag_out (device or
 * pinned host memory, 4-byte aligned), ordered after the work before it on
 * `stream`. The word keeps its value until the next call that chains tiles
 * through `ws` clears it. Returns MSCAN_ERR_INVALID for a null or misaligned
 * ws / flag_out or ws_bytes below the 128-byte header, MSCAN_ERR_HIP for a
 * launch error. */
MSCAN_API mscan_status mscan_workspace_error(const void* ws, size_t ws_bytes, int32_t* flag_out, void* stream);

/* Test hook for the loud failure above: the forward of scan_fwd (fp32 g = a,
 * x = b; k = v = 1) or matrix_affine_scan_fwd (A = a, B = b; any (k, v) of
 * the envelope), with no h0, launching only blocks [first_block, first_block +
 * nblocks) of the call's grid and letting each look-back wait give up after
 * spin_limit polls (0 = the library's default limit). With a block whose
 * predecessors are not launched, its wait runs out, its outputs that depend
 * on the carry are NaN, mscan_workspace_error reports MSCAN_ERR_TIMEOUT, and
 * every launched block still ends. The blocks not launched leave their
 * outputs unwritten. The problem must chain tiles (several tiles per row;
 * always for the matrix-core shapes), else MSCAN_ERR_UNSUPPORTED; a block
 * range outside the grid is MSCAN_ERR_INVALID; other errors as scan_fwd. */
MSCAN_API mscan_status mscan_debug_partial_fwd(const mscan_problem* prob, int k, int v, const float* a, const float* b,
                                               float* out, void* ws, size_t ws_bytes, int64_t first_block,
                                               int64_t nblocks, uint32_t spin_limit, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): scan_fwd
 * with no workspace argument. The look-back descriptors of rows that span
 * several tiles live in a fixed array of MSCAN_NOALLOC_SCRATCH_BYTES that the
 * library holds on every device it runs on, from the first use of its code on
 * that device until the process ends. The call allocates and frees nothing;
 * it clears the part of the array it uses with a small fill kernel on
 * `stream` (no memset node), so a previous call's contents do not matter.
 * Every call on one device shares that device's array: calls that overlap in
 * time on one device (different streams, or graphs replayed concurrently)
 * race and give wrong results; serialise them. A problem whose descriptors do
 * not fit (more than about 349,000 chained tiles of 4096 elements; rows of at
 * most one tile need none) returns MSCAN_ERR_WORKSPACE and enqueues nothing.
 * Arguments, results and every other error are those of scan_fwd; the
 * device's address of the array is resolved on the first call made with that
 * device current (a HIP failure there returns MSCAN_ERR_HIP). */
#define MSCAN_NOALLOC_SCRATCH_BYTES (8u << 20)
MSCAN_API mscan_status scan_fwd_noalloc(const mscan_problem* prob, int in_dtype, const void* g, const void* x,
                                        const float* h0, float* h, void* stream);

MSCAN_API const char* mscan_status_string(int status);
/* Text of the last HIP error this thread saw inside the library ("" if none). */
MSCAN_API const char* mscan_last_hip_error(void);
MSCAN_API int mscan_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSCAN_H_ */
