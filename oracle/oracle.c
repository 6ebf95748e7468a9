/*
 * fp64 reference ("oracle") for the affine associative scan family.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, obviously correct CPU
 * definition that the GPU library is checked against. Only the test suite,
 * the package smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header or constant with the GPU library.
 *
 * Every routine walks time sequentially, one (row, segment) pair at a time,
 * exactly as the recurrences are written on the pages; OpenMP only spreads
 * independent (row, segment) pairs over host cores. Build with
 * -ffp-contract=off so no multiply-add is fused behind the reader's back.
 *
 * Sources (page title, section):
 *  - "associative_scan_triton" README (PheelaV), intro and quick start: the
 *    scalar recurrence h[t] = g[t] * h[t-1] + x[t]; "how it works": one
 *    independent scan per packed sequence given by cu_seqlens (flash-attn
 *    convention), and the backward pass (reverse scan on shifted gates for
 *    d_tokens, d_gates = shifted states * d_tokens); "bidirectional" branch
 *    that scans in the opposite time direction.
 *  - "Triton scan kernels" (minGRU docs), "One associative-scan family": the
 *    first-order affine map h_t = A_t h_{t-1} + B_t for scalar, 2x2 and k x k
 *    A_t, and the log-space form (running log-coefficient cumulative sum plus
 *    an online max-shifted log-sum-exp, writing h = exp(.)); "Autograd
 *    integration and the reversed-scan backward": the adjoint reverse-scans
 *    output gradients with the transposed next-step transition.
 *  - "Our RG-LRU GPU audit" (SAMU_GPU), "Strengthened fused path" and "Exact
 *    real chunk algebra": nonzero initial state and its gradient; a_t = 0 is a
 *    reset that erases the prefix.
 *
 * Conventions (readings where the pages are silent, stated once here):
 *  - Layout: element (r, t) of a row-major [rows][T] problem sits at
 *    r*row_stride + t; matrices add trailing [k][k] / [k][v] row-major blocks.
 *  - cu: NULL means one segment [0, T); otherwise nseg+1 nondecreasing
 *    offsets with cu[0] = 0 and cu[nseg] = T. Empty segments do nothing.
 *  - h0: NULL means a zero initial state; otherwise laid out [nseg][rows]
 *    (scalar) or [nseg][rows][k][v] (matrix). The first step of a segment
 *    multiplies h0 by its own gate: h_s = g_s * h0 + x_s.
 *  - reverse != 0 runs every segment from its last element down to its
 *    first: h_t = g_t * h_{t+1} + x_t, with h0 entering at the last element.
 *  - A zero transition (g_t = 0, log a_t = -inf, or a k x k A_t whose entries
 *    are all zero) is a reset: it erases everything before t, so h_t = x_t
 *    exactly, whatever the state before it holds, Inf and NaN included ("Our
 *    RG-LRU GPU audit", "Exact real chunk algebra": encoding a reset as
 *    a_t = 0 wipes out whatever came before it). For finite states this is the arithmetic
 *    value of g_t * h + x_t; for a non-finite state it is the reading that
 *    makes a reset inside a sequence behave as a sequence start does. The
 *    adjoints follow: no gradient flows through a reset (lam_{t-1} gets no
 *    g_t * lam_t term, and dh0 = 0 when the segment's first step is a reset).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define API __attribute__((visibility("default")))

static int64_t seg_begin(const int32_t* cu, int32_t s, int64_t T) { return cu ? (int64_t)cu[s] : (s == 0 ? 0 : T); }
static int64_t seg_end(const int32_t* cu, int32_t s, int64_t T) { return cu ? (int64_t)cu[s + 1] : T; }

/* ---------------------------------------------------------------------------
 * Scalar forward: per segment [b, e) of row r,
 *   causal : h_b = g_b*h0 + x_b,          h_t = g_t*h_{t-1} + x_t  (b < t < e)
 *   reverse: h_{e-1} = g_{e-1}*h0 + x_{e-1}, h_t = g_t*h_{t+1} + x_t (b <= t < e-1)
 * with a zero gate a reset: h_t = x_t (see the conventions above).
 * ------------------------------------------------------------------------- */
static double lin_step(double g, double state, double x) { return g == 0.0 ? x : g * state + x; }

API void oracle_scan_fwd(int64_t rows, int64_t T, int64_t row_stride, const int32_t* cu, int32_t nseg,
                         int32_t reverse, const double* g, const double* x, const double* h0, double* h) {
  if (!cu) nseg = 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t s = 0; s < nseg; ++s) {
      const int64_t b = seg_begin(cu, s, T), e = seg_end(cu, s, T);
      const double* gr = g + r * row_stride;
      const double* xr = x + r * row_stride;
      double* hr = h + r * row_stride;
      double state = h0 ? h0[(int64_t)s * rows + r] : 0.0;
      if (!reverse) {
        for (int64_t t = b; t < e; ++t) { state = lin_step(gr[t], state, xr[t]); hr[t] = state; }
      } else {
        for (int64_t t = e - 1; t >= b; --t) { state = lin_step(gr[t], state, xr[t]); hr[t] = state; }
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Scalar backward (adjoint of the forward above), given the forward's h:
 *   causal : lam_{e-1} = dy_{e-1};  lam_t = dy_t + g_{t+1}*lam_{t+1}
 *            dx_t = lam_t;  dg_t = lam_t * h_{t-1}  (h_{b-1} := h0, or 0)
 *            dh0  = g_b * lam_b
 *   reverse: lam_b = dy_b;  lam_t = dy_t + g_{t-1}*lam_{t-1}
 *            dx_t = lam_t;  dg_t = lam_t * h_{t+1}  (h_e := h0, or 0)
 *            dh0  = g_{e-1} * lam_{e-1}
 * A zero gate is a reset, so nothing flows through it: the g*lam term (of
 * lam and of dh0) is absent where the gate is 0.
 * dh0 may be NULL; an empty segment writes dh0 = 0.
 * ------------------------------------------------------------------------- */
static double through(double g, double lam) { return g == 0.0 ? 0.0 : g * lam; }

API void oracle_scan_bwd(int64_t rows, int64_t T, int64_t row_stride, const int32_t* cu, int32_t nseg,
                         int32_t reverse, const double* g, const double* h, const double* dy,
                         const double* h0, double* dx, double* dg, double* dh0) {
  if (!cu) nseg = 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t s = 0; s < nseg; ++s) {
      const int64_t b = seg_begin(cu, s, T), e = seg_end(cu, s, T);
      const int64_t o = r * row_stride;
      const double init = h0 ? h0[(int64_t)s * rows + r] : 0.0;
      double lam = 0.0, gnext = 0.0; /* gate of the step after t in scan order; none past the end */
      if (e <= b) {
        if (dh0) dh0[(int64_t)s * rows + r] = 0.0;
        continue;
      }
      if (!reverse) {
        for (int64_t t = e - 1; t >= b; --t) {
          lam = dy[o + t] + through(gnext, lam);
          dx[o + t] = lam;
          dg[o + t] = lam * (t > b ? h[o + t - 1] : init);
          gnext = g[o + t];
        }
        if (dh0) dh0[(int64_t)s * rows + r] = through(g[o + b], lam);
      } else {
        for (int64_t t = b; t < e; ++t) {
          lam = dy[o + t] + through(gnext, lam);
          dx[o + t] = lam;
          dg[o + t] = lam * (t < e - 1 ? h[o + t + 1] : init);
          gnext = g[o + t];
        }
        if (dh0) dh0[(int64_t)s * rows + r] = through(g[o + e - 1], lam);
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Log-space forward. With a_t = exp(log_a_t), b_t = exp(log_b_t) this is the
 * scalar recurrence h_t = a_t h_{t-1} + b_t, evaluated in the form the minGRU
 * page gives for parallel_scan_log: a running log-coefficient cumulative sum
 *   A_t = sum_{u=b..t} log_a_u
 * and an online max-shifted log-sum-exp
 *   h_t = exp( A_t + LSE_{b<=u<=t} (log_b_u - A_u) )   [+ exp(A_t + log_h0) term]
 * The accumulator keeps (m, s) with LSE = m + log(s) and rescales s when the
 * running maximum m grows.
 * A gate log_a_t = -inf (a_t = 0) erases everything before t (h_t = b_t), so
 * the sums restart there; without this the literal formula would form
 * (-inf) - (-inf).
 * log_h0 may be NULL (h0 = 0); it is laid out [nseg][rows].
 * reverse runs each segment from its end, as for the linear scan.
 * ------------------------------------------------------------------------- */
API void oracle_scan_log_fwd(int64_t rows, int64_t T, int64_t row_stride, const int32_t* cu, int32_t nseg,
                             int32_t reverse, const double* log_a, const double* log_b,
                             const double* log_h0, double* h) {
  if (!cu) nseg = 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t s = 0; s < nseg; ++s) {
      const int64_t b = seg_begin(cu, s, T), e = seg_end(cu, s, T), n = e - b;
      const int64_t o = r * row_stride;
      double A = 0.0;          /* running sum of log_a since the last restart */
      double m = -INFINITY;    /* running max of the LSE terms */
      double acc = 0.0;        /* sum of exp(term - m) */
      if (log_h0) {            /* h0 enters as the term log_h0 - A_{b-1} = log_h0 */
        double l0 = log_h0[(int64_t)s * rows + r];
        if (l0 > -INFINITY) { m = l0; acc = 1.0; }
      }
      for (int64_t i = 0; i < n; ++i) {
        const int64_t t = reverse ? e - 1 - i : b + i;
        const double la = log_a[o + t], lb = log_b[o + t];
        if (la == -INFINITY) { A = 0.0; m = -INFINITY; acc = 0.0; }  /* a_t = 0: restart */
        else A += la;
        const double term = lb - A;
        if (term > m) { acc = acc * exp(m - term) + 1.0; m = term; }
        else if (term > -INFINITY) { acc += exp(term - m); }
        h[o + t] = (m == -INFINITY) ? 0.0 : exp(A + m + log(acc));
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Log-space backward: the adjoint of oracle_scan_log_fwd with respect to its
 * log inputs, for L = <dy, h> with h the forward's (linear) output. With
 * a_t = exp(log_a_t), b_t = exp(log_b_t), h0 = exp(log_h0) (0 if NULL), the
 * recurrence is h_t = a_t h_{t-1} + b_t ("Triton scan kernels", "One
 * associative-scan family"), so the chain rule through exp gives, walking
 * each segment against the forward's direction:
 *   lam_t      = dy_t + a_{t+1} lam_{t+1}      (a of the next forward step; 0 past the end)
 *   dlog_b_t   = lam_t * b_t
 *   dlog_a_t   = lam_t * a_t * h_{t-1}         (h_{b-1} := h0)
 *   dlog_h0    = lam_b * a_b * h0              (b = the segment's forward-first step)
 * with no a*lam term through a reset a = 0 (log_a = -inf), as in
 * oracle_scan_bwd. reverse mirrors the neighbours as in oracle_scan_bwd.
 * dlog_h0 may be NULL; an empty segment writes 0.
 * ------------------------------------------------------------------------- */
API void oracle_scan_log_bwd(int64_t rows, int64_t T, int64_t row_stride, const int32_t* cu, int32_t nseg,
                             int32_t reverse, const double* log_a, const double* log_b, const double* h,
                             const double* dy, const double* log_h0, double* dlog_a, double* dlog_b,
                             double* dlog_h0) {
  if (!cu) nseg = 1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t s = 0; s < nseg; ++s) {
      const int64_t b = seg_begin(cu, s, T), e = seg_end(cu, s, T), n = e - b;
      const int64_t o = r * row_stride;
      const double h0 = log_h0 ? exp(log_h0[(int64_t)s * rows + r]) : 0.0;
      double lam = 0.0, anext = 0.0;
      if (n <= 0) {
        if (dlog_h0) dlog_h0[(int64_t)s * rows + r] = 0.0;
        continue;
      }
      int64_t tfirst = b;
      for (int64_t i = n - 1; i >= 0; --i) {
        const int64_t t = reverse ? e - 1 - i : b + i; /* walk opposite to the forward */
        const double at = exp(log_a[o + t]);
        lam = dy[o + t] + through(anext, lam);
        dlog_b[o + t] = lam * exp(log_b[o + t]);
        const double hprev = (i == 0) ? h0 : h[o + (reverse ? t + 1 : t - 1)];
        dlog_a[o + t] = lam * at * hprev;
        anext = at;
        tfirst = t;
      }
      if (dlog_h0) {
        const double af = exp(log_a[o + tfirst]);
        dlog_h0[(int64_t)s * rows + r] = (af == 0.0) ? 0.0 : af * lam * h0; /* none through a reset */
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Matrix-affine forward: h_t = A_t h_{t-1} + B_t with A_t k x k, B_t and h_t
 * k x v (left multiplication, row-major blocks). Same segment / h0 / reverse
 * rules as the scalar scan; h0 is [nseg][rows][k][v]. An all-zero A_t is a
 * reset: h_t = B_t.
 * A is [rows][T][k][k] and B, h are [rows][T][k][v] with row_stride counted in
 * time steps.
 * ------------------------------------------------------------------------- */
static int all_zero(const double* M, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (M[i] != 0.0) return 0;
  return 1;
}

API void oracle_matrix_fwd(int64_t rows, int64_t T, int64_t row_stride, const int32_t* cu, int32_t nseg,
                           int32_t reverse, int32_t k, int32_t v, const double* A, const double* B,
                           const double* h0, double* h) {
  if (!cu) nseg = 1;
  const int64_t kk = (int64_t)k * k, kv = (int64_t)k * v;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t s = 0; s < nseg; ++s) {
      const int64_t b = seg_begin(cu, s, T), e = seg_end(cu, s, T), n = e - b;
      double st[256], nx[256];
      for (int64_t j = 0; j < kv; ++j) st[j] = h0 ? h0[((int64_t)s * rows + r) * kv + j] : 0.0;
      for (int64_t i = 0; i < n; ++i) {
        const int64_t t = reverse ? e - 1 - i : b + i;
        const double* At = A + (r * row_stride + t) * kk;
        const double* Bt = B + (r * row_stride + t) * kv;
        const int reset = all_zero(At, kk);
        for (int p = 0; p < k; ++p)
          for (int q = 0; q < v; ++q) {
            double acc = Bt[p * v + q];
            if (!reset)
              for (int j = 0; j < k; ++j) acc += At[p * k + j] * st[j * v + q];
            nx[p * v + q] = acc;
          }
        memcpy(st, nx, sizeof(double) * kv);
        memcpy(h + (r * row_stride + t) * kv, st, sizeof(double) * kv);
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Matrix-affine backward, given the forward's h:
 *   causal : lam_{e-1} = dy_{e-1};  lam_t = dy_t + A_{t+1}^T lam_{t+1}
 *            dB_t = lam_t;  dA_t = lam_t h_{t-1}^T  (h_{b-1} := h0, or 0)
 *            dh0 = A_b^T lam_b
 *   reverse: mirrored (A_{t-1}, h_{t+1}, dh0 = A_{e-1}^T lam_{e-1}).
 * Nothing flows through an all-zero A (a reset): no A^T lam term there, in
 * lam or in dh0. dh0 may be NULL.
 * ------------------------------------------------------------------------- */
API void oracle_matrix_bwd(int64_t rows, int64_t T, int64_t row_stride, const int32_t* cu, int32_t nseg,
                           int32_t reverse, int32_t k, int32_t v, const double* A, const double* h,
                           const double* dy, const double* h0, double* dA, double* dB, double* dh0) {
  if (!cu) nseg = 1;
  const int64_t kk = (int64_t)k * k, kv = (int64_t)k * v;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
  for (int64_t r = 0; r < rows; ++r) {
    for (int32_t s = 0; s < nseg; ++s) {
      const int64_t b = seg_begin(cu, s, T), e = seg_end(cu, s, T), n = e - b;
      const double* init = h0 ? h0 + ((int64_t)s * rows + r) * kv : NULL;
      double lam[256], nl[256];
      const double* Anext = NULL; /* transition of the step after t in scan order */
      for (int64_t j = 0; j < kv; ++j) lam[j] = 0.0;
      if (n <= 0) {
        if (dh0) for (int64_t j = 0; j < kv; ++j) dh0[((int64_t)s * rows + r) * kv + j] = 0.0;
        continue;
      }
      int64_t tfirst = 0;
      for (int64_t i = n - 1; i >= 0; --i) {
        const int64_t t = reverse ? e - 1 - i : b + i; /* walk opposite to the forward */
        const double* dyt = dy + (r * row_stride + t) * kv;
        for (int p = 0; p < k; ++p)
          for (int q = 0; q < v; ++q) {
            double acc = dyt[p * v + q];
            if (Anext && !all_zero(Anext, kk))
              for (int j = 0; j < k; ++j) acc += Anext[j * k + p] * lam[j * v + q];
            nl[p * v + q] = acc;
          }
        memcpy(lam, nl, sizeof(double) * kv);
        memcpy(dB + (r * row_stride + t) * kv, lam, sizeof(double) * kv);
        /* the forward state before step t, in forward order */
        const int first = (i == 0);
        const double* hprev = first ? init : h + (r * row_stride + (reverse ? t + 1 : t - 1)) * kv;
        double* dAt = dA + (r * row_stride + t) * kk;
        for (int p = 0; p < k; ++p)
          for (int j = 0; j < k; ++j) {
            double acc = 0.0;
            if (hprev)
              for (int q = 0; q < v; ++q) acc += lam[p * v + q] * hprev[j * v + q];
            dAt[p * k + j] = acc;
          }
        Anext = A + (r * row_stride + t) * kk;
        tfirst = t;
      }
      if (dh0) {
        const double* Af = A + (r * row_stride + tfirst) * kk;
        const int reset = all_zero(Af, kk);
        for (int p = 0; p < k; ++p)
          for (int q = 0; q < v; ++q) {
            double acc = 0.0;
            if (!reset)
              for (int j = 0; j < k; ++j) acc += Af[j * k + p] * lam[j * v + q];
            dh0[((int64_t)s * rows + r) * kv + p * v + q] = acc;
          }
      }
    }
  }
}

/* ---------------------------------------------------------------------------
 * Gate activations for scans that take gate logits z instead of gates.
 * The workloads on the pages draw their gates this way: the packed scan's
 * g = sigmoid(z) (README benchmark inputs), and the log-space scan's
 * log_a = -softplus(z) (minGRU, "One associative-scan family": the base
 * log-space MinGRU's coefficient is a positive scalar in (0, 1)).
 *   kind 1: f(z) = sigmoid(z) = 1 / (1 + exp(-z)),  f'(z) = f(z) (1 - f(z))
 *   kind 2: f(z) = -softplus(z) = -log(1 + exp(z)),  f'(z) = -sigmoid(z)
 * oracle_gate writes f(z); oracle_gate_grad writes dz = dact * f'(z).
 * softplus is evaluated as max(z, 0) + log1p(exp(-|z|)) so it neither
 * overflows nor loses its tail for large |z|.
 * ------------------------------------------------------------------------- */
static double sigmoid_d(double z) {
  if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
  const double e = exp(z);
  return e / (1.0 + e);
}
static double softplus_d(double z) { return (z > 0.0 ? z : 0.0) + log1p(exp(-fabs(z))); }

API void oracle_gate(int32_t kind, int64_t n, const double* z, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (kind == 1) ? sigmoid_d(z[i]) : -softplus_d(z[i]);
}

API void oracle_gate_grad(int32_t kind, int64_t n, const double* z, const double* dact, double* dz) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const double s = sigmoid_d(z[i]);
    dz[i] = dact[i] * ((kind == 1) ? s * (1.0 - s) : -s);
  }
}

API int oracle_abi_version(void) { return 1; }

/* Number of threads the parallel loops above use (OpenMP's current team size). */
#ifdef _OPENMP
#include <omp.h>
API int oracle_num_threads(void) { return omp_get_max_threads(); }
#else
API int oracle_num_threads(void) { return 1; }
#endif
