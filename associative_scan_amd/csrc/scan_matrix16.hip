// Matrix-affine scan on the matrix cores, h_t = A_t h_{t-1} + B_t with k x k
// transitions and k x v states, k, v <= 16 ("Triton scan kernels", "One
// associative-scan family": matrix_affine_scan with block size k and injection
// width v; the page's kernel envelope is k, v in {1, 2, 4, 8, 16}), and its
// reverse adjoint (same page, "Autograd integration and the reversed-scan
// backward").
//
// Every block is zero-padded to 16 x 16 in registers: rows and columns past k
// (or v) load as 0 and are never stored, and a zero-padded A and B keep the
// padding of h, the adjoint and the chunk summaries at 0, so the padded
// arithmetic gives the k x v result exactly. Each step is then one or two
// 16 x 16 x 16 products on v_mfma_f32_16x16x4_f32: IEEE fp32 products with fp32
// accumulation, which is the precision the page's TF32 / IEEE guard asks for
// at k = 16. (16, 16) takes 16-byte loads; other shapes load element-wise.
//
// Register layouts of a 16 x 16 matrix X in a wave (lane l = 16 q + c):
//   D layout : lane (q, c) holds X[4q + i][c], i = 0..3 (an MFMA result)
//   R layout : lane (q, c) holds X[c][4q + i]           (a row-major 16-byte load)
// The K index of a 16 x 16 x 16 product is split into four MFMAs as
// {4q + s : q = 0..3}, s = 0..3. Then MFMA s takes element s of M in R layout
// as its A operand and element s of P in D layout as its B operand, so the
// result of one step (D layout) is the next step's B operand without moving
// any data between lanes, and each A_t is one coalesced load.
//
// One kernel per call (below: one wave per chunk of S steps, the chunk held in
// registers, carries chained from chunk to chunk through the workspace).
// Forward element (X, Y) = (A_t, B_t); backward element = (A of the previous
// step in processing order, transposed; dy_t). A sequence's first step in
// processing order is hard: forward h = A h0 + B, backward lam = dy.
#include <algorithm>

#include "mscan_device.hpp"
#include "mscan_launch.hpp"

namespace mscan {

constexpr int kM16Floats = 256;  // floats per padded 16 x 16 block

__device__ __forceinline__ int m16_q() { return (int)(threadIdx.x >> 4) & 3; }
__device__ __forceinline__ int m16_c() { return (int)(threadIdx.x & 15); }

// row-major block X -> R layout (lane (q, c) gets X[c][4q .. 4q+3])
__device__ __forceinline__ v4f m16_ldR(const float* X) {
  return *(const v4f*)(X + m16_c() * 16 + 4 * m16_q());
}
// row-major block X -> D layout (lane (q, c) gets X[4q + i][c]); also the R
// layout of X^T
__device__ __forceinline__ v4f m16_ldD(const float* X) {
  const int q = m16_q(), c = m16_c();
  v4f v;
  v.x = X[(4 * q + 0) * 16 + c];
  v.y = X[(4 * q + 1) * 16 + c];
  v.z = X[(4 * q + 2) * 16 + c];
  v.w = X[(4 * q + 3) * 16 + c];
  return v;
}
__device__ __forceinline__ void m16_stD(float* X, v4f v) {
  const int q = m16_q(), c = m16_c();
  X[(4 * q + 0) * 16 + c] = v.x;
  X[(4 * q + 1) * 16 + c] = v.y;
  X[(4 * q + 2) * 16 + c] = v.z;
  X[(4 * q + 3) * 16 + c] = v.w;
}
// acc + M P with M in R layout and P in D layout; result in D layout
__device__ __forceinline__ v4f m16_mm(v4f mR, v4f pD, v4f acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.x, pD.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.y, pD.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.z, pD.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.w, pD.w, acc, 0, 0, 0);
  return acc;
}
__device__ __forceinline__ v4f m16_zero() { return v4f{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ v4f m16_ident() {
  const int q = m16_q(), c = m16_c();
  return v4f{(4 * q + 0 == c) ? 1.f : 0.f, (4 * q + 1 == c) ? 1.f : 0.f, (4 * q + 2 == c) ? 1.f : 0.f,
             (4 * q + 3 == c) ? 1.f : 0.f};
}

// Block shapes. FULL: k = v = 16, 16-byte loads where the layout allows.
// Otherwise k, v <= 16 at run time, element-wise loads masked to the block
// (zero outside) and stores masked to it.
template <bool FULL>
struct M16Shape {
  int k, v;
  __device__ __forceinline__ int64_t na() const { return FULL ? 256 : k * k; }  // floats of A per step
  __device__ __forceinline__ int64_t nb() const { return FULL ? 256 : k * v; }  // floats of B / h per step
  // element (row, col) of a row-major block with rows x cols, ld = cols; 0 outside
  __device__ static __forceinline__ float el(const float* X, int row, int col, int rows, int cols) {
    return (row < rows && col < cols) ? X[row * cols + col] : 0.f;
  }
  __device__ static __forceinline__ v4f ld_D(const float* X, int rows, int cols) {
    const int q = m16_q(), c = m16_c();
    return v4f{el(X, 4 * q + 0, c, rows, cols), el(X, 4 * q + 1, c, rows, cols), el(X, 4 * q + 2, c, rows, cols),
               el(X, 4 * q + 3, c, rows, cols)};
  }
  __device__ static __forceinline__ v4f ld_R(const float* X, int rows, int cols) {
    const int q = m16_q(), c = m16_c();
    return v4f{el(X, c, 4 * q + 0, rows, cols), el(X, c, 4 * q + 1, rows, cols), el(X, c, 4 * q + 2, rows, cols),
               el(X, c, 4 * q + 3, rows, cols)};
  }
  __device__ static __forceinline__ void st_D(float* X, v4f x, int rows, int cols) {
    const int q = m16_q(), c = m16_c();
    if (c < cols) {
      if (4 * q + 0 < rows) X[(4 * q + 0) * cols + c] = x.x;
      if (4 * q + 1 < rows) X[(4 * q + 1) * cols + c] = x.y;
      if (4 * q + 2 < rows) X[(4 * q + 2) * cols + c] = x.z;
      if (4 * q + 3 < rows) X[(4 * q + 3) * cols + c] = x.w;
    }
  }
  // A (k x k) in R layout, and in D layout (= A^T in R layout)
  __device__ __forceinline__ v4f ldA_R(const float* X) const { return FULL ? m16_ldR(X) : ld_R(X, k, k); }
  __device__ __forceinline__ v4f ldA_D(const float* X) const { return FULL ? m16_ldD(X) : ld_D(X, k, k); }
  // B / h / dy / h0 (k x v) in D layout, and in R layout (= the D layout of the transpose)
  __device__ __forceinline__ v4f ldB_D(const float* X) const { return FULL ? m16_ldD(X) : ld_D(X, k, v); }
  __device__ __forceinline__ v4f ldB_R(const float* X) const { return FULL ? m16_ldR(X) : ld_R(X, k, v); }
  __device__ __forceinline__ void stB_D(float* X, v4f x) const {
    if (FULL) m16_stD(X, x);
    else st_D(X, x, k, v);
  }
  __device__ __forceinline__ void stA_D(float* X, v4f x) const {
    if (FULL) m16_stD(X, x);
    else st_D(X, x, k, k);
  }
};

// Sequence bookkeeping along one row, walked one physical step at a time in
// processing order (uniform across the wave). k = largest index with cu[k] <= t.
struct M16Seq {
  const int32_t* cu;
  int ncu, nseg;
  int k;
  __device__ __forceinline__ void init(const int32_t* cu_, int nseg_, int64_t t) {
    cu = cu_;
    nseg = nseg_;
    ncu = nseg_ + 1;
    int lo = 0, hi = ncu;  // largest i in [0, ncu) with cu[i] <= t (0 if none)
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)cu[mid] <= t) lo = mid; else hi = mid;
    }
    k = lo;
  }
  __device__ __forceinline__ void move_to(int64_t t, bool up) {
    if (up) {
      while (k + 1 < ncu && (int64_t)cu[k + 1] <= t) ++k;
    } else {
      while (k > 0 && (int64_t)cu[k] > t) --k;
    }
  }
  __device__ __forceinline__ bool is_start(int64_t t) const { return (int64_t)cu[k] == t; }
  __device__ __forceinline__ bool is_end(int64_t t) const { return k + 1 < ncu && (int64_t)cu[k + 1] - 1 == t; }
  __device__ __forceinline__ int seg() const { return min(max(k, 0), nseg - 1); }
};

// ---------------------------------------------------------------------------
// step walking along one row
// ---------------------------------------------------------------------------
template <bool FULL, bool BWD, bool REV, bool VARLEN>
struct M16Walk {
  const MatArgs& a;
  M16Shape<FULL> sh;
  int64_t row0, T, r;
  M16Seq seq;
  __device__ __forceinline__ M16Walk(const MatArgs& a_, int64_t r_) : a(a_), r(r_) {
    sh.k = a_.k;
    sh.v = a_.v;
    row0 = r_ * a_.stride;
    T = a_.T;
  }
  __device__ __forceinline__ int64_t phys(int64_t j) const { return REV ? T - 1 - j : j; }
  __device__ __forceinline__ void begin(int64_t j0) {
    if constexpr (VARLEN) seq.init(a.cu, a.nseg, phys(j0));
  }
  // position the sequence walk at processing index j; first / last in processing order
  __device__ __forceinline__ void at(int64_t j, bool& first, bool& last, int& sk) {
    const int64_t t = phys(j);
    if constexpr (VARLEN) {
      seq.move_to(t, !REV);
      const bool s = seq.is_start(t), e = seq.is_end(t);
      // the row's ends always close a sequence, whatever cu_seqlens holds, so
      // no step reaches a neighbour outside the row
      first = (REV ? e : s) || j == 0;
      last = (REV ? s : e) || j == T - 1;
      sk = seq.seg();
    } else {
      first = (j == 0);
      last = (j == T - 1);
      sk = 0;
    }
  }
  // step t of a row of A (k x k blocks) or of B / h / dy / dA-shaped outputs
  // Bit s of first / last: processing step j0 + s (s < n <= 32) opens / closes
  // a sequence in processing order (the row's ends always do).
  __device__ __forceinline__ void masks(int64_t j0, int n, uint32_t& firstm, uint32_t& lastm) {
    firstm = 0u;
    lastm = 0u;
    if constexpr (VARLEN) {
      begin(j0);
      for (int s = 0; s < n; ++s) {
        bool f, l;
        int sk;
        at(j0 + s, f, l, sk);
        firstm |= (uint32_t)f << s;
        lastm |= (uint32_t)l << s;
      }
    } else {
      if (j0 == 0) firstm = 1u;
      if (j0 + n == T) lastm = 1u << (n - 1);
    }
  }
  // sequence index of processing step j (0 without cu_seqlens), clamped to [0, nseg)
  __device__ __forceinline__ int seg_of(int64_t j) const {
    if constexpr (!VARLEN) {
      return 0;
    } else {
      const int64_t t = phys(j);
      int lo = 0, hi = a.nseg + 1;  // largest i with cu[i] <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)a.cu[mid] <= t) lo = mid; else hi = mid;
      }
      return min(lo, a.nseg - 1);
    }
  }
  __device__ __forceinline__ const float* blkA(const float* base, int64_t t) const { return base + (row0 + t) * sh.na(); }
  __device__ __forceinline__ float* blkA(float* base, int64_t t) const { return base + (row0 + t) * sh.na(); }
  __device__ __forceinline__ const float* blkB(const float* base, int64_t t) const { return base + (row0 + t) * sh.nb(); }
  __device__ __forceinline__ float* blkB(float* base, int64_t t) const { return base + (row0 + t) * sh.nb(); }
  // initial state (k x v) of sequence sk of this row
  __device__ __forceinline__ const float* h0p(int sk) const { return a.h0 + ((int64_t)sk * a.rows + r) * sh.nb(); }
  // transition operand (R layout) of the element at processing index j (not first)
  __device__ __forceinline__ v4f xop(int64_t j) const {
    if constexpr (!BWD) return sh.ldA_R(blkA(a.A, phys(j)));
    else return sh.ldA_D(blkA(a.A, phys(j - 1)));  // (A of the previous processing step)^T
  }
  __device__ __forceinline__ v4f h0D(int sk) const { return a.h0 ? sh.ldB_D(h0p(sk)) : m16_zero(); }
};

// ---------------------------------------------------------------------------
// single pass: chunk held in registers, carries chained through the workspace
// ---------------------------------------------------------------------------
// A wave owns S steps of one row. It loads the chunk's transition and
// injection blocks once into registers, walks them for the chunk summary
// (P, Q), takes its carry-in from the chunk before it, publishes the state
// after the chunk (h_out = P h_in + Q) and applies the carry from the same
// registers, so every input block crosses HBM once.
//
// Publication: h_out as 256 self-validating 64-bit words {tag, value} per
// chunk (lane order, four per lane), written and read with relaxed
// agent-scope atomics, so no fence is needed; the words are zero-filled
// before each call. A chunk that contains a sequence start publishes h_out
// right after its summary (it does not depend on the carry-in); the row's
// first chunk always does, so every chain starts. Each chunk reads only its
// predecessor's h_out, never an aggregate further back, so the rounding of
// every result is fixed: repeated calls give identical bits.
constexpr uint32_t kM16Tag = 2u;
constexpr size_t kM16PubBytes = 256 * 8;  // one published h_out

__device__ __forceinline__ void m16_publish(uint64_t* w, v4f v) {
  uint64_t* p = w + threadIdx.x * 4;
  st_u64(p + 0, pack_word(kM16Tag, v.x));
  st_u64(p + 1, pack_word(kM16Tag, v.y));
  st_u64(p + 2, pack_word(kM16Tag, v.z));
  st_u64(p + 3, pack_word(kM16Tag, v.w));
}
// h_out of a chunk once every lane sees all four of its words published;
// false after the spin limit (then the header's error word is set)
__device__ __forceinline__ bool m16_wait(const uint64_t* w, uint32_t* hdr, v4f& v) {
  const uint64_t* p = w + threadIdx.x * 4;
  for (uint32_t spins = 0;; ++spins) {
    const uint64_t a = ld_u64(p + 0), b = ld_u64(p + 1), c = ld_u64(p + 2), d = ld_u64(p + 3);
    const bool ok = word_tag(a) == kM16Tag && word_tag(b) == kM16Tag && word_tag(c) == kM16Tag &&
                    word_tag(d) == kM16Tag;
    if (__ballot(!ok) == 0ull) {
      v = v4f{word_val(a), word_val(b), word_val(c), word_val(d)};
      return true;
    }
    if (spins > kSpinLimit) {
      if (threadIdx.x == 0) st_u32(hdr + kHdrError, 1u);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// D layout in, R layout out (a transpose of the register tile) through LDS
__device__ __forceinline__ v4f m16_d_to_r(float* s_t, v4f x) {
  const int q = m16_q(), c = m16_c();
  s_t[(4 * q + 0) * 20 + c] = x.x;
  s_t[(4 * q + 1) * 20 + c] = x.y;
  s_t[(4 * q + 2) * 20 + c] = x.z;
  s_t[(4 * q + 3) * 20 + c] = x.w;
  wave_lds_sync();
  const v4f r = *(const v4f*)(s_t + c * 20 + 4 * q);
  wave_lds_sync();
  return r;
}

template <bool FULL, bool BWD, bool REV, bool VARLEN, int S>
__global__ __launch_bounds__(64) void k_m16_fused(const MatArgs a) {
  static_assert(S <= 32, "step masks are 32-bit");
  // 16 x 16 transpose tile, rows padded to 20 floats (conflict-free both ways)
  __shared__ __attribute__((aligned(16))) float s_t[16 * 20];
  int64_t r;
  int c;
  tile_of_block<true>(a.rows, a.ntiles, r, c);
  M16Walk<FULL, BWD, REV, VARLEN> wk(a, r);
  const int64_t j0 = (int64_t)c * S;
  const int n = (int)min((int64_t)S, a.T - j0);

  // sequence starts and ends in the chunk (before the loads: nothing is live yet)
  uint32_t firstm, lastm;
  wk.masks(j0, n, firstm, lastm);

  // ---- load the chunk: transition operand X (R layout) and injection Y (D
  // layout); backward also the forward state one processing step on, in R
  // layout (h_prev^T in D layout, for dA = lam h_prev^T). Steps past the row's
  // end (s >= n) hold zeros and are computed but never stored or published.
  v4f X[S], Y[S], H[BWD ? S : 1];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    X[s] = m16_zero();
    Y[s] = m16_zero();
    if constexpr (BWD) H[s] = m16_zero();
    if (s < n) {
      const int64_t j = j0 + s;
      const int64_t t = wk.phys(j);
      Y[s] = wk.sh.ldB_D(wk.blkB(a.B, t));
      if constexpr (!BWD) {
        X[s] = wk.sh.ldA_R(wk.blkA(a.A, t));
      } else {
        if (j > 0) X[s] = wk.sh.ldA_D(wk.blkA(a.A, wk.phys(j - 1)));  // (A one processing step back)^T
        if (j + 1 < a.T) H[s] = wk.sh.ldB_R(wk.blkB(a.hs, wk.phys(j + 1)));
      }
    }
  }
  wait_stage_loads();
  // Sequence boundaries, folded into the registers so that the step loops
  // below hold no loads (a load in them would make every step wait for the
  // stores before it): forward, a first step's value A h0 + B; backward, the
  // h_prev of a sequence's forward-first step is h0.
  if (a.h0 && (BWD ? lastm : firstm)) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if (((BWD ? lastm : firstm) >> s) & 1u) {
        const int sk = wk.seg_of(j0 + s);
        if constexpr (!BWD) Y[s] = m16_mm(X[s], wk.h0D(sk), Y[s]);
        else H[s] = wk.sh.ldB_R(wk.h0p(sk));
      }
    }
    wait_stage_loads();
  } else if (BWD && lastm) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      if ((lastm >> s) & 1u) H[s] = m16_zero();
  }

  // ---- chunk summary (a sequence's first step is hard: P = 0, Q = its value)
  const bool hard = firstm != 0u, first0 = (firstm & 1u) != 0u;
  v4f P = m16_ident(), Q = m16_zero();
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool f = (firstm >> s) & 1u;
    const v4f Pn = m16_mm(X[s], P, m16_zero()), Qn = m16_mm(X[s], Q, Y[s]);
    P = f ? m16_zero() : Pn;
    Q = f ? Y[s] : Qn;
  }

  // ---- carry-in from the chunk before, h_out for the chunk after
  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* pub = (uint64_t*)((char*)a.ws + ws_desc_offset());
  const int64_t me = r * a.ntiles + c;
  const bool publish = c + 1 < a.ntiles;
  if (publish && hard) m16_publish(pub + me * 256, Q);  // h_out = Q whatever the carry-in
  const v4f PR = (publish && !hard) ? m16_d_to_r(s_t, P) : m16_zero();  // off the chain
  v4f hin = m16_zero();
  if (!first0) {
    if (!m16_wait(pub + (me - 1) * 256, hdr, hin)) hin = m16_zero();
  }
  if (publish && !hard) m16_publish(pub + me * 256, m16_mm(PR, hin, Q));

  // ---- apply from the registers
  v4f h = hin;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool first = (firstm >> s) & 1u;
    const v4f hn = m16_mm(X[s], h, Y[s]);
    h = first ? Y[s] : hn;  // h holds lam in the backward
    if (s < n) {
      const int64_t j = j0 + s;
      const int64_t t = wk.phys(j);
      wk.sh.stB_D(wk.blkB(a.out0, t), h);  // forward h; backward dB = lam
      if constexpr (BWD) {
        // dA_t = lam h_prev^T
        wk.sh.stA_D(wk.blkA(a.out1, t), m16_mm(m16_d_to_r(s_t, h), H[s], m16_zero()));
        if (((lastm >> s) & 1u) && a.dh0) {
          // dh0 = A_s^T lam_s (A_s^T in R layout is A_s in D layout)
          const v4f d = m16_mm(wk.sh.ldA_D(wk.blkA(a.A, t)), h, m16_zero());
          wk.sh.stB_D(a.dh0 + ((int64_t)wk.seg_of(j) * a.rows + r) * wk.sh.nb(), d);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
// Steps per chunk of the single-pass kernel, from timing 8 / 16 / 32 at
// (16, 16), 512 rows, T = 4096: the forward is fastest with 32 (half the
// chained hops and published words of 16, despite one wave per SIMD), the
// backward ties at 16 and 32 and takes 16 (32 spills).
constexpr int kChunkFwd = 32, kChunkBwd = 16;

int64_t matrix16_chunks(int64_t T, bool bwd) {
  const int64_t S = bwd ? kChunkBwd : kChunkFwd;
  return (T + S - 1) / S;
}

size_t matrix16_ws_bytes(int64_t rows, int64_t T) {
  const int64_t n = std::max(matrix16_chunks(T, false), matrix16_chunks(T, true));
  return ws_desc_offset() + (size_t)(rows * n) * kM16PubBytes;
}

template <bool FULL, bool BWD, bool REV, bool VARLEN, int S>
static hipError_t launch_m16f_dir(const MatArgs& a0, hipStream_t st) {
  MatArgs a = a0;
  a.ntiles = (int32_t)((a.T + S - 1) / S);
  const int64_t n = a.rows * a.ntiles;
  // fresh words (and header) for this call: a zero tag = not published
  const hipError_t z = launch_zero(a.ws, ws_desc_offset() + (size_t)n * kM16PubBytes, st);
  if (z != hipSuccess) return z;
  hipLaunchKernelGGL((k_m16_fused<FULL, BWD, REV, VARLEN, S>), dim3((unsigned)n), dim3(64), 0, st, a);
  return hipGetLastError();
}

template <bool FULL>
static hipError_t launch_m16_shape(const MatArgs& a, bool bwd, hipStream_t st) {
  constexpr int SF = kChunkFwd, SB = kChunkBwd;
  const bool rev = a.rev != 0, vl = a.cu != nullptr;
  if (bwd) {
    if (rev) return vl ? launch_m16f_dir<FULL, true, true, true, SB>(a, st) : launch_m16f_dir<FULL, true, true, false, SB>(a, st);
    return vl ? launch_m16f_dir<FULL, true, false, true, SB>(a, st) : launch_m16f_dir<FULL, true, false, false, SB>(a, st);
  }
  if (rev) return vl ? launch_m16f_dir<FULL, false, true, true, SF>(a, st) : launch_m16f_dir<FULL, false, true, false, SF>(a, st);
  return vl ? launch_m16f_dir<FULL, false, false, true, SF>(a, st) : launch_m16f_dir<FULL, false, false, false, SF>(a, st);
}

hipError_t launch_matrix16(const MatArgs& a, bool bwd, hipStream_t st) {
  if (a.k < 1 || a.k > 16 || a.v < 1 || a.v > 16) return hipErrorInvalidValue;
  if (a.k == 16 && a.v == 16) return launch_m16_shape<true>(a, bwd, st);
  return launch_m16_shape<false>(a, bwd, st);
}

}  // namespace mscan
