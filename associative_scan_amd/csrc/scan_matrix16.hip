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
// Three kernels per call (workspace per chunk of kChunk steps: P, Q and the
// chunk's carry-in state as padded 16 x 16 blocks, and a flag for chunks that
// contain a sequence start; nothing is read before it is written, so no
// clearing is needed):
//   summary : one wave per (row, chunk) walks the chunk: P <- X P, Q <- X Q + Y
//   carry   : one wave per row composes the chunk summaries in order
//   apply   : one wave per (row, chunk) recomputes every state from its
//             carry-in and stores it (backward: dB, dA and dh0 as well).
// Forward element (X, Y) = (A_t, B_t); backward element = (A of the previous
// step in processing order, transposed; dy_t). A sequence's first step in
// processing order is hard: forward h = A h0 + B, backward lam = dy.
#include "mscan_device.hpp"
#include "mscan_launch.hpp"

namespace mscan {

constexpr int kChunk16 = 64;                     // steps per chunk
constexpr int kM16Floats = 256;                  // floats per padded 16 x 16 block
constexpr size_t kM16ChunkBytes = 3 * 256 * 4;   // P, Q, carry-in per chunk

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

struct M16Ws {
  float* blocks;    // [rows][nchunks][3][256]: P, Q, carry-in
  int32_t* hard;    // [rows][nchunks]
};
__device__ __forceinline__ M16Ws m16_ws(void* ws, int64_t rows, int nchunks) {
  M16Ws w;
  w.blocks = (float*)((char*)ws + ws_desc_offset());
  w.hard = (int32_t*)((char*)ws + ws_desc_offset() + (size_t)rows * nchunks * kM16ChunkBytes);
  return w;
}

// ---------------------------------------------------------------------------
// step walking shared by the summary and apply kernels
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
// kernel 1: chunk summaries
// ---------------------------------------------------------------------------
template <bool FULL, bool BWD, bool REV, bool VARLEN>
__global__ __launch_bounds__(64) void k_m16_summary(const MatArgs a) {
  int64_t r;
  int c;
  tile_of_block<true>(a.rows, a.ntiles, r, c);
  M16Walk<FULL, BWD, REV, VARLEN> wk(a, r);
  const int64_t j0 = (int64_t)c * kChunk16, j1 = min(j0 + kChunk16, a.T);
  wk.begin(j0);
  v4f P = m16_ident(), Q = m16_zero();
  bool hard = false;
#pragma unroll 2
  for (int64_t j = j0; j < j1; ++j) {
    bool first, last;
    int sk;
    wk.at(j, first, last, sk);
    const v4f Y = wk.sh.ldB_D(wk.blkB(a.B, wk.phys(j)));
    if (first) {
      hard = true;
      P = m16_zero();
      if constexpr (!BWD) Q = a.h0 ? m16_mm(wk.sh.ldA_R(wk.blkA(a.A, wk.phys(j))), wk.h0D(sk), Y) : Y;
      else Q = Y;
    } else {
      const v4f X = wk.xop(j);
      P = m16_mm(X, P, m16_zero());
      Q = m16_mm(X, Q, Y);
    }
  }
  const M16Ws w = m16_ws(a.ws, a.rows, a.ntiles);
  float* out = w.blocks + ((int64_t)r * a.ntiles + c) * 3 * kM16Floats;
  m16_stD(out, P);
  m16_stD(out + kM16Floats, Q);
  if (threadIdx.x == 0) w.hard[(int64_t)r * a.ntiles + c] = hard ? 1 : 0;
}

// ---------------------------------------------------------------------------
// kernel 2: carry-in state of every chunk of a row
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_m16_carry(const MatArgs a) {
  const int64_t r = blockIdx.x;
  const M16Ws w = m16_ws(a.ws, a.rows, a.ntiles);
  float* rowb = w.blocks + (int64_t)r * a.ntiles * 3 * kM16Floats;
  const int32_t* hard = w.hard + (int64_t)r * a.ntiles;
  v4f h = m16_zero();
  // the next chunk's summary is loaded while the current one is applied
  v4f Pn = m16_ldR(rowb), Qn = m16_ldD(rowb + kM16Floats);
  int hn = hard[0];
  for (int c = 0; c < a.ntiles; ++c) {
    const v4f P = Pn, Q = Qn;
    const int hc = hn;
    if (c + 1 < a.ntiles) {
      const float* nb = rowb + (int64_t)(c + 1) * 3 * kM16Floats;
      Pn = m16_ldR(nb);
      Qn = m16_ldD(nb + kM16Floats);
      hn = hard[c + 1];
    }
    m16_stD(rowb + (int64_t)c * 3 * kM16Floats + 2 * kM16Floats, h);  // carry-in of chunk c
    h = hc ? Q : m16_mm(P, h, Q);
  }
}

// ---------------------------------------------------------------------------
// kernel 3: states (forward) or adjoints and gradients (backward)
// ---------------------------------------------------------------------------
template <bool FULL, bool BWD, bool REV, bool VARLEN>
__global__ __launch_bounds__(64) void k_m16_apply(const MatArgs a) {
  // 16 x 16 transpose tile, rows padded to 20 floats (conflict-free both ways)
  __shared__ __attribute__((aligned(16))) float s_t[BWD ? 16 * 20 : 4];
  int64_t r;
  int c;
  tile_of_block<true>(a.rows, a.ntiles, r, c);
  M16Walk<FULL, BWD, REV, VARLEN> wk(a, r);
  const int64_t j0 = (int64_t)c * kChunk16, j1 = min(j0 + kChunk16, a.T);
  wk.begin(j0);
  const M16Ws w = m16_ws(a.ws, a.rows, a.ntiles);
  v4f h = m16_ldD(w.blocks + ((int64_t)r * a.ntiles + c) * 3 * kM16Floats + 2 * kM16Floats);
  const int q = m16_q(), cl = m16_c();
#pragma unroll 2
  for (int64_t j = j0; j < j1; ++j) {
    bool first, last;
    int sk;
    wk.at(j, first, last, sk);
    const int64_t t = wk.phys(j);
    const v4f Y = wk.sh.ldB_D(wk.blkB(a.B, t));
    if constexpr (!BWD) {
      if (first) h = a.h0 ? m16_mm(wk.sh.ldA_R(wk.blkA(a.A, t)), wk.h0D(sk), Y) : Y;
      else h = m16_mm(wk.xop(j), h, Y);
      wk.sh.stB_D(wk.blkB(a.out0, t), h);
    } else {
      h = first ? Y : m16_mm(wk.xop(j), h, Y);  // h holds lam
      wk.sh.stB_D(wk.blkB(a.out0, t), h);     // dB = lam
      // dA_t = lam h_prev^T: lam to R layout through LDS, h_prev^T in D
      // layout is h_prev in R layout (h_prev = h0 at the sequence's
      // forward-first step, else the forward state one processing step on)
      s_t[(4 * q + 0) * 20 + cl] = h.x;
      s_t[(4 * q + 1) * 20 + cl] = h.y;
      s_t[(4 * q + 2) * 20 + cl] = h.z;
      s_t[(4 * q + 3) * 20 + cl] = h.w;
      wave_lds_sync();
      const v4f lamR = *(const v4f*)(s_t + cl * 20 + 4 * q);
      wave_lds_sync();
      v4f hpR;
      if (last) {
        hpR = a.h0 ? wk.sh.ldB_R(wk.h0p(sk)) : m16_zero();
      } else {
        hpR = wk.sh.ldB_R(wk.blkB(a.hs, wk.phys(j + 1)));
      }
      wk.sh.stA_D(wk.blkA(a.out1, t), m16_mm(lamR, hpR, m16_zero()));  // dA = lam h_prev^T
      if (last && a.dh0) {
        // dh0 = A_s^T lam_s (A_s^T in R layout is A_s in D layout)
        const v4f d = m16_mm(wk.sh.ldA_D(wk.blkA(a.A, t)), h, m16_zero());
        wk.sh.stB_D(a.dh0 + ((int64_t)sk * a.rows + r) * wk.sh.nb(), d);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
int64_t matrix16_chunks(int64_t T) { return (T + kChunk16 - 1) / kChunk16; }

size_t matrix16_ws_bytes(int64_t rows, int64_t T) {
  const int64_t n = rows * matrix16_chunks(T);
  return ws_desc_offset() + (size_t)n * kM16ChunkBytes + (size_t)n * sizeof(int32_t);
}

template <bool FULL, bool BWD, bool REV, bool VARLEN>
static hipError_t launch_m16_dir(const MatArgs& a, hipStream_t st) {
  const dim3 tiles((unsigned)((uint64_t)a.rows * (uint64_t)a.ntiles)), one(64);
  hipLaunchKernelGGL((k_m16_summary<FULL, BWD, REV, VARLEN>), tiles, one, 0, st, a);
  hipLaunchKernelGGL(k_m16_carry, dim3((unsigned)a.rows), one, 0, st, a);
  hipLaunchKernelGGL((k_m16_apply<FULL, BWD, REV, VARLEN>), tiles, one, 0, st, a);
  return hipGetLastError();
}

template <bool FULL>
static hipError_t launch_m16_shape(const MatArgs& a, bool bwd, hipStream_t st) {
  const bool rev = a.rev != 0, vl = a.cu != nullptr;
  if (bwd) {
    if (rev) return vl ? launch_m16_dir<FULL, true, true, true>(a, st) : launch_m16_dir<FULL, true, true, false>(a, st);
    return vl ? launch_m16_dir<FULL, true, false, true>(a, st) : launch_m16_dir<FULL, true, false, false>(a, st);
  }
  if (rev) return vl ? launch_m16_dir<FULL, false, true, true>(a, st) : launch_m16_dir<FULL, false, true, false>(a, st);
  return vl ? launch_m16_dir<FULL, false, false, true>(a, st) : launch_m16_dir<FULL, false, false, false>(a, st);
}

hipError_t launch_matrix16(const MatArgs& a0, bool bwd, hipStream_t st) {
  if (a0.k < 1 || a0.k > 16 || a0.v < 1 || a0.v > 16) return hipErrorInvalidValue;
  MatArgs a = a0;
  a.ntiles = (int32_t)matrix16_chunks(a.T);
  if (a.k == 16 && a.v == 16) return launch_m16_shape<true>(a, bwd, st);
  return launch_m16_shape<false>(a, bwd, st);
}

}  // namespace mscan
