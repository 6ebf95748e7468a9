// Matrix-affine scan on the matrix cores, h_t = A_t h_{t-1} + B_t with k x k
// transitions and k x v states ("Triton scan kernels", "One associative-scan
// family": matrix_affine_scan with block size k and injection width v; the
// page's kernel envelope is k, v in {1, 2, 4, 8, 16}), and its reverse adjoint
// (same page, "Autograd integration and the reversed-scan backward").
//
// Each step is one or two small dense products, run on the matrix cores with
// fp32 operands and fp32 accumulation (no reduced-precision input rounding, as
// the page's TF32 / IEEE guard asks at k = 16; the accumulation inside one
// instruction is the matrix core's, not a chain of separately rounded FMAs,
// so results agree with the VALU kernels to rounding, not bit for bit).
// Two register tiles:
//   Tile16: one 16 x 16 block per wave (k or v above 4), products on
//           v_mfma_f32_16x16x4_f32;
//   Tile4 : sixteen 4 x 4 blocks per wave (k, v <= 4), products on
//           v_mfma_f32_4x4x1_16b_f32, used by the row-segment kernel below
//           (one row per wave, the 16 blocks in time).
// Reading and writing the 16 x 16 blocks as rows with an LDS transpose per
// block (as the 4 x 4 kernel does) measured no faster forward and 39% slower
// backward, and changing the layout of row accesses on the matrix cores
// (a product with the identity per block) 1.6x / 1.8x slower, so Tile16
// keeps its column-wise dword accesses.
// Blocks smaller than the tile are zero-padded in registers: rows and columns
// past k (or v) load as 0 and are never stored, and a zero-padded A and B keep
// the padding of h, the adjoint and the chunk summaries at 0, so the padded
// arithmetic gives the k x v result exactly.
//
// Layouts, with E the tile edge, dr0 = the lane's first D-layout row and
// dc = its column (Tile16: lane 16 q + c has dr0 = 4 q, dc = c; Tile4: lane
// 4 b + c, block b, has dr0 = 0, dc = c):
//   D layout: register i holds X[dr0 + i][dc]   (an MFMA result)
//   R layout: register i holds X[dc][dr0 + i]   (one 16-byte load of a row)
// A product splits its K index into four MFMAs taking register s of M in R
// layout and register s of P in D layout, so a step's result (D layout) is the
// next step's operand without moving data between lanes; the R layout of X is
// the D layout of X^T.
//
// One kernel per call, carries chained from chunk to chunk through the
// workspace: k_mc_scan (Tile16) gives a wave S steps of one row; k_mc_rowseg
// (Tile4) gives a wave 16 S steps of one row, S per group of 4 lanes; a chunk
// is the consecutive spans of the waves of one workgroup.
// Forward element (X, Y) = (A_t, B_t); backward element = (A of the previous
// step in processing order, transposed; dy_t). A sequence's first step in
// processing order is hard: forward h = A h0 + B, backward lam = dy. So is a
// step whose X is all zero (a reset, "Our RG-LRU GPU audit", "Exact real chunk
// algebra"): it takes Y alone, whatever the state before it holds (Inf and NaN
// included), and a reset on a sequence's first step drops h0 (and gets no dh0).
#include <algorithm>

#include "mscan_device.hpp"
#include "mscan_launch.hpp"

namespace mscan {

__device__ __forceinline__ v4f mc_zero() { return v4f{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ v4f mc_nan() {
  const float q = __builtin_nanf("");
  return v4f{q, q, q, q};
}

// whether any of this lane's four values is nonzero
__device__ __forceinline__ bool mc_nonzero(v4f x) { return x.x != 0.f || x.y != 0.f || x.z != 0.f || x.w != 0.f; }

// ---------------------------------------------------------------------------
// register tiles
// ---------------------------------------------------------------------------
struct Tile16 {
  static constexpr int E = 16;  // tile edge
  // the block is all zero (wave-uniform: the wave holds the whole block)
  __device__ static __forceinline__ bool zero(v4f x) { return __ballot(mc_nonzero(x)) == 0ull; }
  __device__ static __forceinline__ int dr0() { return 4 * (int)((threadIdx.x >> 4) & 3); }
  __device__ static __forceinline__ int dc() { return (int)(threadIdx.x & 15); }
  // acc + M P with M in R layout and P in D layout; result in D layout
  __device__ static __forceinline__ v4f mm(v4f mR, v4f pD, v4f acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.x, pD.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.y, pD.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.z, pD.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(mR.w, pD.w, acc, 0, 0, 0);
    return acc;
  }
  // D layout in, R layout out, through LDS (rows padded to 20 floats)
  __device__ static __forceinline__ v4f d_to_r(float* s, v4f x) {
    const int r0 = dr0(), c = dc();
    s[(r0 + 0) * 20 + c] = x.x;
    s[(r0 + 1) * 20 + c] = x.y;
    s[(r0 + 2) * 20 + c] = x.z;
    s[(r0 + 3) * 20 + c] = x.w;
    wave_lds_sync();
    const v4f r = *(const v4f*)(s + c * 20 + r0);
    wave_lds_sync();
    return r;
  }
};

struct Tile4 {
  static constexpr int E = 4;
  __device__ static __forceinline__ int lrow() { return (int)((threadIdx.x >> 2) & 15); }  // lane group (block)
  // this lane group's block is all zero (uniform across the group)
  __device__ static __forceinline__ bool zero(v4f x) {
    return ((__ballot(mc_nonzero(x)) >> (4 * lrow())) & 0xfull) == 0ull;
  }
  __device__ static __forceinline__ int dr0() { return 0; }
  __device__ static __forceinline__ int dc() { return (int)(threadIdx.x & 3); }
  __device__ static __forceinline__ v4f mm(v4f mR, v4f pD, v4f acc) {
    acc = __builtin_amdgcn_mfma_f32_4x4x1f32(mR.x, pD.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_4x4x1f32(mR.y, pD.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_4x4x1f32(mR.z, pD.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_4x4x1f32(mR.w, pD.w, acc, 0, 0, 0);
    return acc;
  }
  __device__ static __forceinline__ v4f d_to_r(float* s, v4f x) {
    float* b = s + lrow() * 16;
    const int c = dc();
    b[0 * 4 + c] = x.x;
    b[1 * 4 + c] = x.y;
    b[2 * 4 + c] = x.z;
    b[3 * 4 + c] = x.w;
    wave_lds_sync();
    const v4f r = *(const v4f*)(b + c * 4);
    wave_lds_sync();
    return r;
  }
};

template <class TL>
__device__ __forceinline__ v4f tile_ident() {
  const int r0 = TL::dr0(), c = TL::dc();
  return v4f{(r0 + 0 == c) ? 1.f : 0.f, (r0 + 1 == c) ? 1.f : 0.f, (r0 + 2 == c) ? 1.f : 0.f,
             (r0 + 3 == c) ? 1.f : 0.f};
}

// Block shapes on a tile. FULL: k = v = E, 16-byte loads where the layout
// allows. Otherwise k, v <= E at run time, element-wise loads masked to the
// block (zero outside) and stores masked to it.
template <class TL, bool FULL>
struct TileShape {
  static constexpr int E = TL::E;
  int k, v;
  __device__ __forceinline__ int64_t na() const { return FULL ? E * E : k * k; }  // floats of A per step
  __device__ __forceinline__ int64_t nb() const { return FULL ? E * E : k * v; }  // floats of B / h per step
  // Cache policy of the block loads: a 16 x 16 block is read once, whole
  // lines per instruction, and streams (nontemporal; 4% faster on the 16 x 16
  // forward after a large write). A wave's 4 x 4 loads cover each line in two
  // halves, from consecutive steps of a lane group, and need the cache to
  // join them: those stay cached.
  static constexpr bool kNT = E == 16;
  __device__ static __forceinline__ float ldf(const float* p) { return kNT ? __builtin_nontemporal_load(p) : *p; }
  __device__ static __forceinline__ v4f ld4(const float* p) {
    return kNT ? __builtin_nontemporal_load((const v4f*)p) : *(const v4f*)p;
  }
  __device__ static __forceinline__ float el(const float* X, int row, int col, int rows, int cols) {
    return (row < rows && col < cols) ? ldf(X + row * cols + col) : 0.f;
  }
  __device__ static __forceinline__ v4f ld_D(const float* X, int rows, int cols) {
    const int r0 = TL::dr0(), c = TL::dc();
    if (FULL) return v4f{ldf(X + (r0 + 0) * E + c), ldf(X + (r0 + 1) * E + c), ldf(X + (r0 + 2) * E + c), ldf(X + (r0 + 3) * E + c)};
    return v4f{el(X, r0 + 0, c, rows, cols), el(X, r0 + 1, c, rows, cols), el(X, r0 + 2, c, rows, cols),
               el(X, r0 + 3, c, rows, cols)};
  }
  __device__ static __forceinline__ v4f ld_R(const float* X, int rows, int cols) {
    const int r0 = TL::dr0(), c = TL::dc();
    if (FULL) return ld4(X + c * E + r0);
    return v4f{el(X, c, r0 + 0, rows, cols), el(X, c, r0 + 1, rows, cols), el(X, c, r0 + 2, rows, cols),
               el(X, c, r0 + 3, rows, cols)};
  }
  __device__ static __forceinline__ void st_D(float* X, v4f x, int rows, int cols) {
    const int r0 = TL::dr0(), c = TL::dc();
    if (c < cols) {
      if (r0 + 0 < rows) X[(r0 + 0) * cols + c] = x.x;
      if (r0 + 1 < rows) X[(r0 + 1) * cols + c] = x.y;
      if (r0 + 2 < rows) X[(r0 + 2) * cols + c] = x.z;
      if (r0 + 3 < rows) X[(r0 + 3) * cols + c] = x.w;
    }
  }
  // A (k x k) in R layout, and in D layout (= A^T in R layout)
  __device__ __forceinline__ v4f ldA_R(const float* X) const { return ld_R(X, FULL ? E : k, FULL ? E : k); }
  __device__ __forceinline__ v4f ldA_D(const float* X) const { return ld_D(X, FULL ? E : k, FULL ? E : k); }
  // B / h / dy / h0 (k x v) in D layout, and in R layout (= the D layout of the transpose)
  __device__ __forceinline__ v4f ldB_D(const float* X) const { return ld_D(X, FULL ? E : k, FULL ? E : v); }
  __device__ __forceinline__ v4f ldB_R(const float* X) const { return ld_R(X, FULL ? E : k, FULL ? E : v); }
  __device__ __forceinline__ void stB_D(float* X, v4f x) const { st_D(X, x, FULL ? E : k, FULL ? E : v); }
  __device__ __forceinline__ void stA_D(float* X, v4f x) const { st_D(X, x, FULL ? E : k, FULL ? E : k); }
};

// Sequence bookkeeping along one row, walked one physical step at a time in
// processing order (uniform across the wave). k = largest index with cu[k] <= t.
struct McSeq {
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
// step walking along one row (the lane's row)
// ---------------------------------------------------------------------------
template <class TL, bool FULL, bool BWD, bool REV, bool VARLEN>
struct McWalk {
  const MatArgs& a;
  TileShape<TL, FULL> sh;
  int64_t row0, T, r;
  McSeq seq;
  __device__ __forceinline__ McWalk(const MatArgs& a_, int64_t r_) : a(a_), r(r_) {
    sh.k = a_.k;
    sh.v = a_.v;
    row0 = r_ * a_.stride;
    T = a_.T;
  }
  __device__ __forceinline__ int64_t phys(int64_t j) const { return REV ? T - 1 - j : j; }
  // Bit s of first / last: processing step j0 + s (s < n <= 32) opens / closes
  // a sequence in processing order; the row's ends always do, whatever
  // cu_seqlens holds, so no step reaches a neighbour outside the row.
  __device__ __forceinline__ void masks(int64_t j0, int n, uint32_t& firstm, uint32_t& lastm) {
    firstm = 0u;
    lastm = 0u;
    if (n <= 0) return;
    if constexpr (VARLEN) {
      seq.init(a.cu, a.nseg, phys(j0));
      for (int s = 0; s < n; ++s) {
        const int64_t j = j0 + s, t = phys(j);
        seq.move_to(t, !REV);
        const bool st = seq.is_start(t), en = seq.is_end(t);
        firstm |= (uint32_t)((REV ? en : st) || j == 0) << s;
        lastm |= (uint32_t)((REV ? st : en) || j == T - 1) << s;
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
  // step t of this row of A (k x k blocks) or of B / h / dy (k x v blocks)
  __device__ __forceinline__ const float* blkA(const float* base, int64_t t) const { return base + (row0 + t) * sh.na(); }
  __device__ __forceinline__ float* blkA(float* base, int64_t t) const { return base + (row0 + t) * sh.na(); }
  __device__ __forceinline__ const float* blkB(const float* base, int64_t t) const { return base + (row0 + t) * sh.nb(); }
  __device__ __forceinline__ float* blkB(float* base, int64_t t) const { return base + (row0 + t) * sh.nb(); }
  // initial state (k x v) of sequence sk of this row
  __device__ __forceinline__ const float* h0p(int sk) const { return a.h0 + ((int64_t)sk * a.rows + r) * sh.nb(); }
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
// chunk, written and read with relaxed agent-scope atomics, so no fence is
// needed. Word i of lane l sits at 64 i + l: each of the four stores of a wave
// covers 512 contiguous bytes. (With a lane's four words adjacent, every store
// touched 64 scattered 8-byte words, and the write-through of agent-scope
// stores wrote each as a 32-byte request: 8 KiB of HBM writes per 2 KiB
// published, 1.25x the algorithmic writes of the 16x16 forward.) The words
// are zero-filled
// before each call. A chunk that contains a sequence start publishes h_out
// right after its summary (it does not depend on the carry-in); the row's
// first chunk always does, so every chain starts. Each chunk reads only its
// predecessor's h_out, never an aggregate further back, so the rounding of
// every result is fixed: repeated calls give identical bits.
constexpr uint32_t kMcTag = 2u;
constexpr size_t kMcPubBytes = 256 * 8;  // one published h_out

__device__ __forceinline__ void mc_publish(uint64_t* w, v4f v) {
  stress_pause(3);
  uint64_t* p = w + (threadIdx.x & 63);
  st_u64(p + 0 * 64, pack_word(kMcTag, v.x));
  st_u64(p + 1 * 64, pack_word(kMcTag, v.y));
  st_u64(p + 2 * 64, pack_word(kMcTag, v.z));
  st_u64(p + 3 * 64, pack_word(kMcTag, v.w));
}
// h_out of a chunk once every lane sees all four of its words published;
// false after `limit` polls (then the header's error word is set)
__device__ __forceinline__ bool mc_wait(const uint64_t* w, uint32_t* hdr, uint32_t limit, v4f& v) {
  const uint64_t* p = w + (threadIdx.x & 63);
  for (uint32_t spins = 0;; ++spins) {
    const uint64_t a = ld_u64(p + 0 * 64), b = ld_u64(p + 1 * 64), c = ld_u64(p + 2 * 64), d = ld_u64(p + 3 * 64);
    const bool ok = word_tag(a) == kMcTag && word_tag(b) == kMcTag && word_tag(c) == kMcTag &&
                    word_tag(d) == kMcTag;
    if (__ballot(!ok) == 0ull) {
      v = v4f{word_val(a), word_val(b), word_val(c), word_val(d)};
      return true;
    }
    if (spins > limit) {
      if ((threadIdx.x & 63) == 0) st_u32(hdr + kHdrError, 1u);  // lane 0 of the waiting wave
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

// A 16 x 16 block staged in LDS by one direct 16-byte load per lane: lane l
// takes 16-byte unit swz(l) of the block (unit 4 row + col / 4) into LDS slot
// l. The swizzle spreads the four row groups of a column-wise read (rows
// 4q .. 4q+3, q = 0..3) over different banks; it is its own inverse.
__device__ __forceinline__ int mc_swz(int u) { return u ^ (((u >> 4) & 3) << 2); }
__device__ __forceinline__ void mc_stage(const float* blk, float* lds) {
  __builtin_amdgcn_global_load_lds((const void*)(blk + mc_swz((int)(threadIdx.x & 63)) * 4),
                                   (__attribute__((address_space(3))) void*)lds, 16, 0, kLdsNT);
}
// the staged block in D layout: register i = X[dr0 + i][dc]
__device__ __forceinline__ v4f mc_unstage(const float* lds) {
  const int r0 = Tile16::dr0(), c = Tile16::dc();
  const int o = c & 3, u = c >> 2;
  return v4f{lds[mc_swz((r0 + 0) * 4 + u) * 4 + o], lds[mc_swz((r0 + 1) * 4 + u) * 4 + o],
             lds[mc_swz((r0 + 2) * 4 + u) * 4 + o], lds[mc_swz((r0 + 3) * 4 + u) * 4 + o]};
}

// Tile16 only: a workgroup of WG waves owns a chunk of WG S consecutive steps
// of one row, wave w the steps w S .. w S + S - 1 of it. With WG > 1 the waves
// pass their summaries through LDS: wave w composes the summaries of waves
// 0 .. w-1 in that fixed order (its carry-in as a map of the chunk's
// carry-in), the last wave also its own (the chunk's summary), so rounding
// stays the same from call to call. The last wave waits for the chunk before,
// publishes h_out and hands the carry-in to the others. Several waves per
// chunk keep a CU's waves on one contiguous stretch of a row: as timing-only
// copies with the 16 x 16 forward's loads and stores (512 rows x T = 4096),
// one wave per 32-step chunk took 1.18 ms, two or four waves of 32 steps
// 1.05 ms; the kernels' own timings are with the chunk sizes below.
template <class TL, bool FULL, bool BWD, bool REV, bool VARLEN, int S, int WG>
__global__ __launch_bounds__(64 * WG) void k_mc_scan(const MatArgs a) {
  static_assert(S <= 32, "step masks are 32-bit");
  static_assert(WG >= 1 && WG <= 8, "waves per chunk");
  __shared__ __attribute__((aligned(16))) float s_tw[WG][16 * 20];  // transpose tile per wave
  const int w = WG > 1 ? (int)(threadIdx.x >> 6) : 0;
  float* const s_t = s_tw[w];
  int64_t r;
  int c;
  tile_of_block<true>(a.rows, a.ntiles, a.blk0, r, c);
  McWalk<TL, FULL, BWD, REV, VARLEN> wk(a, r);
  const int64_t j0 = ((int64_t)c * WG + w) * S;
  const int n = (int)max((int64_t)0, min((int64_t)S, a.T - j0));  // 0: a wave past the row's end

  // sequence starts and ends in the chunk (before the loads: nothing is live yet)
  uint32_t firstm, lastm;
  wk.masks(j0, n, firstm, lastm);

  // ---- load the chunk: transition operand X (R layout) and injection Y (D
  // layout); backward also the forward state one processing step on, in R
  // layout (h_prev^T in D layout, for dA = lam h_prev^T). Steps past the row's
  // end (s >= n) hold zeros and are computed but never stored or published.
  // The FULL backward stages X and Y in LDS instead (kStage): each block is
  // one direct 16-byte-per-lane row load into LDS, read back column-wise at
  // each use, so neither the column-wise global loads nor their registers are
  // needed. Xs(s) / Ys(s) give a step's operands either way.
  constexpr bool kStage = FULL && BWD;
  __shared__ __attribute__((aligned(16))) float s_stg[kStage ? WG * S * 2 * 256 : 4];
  float* const stg = s_stg + (kStage ? w * S * 2 * 256 : 0);
  v4f X[kStage ? 1 : S], Y[kStage ? 1 : S], H[BWD ? S : 1];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    if constexpr (!kStage) {
      X[s] = mc_zero();
      Y[s] = mc_zero();
    }
    if constexpr (BWD) H[s] = mc_zero();
    if (s < n) {
      const int64_t j = j0 + s;
      const int64_t t = wk.phys(j);
      if constexpr (kStage) {
        if (j > 0) mc_stage(wk.blkA(a.A, wk.phys(j - 1)), stg + (2 * s) * 256);  // A one processing step back
        mc_stage(wk.blkB(a.B, t), stg + (2 * s + 1) * 256);
      } else {
        // forward, FULL: B is read as rows (one 16-byte load per lane instead
        // of four 4-byte ones) and turned into the D layout below
        Y[s] = (FULL && !BWD) ? wk.sh.ldB_R(wk.blkB(a.B, t)) : wk.sh.ldB_D(wk.blkB(a.B, t));
        if constexpr (!BWD) {
          X[s] = wk.sh.ldA_R(wk.blkA(a.A, t));
        } else {
          if (j > 0) X[s] = wk.sh.ldA_D(wk.blkA(a.A, wk.phys(j - 1)));  // (A one processing step back)^T
        }
      }
      if constexpr (BWD) {
        if (j + 1 < a.T) H[s] = wk.sh.ldB_R(wk.blkB(a.hs, wk.phys(j + 1)));
      }
    }
  }
  wait_stage_loads();
  // operands of step s (zero where nothing was loaded: past the row's end,
  // and X at the row's first processing step)
  auto Xs = [&](int s) -> v4f {
    if constexpr (kStage) return (s < n && j0 + s > 0) ? mc_unstage(stg + (2 * s) * 256) : mc_zero();
    else return X[s];
  };
  auto Ys = [&](int s) -> v4f {
    if constexpr (kStage) return s < n ? mc_unstage(stg + (2 * s + 1) * 256) : mc_zero();
    else return Y[s];
  };
  if constexpr (FULL && !BWD) {
#pragma unroll
    for (int s = 0; s < S; ++s) Y[s] = TL::d_to_r(s_t, Y[s]);  // rows -> D layout
  }
  // Sequence boundaries, folded into the registers so that the step loops
  // below hold no loads (a load in them would make every step wait for the
  // stores before it): forward, a first step's value A h0 + B (B alone at a
  // reset, an all-zero A); backward, the h_prev of a sequence's forward-first
  // step is h0.
  const uint32_t foldm = BWD ? lastm : firstm;
  if (a.h0 && foldm) {
#pragma unroll
    for (int s = 0; s < S; ++s) {
      if ((foldm >> s) & 1u) {
        const int sk = wk.seg_of(j0 + s);
        if constexpr (!BWD) {
          if (!TL::zero(X[s])) Y[s] = TL::mm(X[s], wk.sh.ldB_D(wk.h0p(sk)), Y[s]);
        } else {
          H[s] = wk.sh.ldB_R(wk.h0p(sk));
        }
      }
    }
    wait_stage_loads();
  } else if (BWD && lastm) {
#pragma unroll
    for (int s = 0; s < S; ++s)
      if ((lastm >> s) & 1u) H[s] = mc_zero();
  }

  // ---- chunk summary (a sequence's first step and a reset, a step in the row
  // whose transition operand is all zero, are hard: P = 0, Q = its value)
  uint32_t zerom = 0u;
  v4f P = tile_ident<TL>(), Q = mc_zero();
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const v4f Xv = Xs(s), Yv = Ys(s);
    zerom |= (uint32_t)(s < n && TL::zero(Xv)) << s;
    const bool f = ((firstm | zerom) >> s) & 1u;
    const v4f Pn = TL::mm(Xv, P, mc_zero()), Qn = TL::mm(Xv, Q, Yv);
    P = f ? mc_zero() : Pn;
    Q = f ? Yv : Qn;
  }
  const uint32_t hardm = firstm | zerom;
  const bool hard = hardm != 0u, first0 = (hardm & 1u) != 0u;

  // ---- carry-in from the chunk before, h_out for the chunk after
  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* pub = (uint64_t*)((char*)a.ws + ws_desc_offset());
  const int64_t me = r * a.ntiles + c;
  const bool publish = c + 1 < a.ntiles;
  v4f h;  // this wave's carry-in
  if constexpr (WG == 1) {
    if (publish && hard) mc_publish(pub + me * 256, Q);  // h_out = Q whatever the carry-in
    const v4f PR = (publish && !hard) ? TL::d_to_r(s_t, P) : mc_zero();  // off the chain
    v4f hin = mc_zero();
    if (!first0) {
      // a wait that gave up leaves NaN, never a plausible wrong carry
      if (!mc_wait(pub + (me - 1) * 256, hdr, spin_limit(a.spin), hin)) hin = mc_nan();
    }
    if (publish && !hard) mc_publish(pub + me * 256, TL::mm(PR, hin, Q));
    h = hin;
  } else {
    // wave summaries F_u = (P_u, Q_u): P_u in D and R layout, Q_u in D layout
    __shared__ v4f s_PD[WG][64], s_PR[WG][64], s_Q[WG][64], s_hin[64];
    __shared__ uint32_t s_hard[WG];
    const int lane = (int)(threadIdx.x & 63);
    s_PD[w][lane] = P;
    s_PR[w][lane] = TL::d_to_r(s_t, P);
    s_Q[w][lane] = Q;
    if (lane == 0) s_hard[w] = (uint32_t)hard | ((uint32_t)first0 << 1);
    __syncthreads();
    // G = F_{w-1} o ... o F_0, the map from the chunk's carry-in to this
    // wave's: `have` once a summary is taken, hardG once one of them is hard
    // (then G no longer depends on the carry-in: PG = 0)
    v4f PG = mc_zero(), QG = mc_zero();
    bool have = false, hardG = false;
    for (int u = 0; u < w; ++u) {
      const uint32_t hu = s_hard[u];
      const v4f Qu = s_Q[u][lane];
      if (hu & 1u) {
        PG = mc_zero();
        QG = Qu;
        hardG = true;
      } else if (!have) {
        PG = s_PD[u][lane];
        QG = Qu;
      } else {
        const v4f PuR = s_PR[u][lane];
        if (!hardG) PG = TL::mm(PuR, PG, mc_zero());
        QG = TL::mm(PuR, QG, Qu);
      }
      have = true;
    }
    // the chunk's carry-in is needed unless its first step is hard
    const bool need_in = (s_hard[0] & 2u) == 0u;
    const v4f PGR = (have && !hardG) ? TL::d_to_r(s_t, PG) : mc_zero();  // off the chain
    if (w == WG - 1) {
      // chunk summary F_w o G, published at once when it is hard
      v4f PC = P, QC = Q;
      const bool hardC = hard || hardG;
      if (!hard && have) {
        const v4f PwR = s_PR[w][lane];
        PC = hardG ? mc_zero() : TL::mm(PwR, PG, mc_zero());
        QC = TL::mm(PwR, QG, Q);
      }
      if (publish && hardC) mc_publish(pub + me * 256, QC);
      const v4f PCR = (publish && !hardC) ? TL::d_to_r(s_t, PC) : mc_zero();  // off the chain
      v4f hin = mc_zero();
      if (need_in) {
        // a wait that gave up leaves NaN, never a plausible wrong carry
        if (!mc_wait(pub + (me - 1) * 256, hdr, spin_limit(a.spin), hin)) hin = mc_nan();
      }
      if (publish && !hardC) mc_publish(pub + me * 256, TL::mm(PCR, hin, QC));
      s_hin[lane] = hin;
    }
    __syncthreads();
    const v4f hin = s_hin[lane];
    h = !have ? hin : hardG ? QG : TL::mm(PGR, hin, QG);
  }

  // ---- apply from the registers
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool first = (hardm >> s) & 1u;
    const v4f Yv = Ys(s);
    const v4f hn = TL::mm(Xs(s), h, Yv);
    h = first ? Yv : hn;  // h holds lam in the backward
    if constexpr (BWD) {
      // dA_t = lam h_prev^T (the transpose is a whole-wave operation)
      const v4f lamR = TL::d_to_r(s_t, h);
      if (s < n) {
        const int64_t j = j0 + s;
        const int64_t t = wk.phys(j);
        if constexpr (FULL) {
          // both leave as rows, one 16-byte store per lane each: dB = lam from
          // its R layout, and dA from h_prev lam^T = dA^T, whose D layout is
          // the R layout of dA (16 x 16, 512 rows x T = 4096: 2.29 -> 2.23 ms)
          // (nontemporal: 2.22 -> 2.18 ms at 2 waves x 16 steps; A and dy read
          // as rows instead, with two more LDS transposes per step, 2.9-3.1 ms)
          __builtin_nontemporal_store(lamR, (v4f*)(wk.blkB(a.out0, t) + TL::dc() * 16 + TL::dr0()));
          __builtin_nontemporal_store(TL::mm(H[s], lamR, mc_zero()),
                                      (v4f*)(wk.blkA(a.out1, t) + TL::dc() * 16 + TL::dr0()));
        } else {
          wk.sh.stB_D(wk.blkB(a.out0, t), h);  // dB = lam
          wk.sh.stA_D(wk.blkA(a.out1, t), TL::mm(lamR, H[s], mc_zero()));
        }
      }
      if (((lastm >> s) & 1u) && a.dh0 && s < n) {
        // dh0 = A_s^T lam_s (A_s^T in R layout is A_s in D layout); 0 where
        // A_s = 0: nothing flows through a reset
        const int64_t j = j0 + s;
        const v4f As = wk.sh.ldA_D(wk.blkA(a.A, wk.phys(j)));
        const v4f d = TL::mm(As, h, mc_zero());
        wk.sh.stB_D(a.dh0 + ((int64_t)wk.seg_of(j) * a.rows + r) * wk.sh.nb(), TL::zero(As) ? mc_zero() : d);
      }
    } else if constexpr (FULL) {
      // h leaves as rows: one 16-byte store per lane (16 x 16 forward, 512 rows
      // x T = 4096 after a 1 GiB fill, with the row loads above: 1.35 -> 1.22
      // ms), nontemporal like the backward's.
      const v4f hR = TL::d_to_r(s_t, h);
      if (s < n) __builtin_nontemporal_store(hR, (v4f*)(wk.blkB(a.out0, wk.phys(j0 + s)) + TL::dc() * 16 + TL::dr0()));
    } else {
      if (s < n) wk.sh.stB_D(wk.blkB(a.out0, wk.phys(j0 + s)), h);
    }
  }
}

// ---------------------------------------------------------------------------
// 4 x 4 blocks, one row per wave: blocks in time
// ---------------------------------------------------------------------------
// For k, v <= 4 a wave owns 16 S consecutive steps of ONE row: lane group b
// (lanes 4b .. 4b+3) owns steps b S .. b S + S - 1 of the wave's span, so the
// wave's loads stay inside one contiguous window of the row. Each group walks
// its S steps for its block summary (sixteen 4x4x4 products per MFMA), the
// groups combine their summaries by an inclusive scan over groups (4 levels,
// operands moved 4, 8, 16, 32 lanes up), every group applies the result to
// the carry-in of the wave to get the state after it, and group b starts from
// group b-1's. Waves chain as above, through 16 published words (a 4x4 h_out).
// Control flow stays uniform across the wave around every MFMA: a step where
// only some groups start or end a sequence is computed for all groups and
// selected per lane.
constexpr size_t kSegPubBytes = 16 * 8;  // one published 4 x 4 h_out

// lane (b, q) publishes / reads column q of a 4 x 4 block (word 4 i + j = h[i][j])
__device__ __forceinline__ void seg_publish(uint64_t* w, v4f v) {
  stress_pause(4);
  const int q = (int)(threadIdx.x & 3);
  st_u64(w + 0 * 4 + q, pack_word(kMcTag, v.x));
  st_u64(w + 1 * 4 + q, pack_word(kMcTag, v.y));
  st_u64(w + 2 * 4 + q, pack_word(kMcTag, v.z));
  st_u64(w + 3 * 4 + q, pack_word(kMcTag, v.w));
}
__device__ __forceinline__ bool seg_wait(const uint64_t* w, uint32_t* hdr, uint32_t limit, v4f& v) {
  const int q = (int)(threadIdx.x & 3);
  for (uint32_t spins = 0;; ++spins) {
    const uint64_t a = ld_u64(w + 0 * 4 + q), b = ld_u64(w + 1 * 4 + q), c = ld_u64(w + 2 * 4 + q),
                   d = ld_u64(w + 3 * 4 + q);
    const bool ok = word_tag(a) == kMcTag && word_tag(b) == kMcTag && word_tag(c) == kMcTag &&
                    word_tag(d) == kMcTag;
    if (__ballot(!ok) == 0ull) {
      v = v4f{word_val(a), word_val(b), word_val(c), word_val(d)};
      return true;
    }
    if (spins > limit) {
      if ((threadIdx.x & 63) == 0) st_u32(hdr + kHdrError, 1u);  // lane 0 of the waiting wave
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}
__device__ __forceinline__ v4f shfl_up4(v4f x, int d) {
  return v4f{__shfl_up(x.x, d, 64), __shfl_up(x.y, d, 64), __shfl_up(x.z, d, 64), __shfl_up(x.w, d, 64)};
}
__device__ __forceinline__ v4f sel4(bool c, v4f a, v4f b) {
  return v4f{c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w};
}

// Dispatch order of the row-segment kernel: groups of 8 consecutive chunks of
// a row run back to back (tile_of_block_grouped). At (4, 4), 4096 rows x
// T = 8192 (rows 512 KiB apart), workgroups that start together then read
// 128 KiB stretches instead of 16 KiB pieces of 2048 different rows: forward
// 1.30 -> 1.24-1.26 ms, backward 2.23 -> 2.15-2.19 ms. A copy with the
// kernel's loads and stores and no arithmetic takes the same time in either
// order, so the order, not the chain, sets the pace; whole rows back to back
// (row-major) would stream faster still (copy 1.21 ms) but serialise the
// carry chain (2.09 ms), and 16-chunk groups were slower (1.46 ms).
// The forward's chunks are 4 waves long (4 x 256 steps per workgroup) and run
// in groups of 2 (forward 1.26 -> 1.21 ms; waves x group: 1 x 8 1.26 ms,
// 2 x 8 1.32, 2 x 4 1.25, 2 x 2 1.24, 4 x 8 1.33, 4 x 4 1.26, 4 x 1 1.22,
// 8 x 1 1.44); the backward keeps one wave per chunk (2 waves: 2.18 -> 2.45 ms).
constexpr int kSegGroupFwd = 2, kSegGroupBwd = 8;

// A workgroup of WG waves owns WG consecutive wave spans of the row; with
// WG > 1 the waves combine their spans' summaries through LDS as k_mc_scan's
// do, and only the last one waits for the chunk before and publishes.
template <bool FULL, bool BWD, bool REV, bool VARLEN, int S, int WG>
__global__ __launch_bounds__(64 * WG) void k_mc_rowseg(const MatArgs a) {
  static_assert(S <= 32, "step masks are 32-bit");
  static_assert(WG >= 1 && WG <= 8, "waves per chunk");
  using TL = Tile4;
  __shared__ __attribute__((aligned(16))) float s_tw[WG][16 * 20];  // transpose tile per wave
  const int w = WG > 1 ? (int)(threadIdx.x >> 6) : 0;
  float* const s_t = s_tw[w];
  int64_t r;
  int c;
  tile_of_block_grouped(a.rows, a.ntiles, a.blk0, BWD ? kSegGroupBwd : kSegGroupFwd, r, c);
  McWalk<TL, FULL, BWD, REV, VARLEN> wk(a, r);
  const int b = TL::lrow();
  // this group's first processing step
  const int64_t jb = ((int64_t)c * WG + w) * (16 * S) + (int64_t)b * S;
  const int nb = (int)max((int64_t)0, min((int64_t)S, a.T - jb));

  uint32_t firstm, lastm;  // per group
  wk.masks(jb, nb, firstm, lastm);

  // ---- load the group's S steps (as in k_mc_scan, per lane group)
  v4f X[S], Y[S], H[BWD ? S : 1];
#pragma unroll
  for (int s = 0; s < S; ++s) {
    X[s] = mc_zero();
    Y[s] = mc_zero();
    if constexpr (BWD) H[s] = mc_zero();
    if (s < nb) {
      const int64_t j = jb + s;
      const int64_t t = wk.phys(j);
      // FULL: every block is read as rows (one 16-byte load per lane) and
      // turned into the layout it is used in below
      Y[s] = FULL ? wk.sh.ldB_R(wk.blkB(a.B, t)) : wk.sh.ldB_D(wk.blkB(a.B, t));
      if constexpr (!BWD) {
        X[s] = wk.sh.ldA_R(wk.blkA(a.A, t));
      } else {
        if (j > 0) X[s] = FULL ? wk.sh.ldA_R(wk.blkA(a.A, wk.phys(j - 1))) : wk.sh.ldA_D(wk.blkA(a.A, wk.phys(j - 1)));
        if (j + 1 < a.T) H[s] = wk.sh.ldB_R(wk.blkB(a.hs, wk.phys(j + 1)));
      }
    }
  }
  wait_stage_loads();
  if constexpr (FULL) {
    // rows -> D layout (Y), and A -> A^T in R layout (the backward's X): the
    // same per-group transpose through LDS
#pragma unroll
    for (int s = 0; s < S; ++s) {
      Y[s] = TL::d_to_r(s_t, Y[s]);
      if constexpr (BWD) X[s] = TL::d_to_r(s_t, X[s]);
    }
  }
  // sequence boundaries folded into the registers (forward: A h0 + B at a
  // first step, B alone at a reset, an all-zero A; backward: h_prev = h0 or 0
  // at a forward-first step)
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool z = BWD ? false : TL::zero(X[s]);  // whole wave: the test is a ballot
    const bool f = BWD ? ((lastm >> s) & 1u) : (((firstm >> s) & 1u) && !z);
    if (__ballot(f) == 0ull) continue;
    v4f h0v = mc_zero();
    if (f && a.h0) {
      const int sk = wk.seg_of(jb + s);
      h0v = BWD ? wk.sh.ldB_R(wk.h0p(sk)) : wk.sh.ldB_D(wk.h0p(sk));
    }
    wait_stage_loads();
    if constexpr (!BWD) {
      const v4f yf = TL::mm(X[s], h0v, Y[s]);
      if (f && a.h0) Y[s] = yf;
    } else {
      if (f) H[s] = h0v;
    }
  }

  // ---- group summary (a sequence's first step and a reset, a step in the row
  // whose transition operand is all zero, are hard)
  uint32_t zerom = 0u;
  v4f P = tile_ident<TL>(), Q = mc_zero();
#pragma unroll
  for (int s = 0; s < S; ++s) {
    zerom |= (uint32_t)(s < nb && TL::zero(X[s])) << s;
    const bool f = ((firstm | zerom) >> s) & 1u;
    const v4f Pn = TL::mm(X[s], P, mc_zero()), Qn = TL::mm(X[s], Q, Y[s]);
    P = sel4(f, mc_zero(), Pn);
    Q = sel4(f, Y[s], Qn);
  }
  const uint32_t hardm = firstm | zerom;

  // ---- inclusive scan over the 16 groups: group b <- (group b) after (groups before)
  bool hard = hardm != 0u;
#pragma unroll
  for (int k = 1; k < 16; k <<= 1) {
    const v4f Pp = shfl_up4(P, 4 * k), Qp = shfl_up4(Q, 4 * k);
    const bool hp = __shfl_up((int)hard, 4 * k, 64) != 0;
    const v4f PR = TL::d_to_r(s_t, P);
    const v4f Pn = TL::mm(PR, Pp, mc_zero()), Qn = TL::mm(PR, Qp, Q);
    const bool take = b >= k && !hard;
    P = sel4(take, Pn, P);
    Q = sel4(take, Qn, Q);
    hard = hard || (b >= k && hp);
  }
  // the wave is hard if group 15's inclusive summary is; it needs no carry-in
  // if its first step starts a sequence
  const bool whard = __shfl((int)hard, 60, 64) != 0;
  const bool first0 = __shfl((int)(hardm & 1u), 0, 64) != 0;

  // ---- carry-in from the chunk before, h_out for the chunk after
  uint32_t* hdr = (uint32_t*)a.ws;
  uint64_t* pub = (uint64_t*)((char*)a.ws + ws_desc_offset());
  const int64_t me = r * a.ntiles + c;
  const bool publish = c + 1 < a.ntiles;
  const v4f PR = TL::d_to_r(s_t, P);
  v4f hin = mc_zero();  // the wave's carry-in, in every group
  v4f out;              // out_b = state after group b
  if constexpr (WG == 1) {
    if (publish && whard && b == 15) seg_publish(pub + me * 16, Q);  // group 15's Q is the wave's h_out
    if (!first0) {
      if (!seg_wait(pub + (me - 1) * 16, hdr, spin_limit(a.spin), hin)) hin = mc_nan();
    }
    out = sel4(hard, Q, TL::mm(PR, hin, Q));
    if (publish && !whard && b == 15) seg_publish(pub + me * 16, out);
  } else {
    // wave summaries F_u = group 15's inclusive (P, Q), copied to every group
    __shared__ v4f s_PD[WG][4], s_PR[WG][4], s_Q[WG][4], s_hin[4];
    __shared__ uint32_t s_fl[WG];
    const int q = (int)(threadIdx.x & 3);
    if (b == 15) {
      s_PD[w][q] = P;
      s_PR[w][q] = PR;
      s_Q[w][q] = Q;
    }
    if ((threadIdx.x & 63) == 0) s_fl[w] = (uint32_t)whard | ((uint32_t)first0 << 1);
    __syncthreads();
    // G = F_{w-1} o ... o F_0 in that order (PG = 0 once one of them is hard)
    v4f PG = mc_zero(), QG = mc_zero();
    bool have = false, hardG = false;
    for (int u = 0; u < w; ++u) {
      const v4f Qu = s_Q[u][q];
      if (s_fl[u] & 1u) {
        PG = mc_zero();
        QG = Qu;
        hardG = true;
      } else if (!have) {
        PG = s_PD[u][q];
        QG = Qu;
      } else {
        const v4f PuR = s_PR[u][q];
        if (!hardG) PG = TL::mm(PuR, PG, mc_zero());
        QG = TL::mm(PuR, QG, Qu);
      }
      have = true;
    }
    const bool need_in = (s_fl[0] & 2u) == 0u;  // unless the chunk's first step is hard
    const v4f PGR = (have && !hardG) ? TL::d_to_r(s_t, PG) : mc_zero();  // off the chain
    if (w == WG - 1) {
      // chunk summary F_w o G, published at once when it is hard
      v4f PC = s_PD[w][q], QC = s_Q[w][q];
      const bool hardC = whard || hardG;
      if (!whard && have) {
        const v4f PwR = s_PR[w][q];
        PC = hardG ? mc_zero() : TL::mm(PwR, PG, mc_zero());
        QC = TL::mm(PwR, QG, QC);
      }
      if (publish && hardC && b == 15) seg_publish(pub + me * 16, QC);
      const v4f PCR = (publish && !hardC) ? TL::d_to_r(s_t, PC) : mc_zero();  // off the chain
      v4f hc = mc_zero();
      if (need_in) {
        if (!seg_wait(pub + (me - 1) * 16, hdr, spin_limit(a.spin), hc)) hc = mc_nan();
      }
      const v4f hout = TL::mm(PCR, hc, QC);
      if (publish && !hardC && b == 15) seg_publish(pub + me * 16, hout);
      if ((threadIdx.x & 63) < 4) s_hin[q] = hc;
    }
    __syncthreads();
    const v4f hc = s_hin[q];
    if (w > 0 || need_in) hin = !have ? hc : hardG ? QG : TL::mm(PGR, hc, QG);
    out = sel4(hard, Q, TL::mm(PR, hin, Q));
  }
  v4f h = shfl_up4(out, 4);
  if (b == 0) h = hin;

  // ---- apply from the registers
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const bool first = (hardm >> s) & 1u;
    const v4f hn = TL::mm(X[s], h, Y[s]);
    h = sel4(first, Y[s], hn);  // h holds lam in the backward
    if constexpr (BWD) {
      const v4f lamR = TL::d_to_r(s_t, h);
      // dA = lam h_prev^T; FULL stores it as rows, computed as h_prev lam^T =
      // dA^T, whose D layout is the R layout of dA (no transpose)
      const v4f dAR = FULL ? TL::mm(H[s], lamR, mc_zero()) : TL::mm(lamR, H[s], mc_zero());
      if (s < nb) {
        const int64_t t = wk.phys(jb + s);
        if constexpr (FULL) {
          *(v4f*)(wk.blkB(a.out0, t) + TL::dc() * 4) = lamR;  // dB = lam
          *(v4f*)(wk.blkA(a.out1, t) + TL::dc() * 4) = dAR;
        } else {
          wk.sh.stB_D(wk.blkB(a.out0, t), h);  // dB = lam
          wk.sh.stA_D(wk.blkA(a.out1, t), dAR);
        }
      }
      const bool l = ((lastm >> s) & 1u) && s < nb;
      if (a.dh0 && __ballot(l) != 0ull) {
        // dh0 = A_s^T lam_s (A_s^T in R layout is A_s in D layout); 0 where
        // A_s = 0: nothing flows through a reset
        const v4f Ad = l ? wk.sh.ldA_D(wk.blkA(a.A, wk.phys(jb + s))) : mc_zero();
        wait_stage_loads();
        const v4f d = TL::mm(Ad, h, mc_zero());
        const bool reset = TL::zero(Ad);
        if (l) wk.sh.stB_D(a.dh0 + ((int64_t)wk.seg_of(jb + s) * a.rows + r) * wk.sh.nb(), reset ? mc_zero() : d);
      }
    } else {
      if constexpr (FULL) {
        const v4f hR = TL::d_to_r(s_t, h);
        if (s < nb) *(v4f*)(wk.blkB(a.out0, wk.phys(jb + s)) + TL::dc() * 4) = hR;
      } else {
        if (s < nb) wk.sh.stB_D(wk.blkB(a.out0, wk.phys(jb + s)), h);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host
// ---------------------------------------------------------------------------
// Steps per wave (kChunk) and waves per chunk (kWaves; a chunk is kWaves x
// kChunk steps), from timing at (16, 16), 512 rows, T = 4096, flushed.
// Forward, waves x steps: 1 x 32 1.24 ms (one wave per SIMD), 2 x 32 1.35,
// 4 x 32 1.54, 2 x 16 1.19, 4 x 8 1.19, 4 x 12 1.21, 8 x 8 1.11, 8 x 16 1.42,
// 4 x 16 1.09-1.11 (two waves per SIMD, a 64-step chunk). Backward, operands
// in registers: 1 x 16 2.24 ms, 2 x 16 2.21, 4 x 16 2.60, 4 x 8 3.62, 8 x 8
// 2.72 (32 steps per wave spill); with A and dy staged in LDS: 2 x 16
// 2.13 ms against 2.14-2.15 in registers, 1 x 16 2.21, 4 x 16 2.44, 2 x 8 3.56,
// 4 x 8 3.69, 4 x 4 2.41. Shapes that keep more chunks resident than there are
// rows (512 here) put chunks of one row side by side, each waiting for the one
// before it.
constexpr int kChunkFwd = 16, kChunkBwd = 16;
constexpr int kWavesFwd = 4, kWavesBwd = 2;
// Steps per lane group of the 4 x 4 row-segment kernel (a wave spans 16 x that),
// from timing 4 / 8 / 16 / 24 / 32 at (4, 4), 4096 rows x T = 8192: 16 and 32
// tie (forward 1.27 ms, backward 2.19 ms; 8 took 1.37 / 2.46 ms) and 32 spills
// in the backward. A backward of 8 steps per group at two waves per SIMD, 2 or
// 4 waves per chunk, chunks in groups of 2 to 8, took 2.30-2.38 ms against
// 2.17 ms.
constexpr int kSegStepsFwd = 16, kSegStepsBwd = 16;
// Waves per chunk of the row-segment kernel (a chunk is kSegWaves x 16 x
// kSegSteps steps).
constexpr int kSegWavesFwd = 4, kSegWavesBwd = 1;

static bool tile4_shape(int k, int v) { return k <= 4 && v <= 4; }

int64_t matrix_core_chunks(int64_t T, bool bwd, int k, int v) {
  const int64_t S = tile4_shape(k, v) ? (bwd ? kSegWavesBwd * 16 * kSegStepsBwd : kSegWavesFwd * 16 * kSegStepsFwd)
                                      : (bwd ? kWavesBwd * kChunkBwd : kWavesFwd * kChunkFwd);
  return (T + S - 1) / S;
}

size_t matrix_core_ws_bytes(int64_t rows, int64_t T, int k, int v) {
  const int64_t n = std::max(matrix_core_chunks(T, false, k, v), matrix_core_chunks(T, true, k, v));
  return ws_desc_offset() + (size_t)(rows * n) * (tile4_shape(k, v) ? kSegPubBytes : kMcPubBytes);
}

template <class TL, bool FULL, bool BWD, bool REV, bool VARLEN, int S, int WG>
static hipError_t launch_mc_dir(const MatArgs& a0, hipStream_t st) {
  MatArgs a = a0;
  a.ntiles = (int32_t)((a.T + WG * S - 1) / (WG * S));
  const int64_t n = a.rows * a.ntiles;
  // fresh words (and header) for this call: a zero tag = not published
  const hipError_t z = launch_zero(a.ws, ws_desc_offset() + (size_t)n * kMcPubBytes, st);
  if (z != hipSuccess) return z;
  hipLaunchKernelGGL((k_mc_scan<TL, FULL, BWD, REV, VARLEN, S, WG>), dim3(launch_blocks((uint64_t)n, a.nblk)),
                     dim3(64 * WG), 0, st, a);
  return hipGetLastError();
}

template <bool FULL, bool BWD, bool REV, bool VARLEN, int S, int WG>
static hipError_t launch_seg_dir(const MatArgs& a0, hipStream_t st) {
  MatArgs a = a0;
  a.ntiles = (int32_t)((a.T + WG * 16 * S - 1) / (WG * 16 * S));
  const int64_t n = a.rows * a.ntiles;
  const hipError_t z = launch_zero(a.ws, ws_desc_offset() + (size_t)n * kSegPubBytes, st);
  if (z != hipSuccess) return z;
  hipLaunchKernelGGL((k_mc_rowseg<FULL, BWD, REV, VARLEN, S, WG>), dim3(launch_blocks((uint64_t)n, a.nblk)),
                     dim3(64 * WG), 0, st, a);
  return hipGetLastError();
}

template <class TL, bool FULL>
static hipError_t launch_mc_shape(const MatArgs& a, bool bwd, hipStream_t st) {
  constexpr int SF = kChunkFwd, SB = kChunkBwd, WF = kWavesFwd, WB = kWavesBwd;
  const bool rev = a.rev != 0, vl = a.cu != nullptr;
  if (bwd) {
    if (rev) return vl ? launch_mc_dir<TL, FULL, true, true, true, SB, WB>(a, st) : launch_mc_dir<TL, FULL, true, true, false, SB, WB>(a, st);
    return vl ? launch_mc_dir<TL, FULL, true, false, true, SB, WB>(a, st) : launch_mc_dir<TL, FULL, true, false, false, SB, WB>(a, st);
  }
  if (rev) return vl ? launch_mc_dir<TL, FULL, false, true, true, SF, WF>(a, st) : launch_mc_dir<TL, FULL, false, true, false, SF, WF>(a, st);
  return vl ? launch_mc_dir<TL, FULL, false, false, true, SF, WF>(a, st) : launch_mc_dir<TL, FULL, false, false, false, SF, WF>(a, st);
}

template <bool FULL>
static hipError_t launch_seg_shape(const MatArgs& a, bool bwd, hipStream_t st) {
  constexpr int SF = kSegStepsFwd, SB = kSegStepsBwd, WF = kSegWavesFwd, WB = kSegWavesBwd;
  const bool rev = a.rev != 0, vl = a.cu != nullptr;
  if (bwd) {
    if (rev) return vl ? launch_seg_dir<FULL, true, true, true, SB, WB>(a, st) : launch_seg_dir<FULL, true, true, false, SB, WB>(a, st);
    return vl ? launch_seg_dir<FULL, true, false, true, SB, WB>(a, st) : launch_seg_dir<FULL, true, false, false, SB, WB>(a, st);
  }
  if (rev) return vl ? launch_seg_dir<FULL, false, true, true, SF, WF>(a, st) : launch_seg_dir<FULL, false, true, false, SF, WF>(a, st);
  return vl ? launch_seg_dir<FULL, false, false, true, SF, WF>(a, st) : launch_seg_dir<FULL, false, false, false, SF, WF>(a, st);
}

hipError_t launch_matrix_core(const MatArgs& a, bool bwd, hipStream_t st) {
  if (a.k < 1 || a.k > 16 || a.v < 1 || a.v > 16) return hipErrorInvalidValue;
  if (tile4_shape(a.k, a.v)) {
    if (a.k == 4 && a.v == 4) return launch_seg_shape<true>(a, bwd, st);
    return launch_seg_shape<false>(a, bwd, st);
  }
  if (a.k == 16 && a.v == 16) return launch_mc_shape<Tile16, true>(a, bwd, st);
  return launch_mc_shape<Tile16, false>(a, bwd, st);
}

}  // namespace mscan
