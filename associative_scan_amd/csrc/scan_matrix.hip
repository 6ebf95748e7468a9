// Matrix-affine scan kernels: h_t = A_t h_{t-1} + B_t with A_t k x k and B_t,
// h_t k x v ("Triton scan kernels", "One associative-scan family": matrix_scan
// is k = 2, v = 1 and matrix_affine_scan is generic (k, v)), and the reverse
// adjoint (same page, "Autograd integration and the reversed-scan backward":
// reverse-scan the output gradients with A_{t+1}^T, then form dA_t from the
// forward state before t).
//
// Every product here is a 2x2 or 4x4 block on the VALU in IEEE fp32; the path
// is bound by HBM bandwidth and the blocks are far too small for matrix cores,
// and fp32 VALU keeps the precision the page's precision guard asks for.
//
// Work decomposition. A wave owns a window of 64 x EL consecutive time steps;
// a tile is WAVES such windows. Each array of the window (A, B or dy, h) is
// staged in LDS:
//   - global -> LDS by direct loads (global_load_lds), 1 KiB per wave
//     instruction, so HBM sees only fully coalesced 16-byte accesses and no
//     VGPR holds data in flight;
//   - lane l owns EL consecutive steps and reads them from LDS; the 16-byte
//     units are XOR-swizzled (a permutation inside each aligned group of 16
//     units) so that those lane-owned reads hit distinct banks, while every
//     load or store instruction still covers one aligned block of memory;
//   - outputs are written back into the slots of the inputs they replace and
//     leave LDS with coalesced 16-byte stores.
// Inside a tile the steps are summarised per lane as (P, Q) = (product of the
// A's, accumulated B's), scanned across the wave with DPP and across waves
// through LDS; across tiles the scalar kernels' two modes apply unchanged
// (a row that fits one tile on its own, longer rows chained by look-back;
// see scan_scalar_kernel.hpp).
//
// Tiles are aligned to the row start in both directions; with `reverse` the
// row is processed from its last tile down, each tile from its last window,
// each window from lane 63's block, each block from its last step.
//
// Backward: processing order is the reverse of the forward's; element j is
// (A of the step before it in that order, transposed; dy_j), a sequence's
// first element is (0, dy). Outputs dB = lam, dA_t = lam_t h_prev^T with
// h_prev the forward state before t (h0 at a sequence start), and
// dh0 = A_s^T lam_s at each sequence's forward-first step s.
#include <type_traits>

#include "mscan_device.hpp"
#include "mscan_launch.hpp"

namespace mscan {

// ---------------------------------------------------------------------------
// k x k transition / k x v state algebra
// ---------------------------------------------------------------------------
template <int K, int V>
struct MatOps {
  static constexpr int KK = K * K, KV = K * V, NS = KK + KV, NC = KV;
  struct S { float v[NS]; };  // P (row-major k x k) then Q (row-major k x v)
  struct C { float v[NC]; };  // state h (row-major k x v)

  __device__ static __forceinline__ S ident() {
    S s;
#pragma unroll
    for (int i = 0; i < KK; ++i) s.v[i] = (i % (K + 1) == 0) ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < KV; ++i) s.v[KK + i] = 0.f;
    return s;
  }
  __device__ static __forceinline__ C cident() {
    C c;
#pragma unroll
    for (int i = 0; i < KV; ++i) c.v[i] = 0.f;
    return c;
  }
  __device__ static __forceinline__ bool zero_k(const float* p) {
    bool z = true;
#pragma unroll
    for (int i = 0; i < KK; ++i) z = z && (p[i] == 0.f);
    return z;
  }
  __device__ static __forceinline__ bool hard(const S& s) { return zero_k(s.v); }
  // out = M * X (+ add) for M k x k and X k x n, row-major
  template <int N>
  __device__ static __forceinline__ void mul(const float* M, const float* X, const float* add, float* out) {
#pragma unroll
    for (int i = 0; i < K; ++i)
#pragma unroll
      for (int c = 0; c < N; ++c) {
        float acc = add ? add[i * N + c] : 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) acc = __builtin_fmaf(M[i * K + j], X[j * N + c], acc);
        out[i * N + c] = acc;
      }
  }
  // s := (M sP, M sQ + add), one row of the result at a time (row i needs
  // only row i of M, and all of s, so rows are written after all are formed)
  __device__ static __forceinline__ void premul(const float* M, S& s, const float* add) {
    S r;
    mul<K>(M, s.v, nullptr, r.v);
    mul<V>(M, s.v + KK, add, r.v + KK);
    s = r;
  }
  // l := (e then l) = (lP eP, lP eQ + lQ), in place one row of l at a time
  // (row i of the result needs only row i of l); a zero l.P keeps l (a reset
  // or a sequence start)
  __device__ static __forceinline__ void compose(const S& e, S& l) {
    if (zero_k(l.v)) return;
#pragma unroll
    for (int i = 0; i < K; ++i) {
      float rp[K], rq[V];
#pragma unroll
      for (int c = 0; c < K; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < K; ++j) acc = __builtin_fmaf(l.v[i * K + j], e.v[j * K + c], acc);
        rp[c] = acc;
      }
#pragma unroll
      for (int c = 0; c < V; ++c) {
        float acc = l.v[KK + i * V + c];
#pragma unroll
        for (int j = 0; j < K; ++j) acc = __builtin_fmaf(l.v[i * K + j], e.v[KK + j * V + c], acc);
        rq[c] = acc;
      }
#pragma unroll
      for (int c = 0; c < K; ++c) l.v[i * K + c] = rp[c];
#pragma unroll
      for (int c = 0; c < V; ++c) l.v[KK + i * V + c] = rq[c];
    }
  }
  __device__ static __forceinline__ C apply(const S& s, const C& c) {
    C r;
    if (zero_k(s.v)) {
#pragma unroll
      for (int i = 0; i < KV; ++i) r.v[i] = s.v[KK + i];
    } else {
      mul<V>(s.v, c.v, s.v + KK, r.v);
    }
    return r;
  }
  __device__ static __forceinline__ S of_carry(const C& c) {
    S s;
#pragma unroll
    for (int i = 0; i < KK; ++i) s.v[i] = 0.f;
#pragma unroll
    for (int i = 0; i < KV; ++i) s.v[KK + i] = c.v[i];
    return s;
  }
  __device__ static __forceinline__ C carry_of_hard(const S& s) {
    C c;
#pragma unroll
    for (int i = 0; i < KV; ++i) c.v[i] = s.v[KK + i];
    return c;
  }
};

// n floats from global memory (plain loads; h0 / halo values)
template <int N>
__device__ __forceinline__ void gload(const float* p, float* o) {
#pragma unroll
  for (int i = 0; i < N; ++i) o[i] = p[i];
}

// Largest i in [0, n) with at(i) <= q (0 if none).
template <class At>
__device__ __forceinline__ int seg_find(const At& at, int n, int64_t q) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (at(mid) <= q) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kMatCuLds = 1024;  // cu_seqlens entries cached in LDS per workgroup
enum : int { kMatSingle = 0, kMatLookback = 1 };

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int K, int V, bool BWD, bool REV, bool VARLEN, int MODE, int WAVES, int EL>
__global__ __launch_bounds__(WAVES * 64) void k_matrix(const MatArgs a) {
  using Ops = MatOps<K, V>;
  using S = typename Ops::S;
  using C = typename Ops::C;
  constexpr int KK = K * K, KV = K * V, NS = Ops::NS, NC = Ops::NC, ND = NS + NC;
  constexpr int WSTEPS = 64 * EL;       // steps per wave window
  constexpr int TILE = WAVES * WSTEPS;  // steps per tile
  using SA = Stage<KK, EL>;             // A
  using SB = Stage<KV, EL>;             // B (forward) / dy (backward)
  using SH = Stage<KV, EL>;             // h (backward)
  constexpr int HALO = BWD ? (KK + KV + 3) / 4 * 4 : 0;  // whole 16-byte units
  constexpr int WFLOATS = SA::FLOATS + SB::FLOATS + (BWD ? SH::FLOATS : 0) + HALO;

  __shared__ __attribute__((aligned(16))) float s_stage[WAVES][WFLOATS];
  __shared__ float s_agg[WAVES][NS];
  __shared__ float s_carry[NC];
  __shared__ int32_t s_cu[VARLEN ? kMatCuLds : 1];

  const int l = lane_id();
  const int w = (int)(threadIdx.x >> 6);
  // one tile per workgroup: the row's only tile, or tile c of a chained row
  int64_t r;
  int c;
  if constexpr (MODE == kMatSingle) {
    r = blockIdx.x;
    c = 0;
  } else {
    // tile-major, except the k = 2 backward, which streams faster row-major
    // (4096 rows x T = 8192: (2,1) 0.341 vs 0.360 ms, (2,2) 0.491 vs 0.546 ms;
    // the (4,1) backward is 19% slower that way)
    tile_of_block<!(BWD && K == 2)>(a.rows, a.ntiles, a.blk0, r, c);
  }
  const int64_t T = a.T;
  const int64_t row0 = r * a.stride;  // first step of the row
  const bool has_h0 = a.h0 != nullptr;
  // the k x v arrays of this row start 16-byte aligned (the k x k ones always do)
  const bool vecB = ((row0 * KV) & 3) == 0;

  float* stA = s_stage[w];
  float* stB = stA + SA::FLOATS;
  float* stH = stB + SB::FLOATS;
  float* halo = stB + SB::FLOATS + (BWD ? SH::FLOATS : 0);  // bwd: A before, h after the window

  Workspace ws{};
  if constexpr (MODE == kMatLookback) ws = ws_view(a.ws);

  // h0 of sequence k for this row (zero when absent)
  auto load_h0 = [&](int k, float* o) {
    if (has_h0) gload<KV>(a.h0 + ((int64_t)k * a.rows + r) * KV, o);
    else {
#pragma unroll
      for (int i = 0; i < KV; ++i) o[i] = 0.f;
    }
  };

  bool cu_lds = false;  // the table is in s_cu (else read from global memory)
  const int ncu = a.nseg + 1;

  C carry = Ops::cident();  // state entering the tile
  {
    // physical window of this wave: tile pc, window pw (mirrored for reverse)
    const int pc = REV ? a.ntiles - 1 - c : c;
    const int pw = REV ? WAVES - 1 - w : w;
    const int64_t wlo = (int64_t)pc * TILE + (int64_t)pw * WSTEPS;  // first step of the window
    const int nv = (int)max((int64_t)0, min((int64_t)WSTEPS, T - wlo));  // valid steps

    // ---- stage the window ------------------------------------------------
    if (nv > 0) {
      SA::load(a.A + (row0 + wlo) * KK, stA, nv * KK, true);
      SB::load(a.B + (row0 + wlo) * KV, stB, nv * KV, vecB);
      if constexpr (BWD) SH::load(a.hs + (row0 + wlo) * KV, stH, nv * KV, vecB);
    }
    if constexpr (BWD) {
      // A of the step before the window and h of the step after it, in
      // processing order (zero outside the row)
      const int64_t tA = REV ? wlo + WSTEPS : wlo - 1;
      const int64_t tH = REV ? wlo - 1 : wlo + WSTEPS;
      if (l < KK) halo[l] = (tA >= 0 && tA < T) ? a.A[(row0 + tA) * KK + l] : 0.f;
      if (l < KV) halo[KK + l] = (tH >= 0 && tH < T) ? a.hs[(row0 + tH) * KV + l] : 0.f;
    }
    // the sequence table, once per workgroup (after the window loads are in
    // flight, so its latency overlaps theirs)
    if constexpr (VARLEN) {
      if (ncu <= kMatCuLds) {
        for (int i = threadIdx.x; i < ncu; i += WAVES * 64) s_cu[i] = a.cu[i];
        __syncthreads();
        cu_lds = true;
      }
    }
    wait_stage_loads();

    // lane-owned steps: processing element e <-> window step sidx(e)
    auto sidx = [&](int e) -> int { return REV ? (63 - l) * EL + (EL - 1 - e) : l * EL + e; };
    const int64_t tlane = wlo + (REV ? (63 - l) * EL : l * EL);  // lowest step of the lane

    // ---- sequence boundaries ------------------------------------------------
    // first: a sequence's first step in processing order; last: its last one
    uint32_t firstm = 0, lastm = 0;
    int segk[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) segk[e] = 0;
    if constexpr (!VARLEN) {
      const int64_t tf = REV ? T - 1 : 0, tl = REV ? 0 : T - 1;
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int64_t t = wlo + sidx(e);
        if (t == tf) firstm |= 1u << e;
        if (t == tl) lastm |= 1u << e;
      }
    } else {
      // instantiated for the LDS copy and for global memory, chosen by a
      // uniform flag (a pointer that could be either compiles to flat loads,
      // whose waits also wait for the window's outstanding loads)
      auto walk = [&](auto in_lds) {
        auto cuv = [&](int i) -> int64_t {
          if constexpr (decltype(in_lds)::value) return (int64_t)s_cu[i];
          else return (int64_t)a.cu[i];
        };
        int k = seg_find(cuv, ncu, max(tlane, (int64_t)0));
#pragma unroll
        for (int ep = 0; ep < EL; ++ep) {
          const int64_t q = tlane + ep;
          if (q >= T) continue;
          while (k + 1 < ncu && cuv(k + 1) <= q) ++k;
          const bool is_start = cuv(k) == q;
          const bool is_end = (k + 1 < ncu) && (cuv(k + 1) - 1 == q);
          const int e = REV ? EL - 1 - ep : ep;
          segk[e] = min(max(k, 0), a.nseg - 1);
          if (REV ? is_end : is_start) firstm |= 1u << e;
          if (REV ? is_start : is_end) lastm |= 1u << e;
        }
      };
      if (cu_lds) walk(std::true_type{});
      else walk(std::false_type{});
    }
    auto valid = [&](int e) -> bool { return wlo + sidx(e) < T; };

    // ---- element e of the scan, in processing order ------------------------------
    // fwd: X = A_t, Y = B_t; a sequence start becomes (0, A h0 + B).
    // bwd: X = (A of the previous step in processing order)^T, Y = dy_t; a
    //      sequence start becomes (0, dy).
    // A of processing element e - 1 (bwd): window step sidx(e) -/+ 1, or the halo
    auto prevA = [&](int e, float* o) {
      const int s = REV ? sidx(e) + 1 : sidx(e) - 1;
      if (s < 0 || s >= WSTEPS) {
#pragma unroll
        for (int i = 0; i < KK; ++i) o[i] = halo[i];
      } else {
        SA::get(stA, s, o);
      }
    };
    // h of processing element e + 1 (bwd): the forward state before step t
    auto nextH = [&](int e, float* o) {
      const int sn = REV ? sidx(e) - 1 : sidx(e) + 1;
      if (sn < 0 || sn >= WSTEPS) {
#pragma unroll
        for (int i = 0; i < KV; ++i) o[i] = halo[KK + i];
      } else {
        SH::get(stH, sn, o);
      }
    };
    // (X, Y) of element e; false for a step outside the row (identity)
    auto element = [&](int e, float* X, float* Y) -> bool {
      if (!valid(e)) return false;
      const int s = sidx(e);
      const bool first = firstm & (1u << e);
      if constexpr (!BWD) {
        SA::get(stA, s, X);
        SB::get(stB, s, Y);
        if (first) {
          // A h0 + B, or B alone where A = 0 (a reset drops h0)
          if (!Ops::zero_k(X)) {
            float h0v[KV], y[KV];
            load_h0(segk[e], h0v);
            Ops::template mul<V>(X, h0v, Y, y);
#pragma unroll
            for (int i = 0; i < KV; ++i) Y[i] = y[i];
          }
#pragma unroll
          for (int i = 0; i < KK; ++i) X[i] = 0.f;
        }
      } else {
        SB::get(stB, s, Y);
        if (first) {
#pragma unroll
          for (int i = 0; i < KK; ++i) X[i] = 0.f;
        } else {
          float Ap[KK];
          prevA(e, Ap);
#pragma unroll
          for (int p = 0; p < K; ++p)
#pragma unroll
            for (int q = 0; q < K; ++q) X[p * K + q] = Ap[q * K + p];
        }
      }
      return true;
    };

    // ---- lane-serial summary ------------------------------------------------------
    S sum = Ops::ident();
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      float X[KK], Y[KV];
      if (!element(e, X, Y)) continue;
      if (Ops::zero_k(X)) {
#pragma unroll
        for (int i = 0; i < KK; ++i) sum.v[i] = 0.f;
#pragma unroll
        for (int i = 0; i < KV; ++i) sum.v[KK + i] = Y[i];
      } else {
        Ops::premul(X, sum, Y);
      }
    }
    // ---- wave scan --------------------------------------------------------------
    scan_step<Ops, kRowShr1, 0xf>(sum, (l & 15) >= 1);
    scan_step<Ops, kRowShr2, 0xf>(sum, (l & 15) >= 2);
    scan_step<Ops, kRowShr4, 0xf>(sum, (l & 15) >= 4);
    scan_step<Ops, kRowShr8, 0xf>(sum, (l & 15) >= 8);
    scan_step<Ops, kRowBcast15, 0xa>(sum, (l & 16) != 0);
    scan_step<Ops, kRowBcast31, 0xc>(sum, l >= 32);
    S wagg;
#pragma unroll
    for (int i = 0; i < NS; ++i) wagg.v[i] = readlane_f(sum.v[i], 63);

    // ---- across waves ---------------------------------------------------------------
    // tile aggregate = the waves' aggregates in order; a wave's lanes prepend
    // the waves before it to their own summaries (so only `sum` stays live
    // through the look-back)
    auto tile_agg = [&]() -> S {
      S t = Ops::ident();
#pragma unroll
      for (int q = 0; q < WAVES; ++q) {
        S x;
#pragma unroll
        for (int i = 0; i < NS; ++i) x.v[i] = s_agg[q][i];
        Ops::compose(t, x);
        t = x;
      }
      return t;
    };
    // composition of the waves before this one
    auto waves_before = [&]() -> S {
      S ex = Ops::ident();
      for (int q = 0; q < w; ++q) {
        S x;
#pragma unroll
        for (int i = 0; i < NS; ++i) x.v[i] = s_agg[q][i];
        Ops::compose(ex, x);
        ex = x;
      }
      return ex;
    };
    if constexpr (WAVES > 1) {
      if (l == 0) {
#pragma unroll
        for (int i = 0; i < NS; ++i) s_agg[w][i] = wagg.v[i];
      }
      __syncthreads();
      if (w > 0) Ops::compose(waves_before(), sum);
    }

    // ---- across tiles: decoupled look-back ------------------------------------------
    if constexpr (MODE == kMatLookback) {
      uint64_t* rd = ws.desc + (int64_t)ND * ((int64_t)r * a.ntiles);
      uint64_t* my = rd + (int64_t)ND * c;
      if (w == 0) {
        const uint32_t tagA = kTagAgg, tagI = kTagIncl;
        bool hard;
        {
          const S tagg = (WAVES > 1) ? tile_agg() : wagg;
          hard = Ops::hard(tagg);
          stress_pause(1);
          if (l == 0) {
            if (!hard) {
#pragma unroll
              for (int i = 0; i < NS; ++i) st_u64(my + i, pack_word(tagA, tagg.v[i]));
            } else {
              const C inc = Ops::carry_of_hard(tagg);
#pragma unroll
              for (int i = 0; i < NC; ++i) st_u64(my + NS + i, pack_word(tagI, inc.v[i]));
            }
          }
        }
        if (c > 0) carry = lookback<Ops, true>(ws, rd, c, spin_limit(a.spin));
        stress_pause(2);
        if (l == 0) {
          if (!hard) {
            const S tagg = (WAVES > 1) ? tile_agg() : wagg;
            const C inc = Ops::apply(tagg, carry);
#pragma unroll
            for (int i = 0; i < NC; ++i) st_u64(my + NS + i, pack_word(tagI, inc.v[i]));
          }
#pragma unroll
          for (int i = 0; i < NC; ++i) s_carry[i] = carry.v[i];
        }
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < NC; ++i) carry.v[i] = s_carry[i];
    }

    // ---- apply: each step from its exact carry-in, outputs into the staging slots
    {
      // state entering this wave's window (lane 0) and after this lane
      C hw = carry;
      if constexpr (WAVES > 1) {
        if (w > 0) hw = Ops::apply(waves_before(), carry);
      }
      const C v = Ops::apply(sum, carry);
      C st;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        st.v[i] = __shfl_up(v.v[i], 1, 64);
        if (l == 0) st.v[i] = hw.v[i];
      }
      // bwd: the lane's first A_prev is read before any lane overwrites its A
      // slots with dA (all lanes run this code in step)
      float Aown[BWD ? KK : 1];
      if constexpr (BWD) prevA(0, Aown);
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        if (!valid(e)) continue;
        const int s = sidx(e);
        const bool first = firstm & (1u << e);
        float Y[KV];
        SB::get(stB, s, Y);
        if constexpr (!BWD) {
          float X[KK];
          SA::get(stA, s, X);
          if (first && !Ops::zero_k(X)) {
            float h0v[KV], y[KV];
            load_h0(segk[e], h0v);
            Ops::template mul<V>(X, h0v, Y, y);
#pragma unroll
            for (int i = 0; i < KV; ++i) st.v[i] = y[i];
          } else if (Ops::zero_k(X)) {
#pragma unroll
            for (int i = 0; i < KV; ++i) st.v[i] = Y[i];
          } else {
            C nx;
            Ops::template mul<V>(X, st.v, Y, nx.v);
            st = nx;
          }
          SB::put(stB, s, st.v);  // h over B
        } else {
          // Aown holds A of the previous processing step; X = its transpose
          float X[KK];
#pragma unroll
          for (int p = 0; p < K; ++p)
#pragma unroll
            for (int q = 0; q < K; ++q) X[p * K + q] = first ? 0.f : Aown[q * K + p];
          if (first || Ops::zero_k(X)) {
#pragma unroll
            for (int i = 0; i < KV; ++i) st.v[i] = Y[i];
          } else {
            C nx;
            Ops::template mul<V>(X, st.v, Y, nx.v);
            st = nx;
          }
          SA::get(stA, s, Aown);  // own A: dh0 below, and the next element's X
          float N[KV];
          if (lastm & (1u << e)) load_h0(segk[e], N);
          else nextH(e, N);
          // dA_t = lam_t h_prev^T (k x k)
          float dA[KK];
#pragma unroll
          for (int p = 0; p < K; ++p)
#pragma unroll
            for (int q = 0; q < K; ++q) {
              float acc = 0.f;
#pragma unroll
              for (int u = 0; u < V; ++u) acc = __builtin_fmaf(st.v[p * V + u], N[q * V + u], acc);
              dA[p * K + q] = acc;
            }
          SB::put(stB, s, st.v);  // dB = lam over dy
          SA::put(stA, s, dA);    // dA over A
          if (a.dh0 && (lastm & (1u << e))) {
            // dh0 = A_s^T lam_s (0 where A_s = 0: nothing flows through a reset)
            float* dst = a.dh0 + ((int64_t)segk[e] * a.rows + r) * KV;
            const bool reset = Ops::zero_k(Aown);
#pragma unroll
            for (int p = 0; p < K; ++p)
#pragma unroll
              for (int u = 0; u < V; ++u) {
                float acc = 0.f;
#pragma unroll
                for (int q = 0; q < K; ++q) acc = __builtin_fmaf(Aown[q * K + p], st.v[q * V + u], acc);
                dst[p * V + u] = reset ? 0.f : acc;
              }
          }
        }
      }
    }
    // ---- store ----------------------------------------------------------------------
    wave_lds_sync();
    if (nv > 0) {
      SB::store(a.out0 + (row0 + wlo) * KV, stB, nv * KV, vecB);
      if constexpr (BWD) SA::store(a.out1 + (row0 + wlo) * KK, stA, nv * KK, true);
    }
  }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------
template <int K, int V>
struct MatCfg;
// waves per workgroup and steps per lane, forward (WF, EF) and backward
// (WB, EB), from timing sweeps at 4096 rows x T = 8192 (the (2, 1) shapes
// again with nontemporal staged loads and a 1 GiB write before every timed
// call: forward 4 x 8 0.184 ms, 8 x 4 0.190, 2 x 8 0.194, 4 x 4 0.194, 8 x 8
// 0.31; backward 4 x 4 0.343 ms, 2 x 4 0.345, 2 x 8 0.36, 4 x 2 0.37, 8 x 4
// 0.38)
template <> struct MatCfg<2, 1> { static constexpr int WF = 4, EF = 8, WB = 4, EB = 4; };
template <> struct MatCfg<2, 2> { static constexpr int WF = 4, EF = 4, WB = 4, EB = 2; };
template <> struct MatCfg<4, 1> { static constexpr int WF = 1, EF = 4, WB = 2, EB = 2; };

template <int K, int V>
int64_t matrix_tile_steps(bool bwd) {
  return bwd ? (int64_t)MatCfg<K, V>::WB * 64 * MatCfg<K, V>::EB
             : (int64_t)MatCfg<K, V>::WF * 64 * MatCfg<K, V>::EF;
}

template <int K, int V, bool BWD, bool REV>
static hipError_t launch_mat(const MatArgs& a0, hipStream_t st) {
  constexpr int W = BWD ? MatCfg<K, V>::WB : MatCfg<K, V>::WF;
  constexpr int E = BWD ? MatCfg<K, V>::EB : MatCfg<K, V>::EF;
  MatArgs a = a0;
  a.ntiles = (int32_t)((a.T + W * 64 * E - 1) / (W * 64 * E));
  const bool lookback = scalar_uses_lookback(a.rows, a.ntiles);
  const bool varlen = a.cu != nullptr;
  const dim3 block(W * 64);
  if (!lookback) {
    const dim3 grid((unsigned)a.rows);
    if (varlen) hipLaunchKernelGGL((k_matrix<K, V, BWD, REV, true, kMatSingle, W, E>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_matrix<K, V, BWD, REV, false, kMatSingle, W, E>), grid, block, 0, st, a);
  } else {
    // fresh descriptors for this call (zero tag = not published)
    const size_t words = (size_t)a.rows * (size_t)a.ntiles * (size_t)(MatOps<K, V>::NS + MatOps<K, V>::NC);
    const hipError_t z = launch_zero(a.ws, ws_desc_offset() + words * sizeof(uint64_t), st);
    if (z != hipSuccess) return z;
    const dim3 grid(launch_blocks((uint64_t)a.rows * (uint64_t)a.ntiles, a.nblk));
    if (varlen) hipLaunchKernelGGL((k_matrix<K, V, BWD, REV, true, kMatLookback, W, E>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_matrix<K, V, BWD, REV, false, kMatLookback, W, E>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

template <int K, int V>
static hipError_t launch_kv(const MatArgs& a, bool bwd, hipStream_t st) {
  if (bwd) return a.rev ? launch_mat<K, V, true, true>(a, st) : launch_mat<K, V, true, false>(a, st);
  return a.rev ? launch_mat<K, V, false, true>(a, st) : launch_mat<K, V, false, false>(a, st);
}

static bool envelope_size(int n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

// (4, 4) moved to the matrix cores, which measured 15% / 6% faster forward /
// backward at 4096 rows x T = 8192 (this kernel is bound by its 4x4 DPP
// compositions there).
bool matrix_valu_shape(int k, int v) { return (k == 2 && (v == 1 || v == 2)) || (k == 4 && v == 1); }

bool matrix_core_shape(int k, int v) {
  return envelope_size(k) && envelope_size(v) && !(k == 1 && v == 1) && !matrix_valu_shape(k, v);
}

int64_t matrix_tiles(int64_t T, int k, int v, bool bwd) {
  int64_t tile = 0;
  if (k == 2 && v == 1) tile = matrix_tile_steps<2, 1>(bwd);
  else if (k == 2 && v == 2) tile = matrix_tile_steps<2, 2>(bwd);
  else if (k == 4 && v == 1) tile = matrix_tile_steps<4, 1>(bwd);
  else if (matrix_core_shape(k, v)) return matrix_core_chunks(T, bwd, k, v);
  else return 0;
  return (T + tile - 1) / tile;
}

hipError_t launch_matrix(const MatArgs& a, int k, int v, bool bwd, hipStream_t st) {
  if (k == 2 && v == 1) return launch_kv<2, 1>(a, bwd, st);
  if (k == 2 && v == 2) return launch_kv<2, 2>(a, bwd, st);
  if (k == 4 && v == 1) return launch_kv<4, 1>(a, bwd, st);
  if (matrix_core_shape(k, v)) {
    MatArgs b = a;
    b.k = k;
    b.v = v;
    return launch_matrix_core(b, bwd, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace mscan
