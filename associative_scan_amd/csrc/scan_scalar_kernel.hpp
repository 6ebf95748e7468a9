// Scalar affine scan kernels: forward h_t = g_t h_{t-1} + x_t and its adjoint.
//
// Forward: associative-scan-triton README, intro / quick start (the recurrence)
// and "how it works" (chunked scan with the running prefix carried across
// chunks, cu_seqlens packing, bidirectional branches).
// Backward: same README, "how it works" (d_tokens is a reverse scan on shifted
// gates; d_gates = shifted states * d_tokens), fused into one kernel that reads
// only the forward's inputs and outputs ("Triton scan kernels", "Autograd
// integration and the reversed-scan backward").
//
// Log-space backward ("Triton scan kernels": parallel_scan_log carries the
// same recurrence with a = e^{log a}, b = e^{log b}): the same adjoint scan with
// the gate exponentiated as it is loaded, and the outputs taken through exp by
// the chain rule: dlog_b = lam * b, dlog_a = lam * a * h_prev,
// dlog_h0 = lam * a * h0 (template flag LOGB).
//
// Gate logits (template GATE): the gate is computed from a logit z as it is
// loaded, so no separate pointwise pass writes and rereads it. The activations
// are the ones the pages' workloads draw gates with: g = sigmoid(z) for the
// linear scan (README benchmark inputs), log a = -softplus(z) for the log-space
// scan (minGRU "One associative-scan family": a positive coefficient in (0,1)).
// The backward recomputes the activation and returns dz = dg * f'(z).
//
// Both directions are the same affine scan run along a "processing order":
//   forward : element (a, b) = (g_t, x_t), order = time (reversed if reverse),
//             a sequence's first element becomes (0, g h0 + x);
//   backward: element (a, b) = (g of the previous element in the backward's
//             order, dy_t), order = opposite of the forward's, a sequence's
//             first element becomes (0, dy); outputs dx = lam,
//             dg = lam * (forward state before t, h0 at the sequence start),
//             dh0 = g * lam at the forward's first element of each sequence.
//
// Work decomposition. A tile = WAVES waves x SUBS sub-chunks x 64 lanes x EL
// elements, contiguous in memory (the lanes of a sub-chunk read consecutive
// 16-byte vectors). Inside a tile:
//   a lane    = EL consecutive elements, summarised serially into (P, Q),
//   a wave    = SUBS independent 64-lane DPP scans chained through lane 63,
//   the waves = chained through LDS.
// Across the tiles of a row, two modes:
//   one tile : a row that fits one tile, one workgroup per row (no workspace,
//              no inter-workgroup traffic; the launcher guarantees the fit);
//   look-back: one workgroup per tile; the tiles of a row chain by decoupled
//              look-back through the workspace. Used whenever a row spans
//              several tiles: it keeps more bytes in flight per CU than
//              walking a row's tiles in one workgroup, which measured slower
//              at every benchmark row count.
// The tile body below is written as a loop over a workgroup's tiles, which
// runs exactly once in both modes; with a constant trip count in the one-tile
// mode the compiler drops the loop, and with it the waits for loads of a
// previous iteration that its back edge made it assume (in the generated
// code: a wait for the backward's halo loads before the tile's own loads).
// Rows whose start is not 16-byte aligned are handled by aligning vector
// groups to absolute addresses and masking the elements outside the row.
#pragma once

#include <type_traits>

#include "mscan_device.hpp"
#include "mscan_launch.hpp"

namespace mscan {

// ---------------------------------------------------------------------------
// input element types
// ---------------------------------------------------------------------------
template <typename Tin>
struct InTraits;

template <>
struct InTraits<float> {
  static constexpr int VEC = 4;  // elements per vector load (16 bytes)
  __device__ static __forceinline__ void loadv(const float* p, float* o) {
    const v4f v = __builtin_nontemporal_load((const v4f*)p);  // streamed once
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
};

// bf16 bit patterns, widened exactly. Four elements (8 bytes) per lane and
// load, so that a lane's fp32 outputs are one 16-byte store and the stores of
// a wave stay fully coalesced (two 16-byte stores per lane, 32 bytes apart,
// measured markedly slower).
template <>
struct InTraits<uint16_t> {
  static constexpr int VEC = 4;
  __device__ static __forceinline__ void loadv(const uint16_t* p, float* o) {
    const v2u v = __builtin_nontemporal_load((const v2u*)p);  // streamed once
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) {
    return __uint_as_float((uint32_t)(*p) << 16);
  }
};

// fp16, widened exactly (every fp16 value is an fp32 value); the same 8-byte
// layout as bf16.
template <>
struct InTraits<_Float16> {
  static constexpr int VEC = 4;
  __device__ static __forceinline__ void loadv(const _Float16* p, float* o) {
    typedef _Float16 v4h __attribute__((ext_vector_type(4)));
    const v4h v = __builtin_nontemporal_load((const v4h*)p);  // streamed once
    o[0] = (float)v.x; o[1] = (float)v.y; o[2] = (float)v.z; o[3] = (float)v.w;
  }
  __device__ static __forceinline__ float load1(const _Float16* p) { return (float)(*p); }
};

// N consecutive elements starting at a vector-aligned address
template <typename T, int N>
__device__ __forceinline__ void load_span(const T* p, float (&o)[N]) {
  constexpr int V = InTraits<T>::VEC;
#pragma unroll
  for (int i = 0; i < N / V; ++i) InTraits<T>::loadv(p + i * V, o + i * V);
}

template <int N>
__device__ __forceinline__ void store_span(float* p, const float (&v)[N]) {
#pragma unroll
  for (int i = 0; i < N / 4; ++i) {
    const v4f t = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
    __builtin_nontemporal_store(t, (v4f*)(p + 4 * i));
  }
}

// ---------------------------------------------------------------------------
// cu_seqlens helpers
// ---------------------------------------------------------------------------
// Number of entries of the sorted array cu[0..n) that are <= key, by a 64-way
// wave-parallel search (every lane returns the same value).
__device__ __forceinline__ int wave_count_le(const int32_t* cu, int n, int64_t key) {
  const int l = lane_id();
  int lo = 0;
  while (n > 64) {
    const int step = (n + 63) / 64;
    const int idx = lo + l * step;
    const bool le = (idx < lo + n) && ((int64_t)cu[idx] <= key);
    const int cnt = __popcll(__ballot(le));
    if (cnt == 0) return lo;
    const int nlo = lo + (cnt - 1) * step + 1;
    const int hi = min(lo + cnt * step, lo + n);
    n = hi - nlo;
    lo = nlo;
    if (n <= 0) return lo;
  }
  const bool le = (l < n) && ((int64_t)cu[lo + l] <= key);
  return lo + __popcll(__ballot(le));
}

constexpr int kCuSlice = 1024;  // cu_seqlens entries cached in LDS per workgroup

// A run of cu_seqlens entries: in the workgroup's LDS copy (lds) or, for a
// slice too long for it, in global memory (g). The kernels read it through
// an accessor that names the array, so each read is an LDS or a global load:
// one pointer that could be either made every read a flat load, whose wait
// also waits for the tile's outstanding global loads.
struct SegSlice {
  const int32_t* g;  // slice values in global memory (when !lds)
  int n;             // entries
  int k0;            // absolute index of entry 0
  bool lds;          // entries in the workgroup's LDS copy
};

// Largest i in [0, n) with at(i) <= q (0 if none).
template <class At>
__device__ __forceinline__ int slice_find(int n, const At& at, int64_t q) {
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (at(mid) <= q) lo = mid; else hi = mid;
  }
  return lo;
}

enum : int { kRowLoop = 0, kLookback = 1 };
enum : int { kGateNone = 0, kGateSigmoid = 1, kGateNegSoftplus = 2 };

// sigmoid(z) = 1 / (1 + e^{-z}) with the hardware reciprocal (1 ulp; exactly 1
// at z = +inf and 0 at z = -inf). The correctly rounded reciprocal is an
// eleven-instruction division sequence that made the gated scans VALU-bound.
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.f + __expf(-z)); }
// log(1 + e^z) = max(z, 0) + log1p(u), u = e^{-|z|} in (0, 1], without overflow
// and without losing its tail for z << 0. log1p(u): for u < 1/16 the series
// u - u^2/2 + u^3/3 - u^4/4 + u^5/5 (truncation below u^6/6 < 1e-8 relative);
// otherwise log(1 + u), whose rounding of 1 + u costs at most ~1e-6 relative
// there, taken as ln 2 times the hardware base-2 logarithm: 1 + u lies in
// (1, 2], where that instruction needs none of the denormal and special-value
// handling a general logf wraps around it. Both branches are a few VALU ops,
// where log1pf's range reduction doubled the time of the (VALU-bound)
// log-space forward.
__device__ __forceinline__ float softplus_f(float z) {
  const float u = __expf(-fabsf(z));
  const float series = u * __builtin_fmaf(-u, __builtin_fmaf(-u, __builtin_fmaf(-u, __builtin_fmaf(-u, 0.2f, 0.25f),
                                                                               1.f / 3.f), 0.5f), 1.f);
  const float lg = __builtin_amdgcn_logf(1.f + u) * 0.693147180559945f;
  return fmaxf(z, 0.f) + (u < 0.0625f ? series : lg);
}

// The gate value the scan uses, from a loaded gate operand: the operand itself,
// the activation of a logit, and, for the log-space backward, a = e^{log a}.
template <int GATE, bool LOGB>
__device__ __forceinline__ float gate_value(float v) {
  if constexpr (GATE == kGateSigmoid) return sigmoid_f(v);                 // g = sigmoid(z)
  if constexpr (GATE == kGateNegSoftplus) return LOGB ? sigmoid_f(-v)      // a = e^{-softplus(z)}
                                                      : -softplus_f(v);    // log a = -softplus(z)
  return LOGB ? __expf(v) : v;
}

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <class Ops, typename Tin, bool BWD, bool REV, bool VARLEN, int MODE, int WAVES, int SUBS, int GPL,
          bool LOGB = false, int GATE = kGateNone, bool XP = false>
__global__ __launch_bounds__(WAVES * 64) void k_scalar(const ScalarArgs a) {
  static_assert(!LOGB || (BWD && sizeof(Tin) == 4), "the log-space adjoint is an fp32 backward");
  static_assert(GATE != kGateNegSoftplus || (sizeof(Tin) == 4 && (LOGB || !BWD)), "-softplus gates feed the log-space scan");
  using S = typename Ops::S;
  using C = typename Ops::C;
  constexpr int NS = Ops::NS, NC = Ops::NC, ND = NS + NC;
  constexpr int VEC = InTraits<Tin>::VEC;
  constexpr int EL = VEC * GPL;          // elements per lane per sub-chunk
  constexpr int WREG = SUBS * 64 * EL;   // elements per wave
  constexpr int TILE = WAVES * WREG;     // elements per tile
  static_assert(EL <= 16, "per-lane span too long");
  // XP: lanes own 16 consecutive elements (one DPP scan per wave instead of
  // one per 256-element sub-chunk); every array of the wave's 1024-element
  // window moves between HBM and registers through an XOR-swizzled LDS stage
  // (coalesced direct loads, coalesced stores), so HBM still sees fully
  // coalesced 16-byte accesses.
  static_assert(!XP || (SUBS == 1 && EL == 16 && sizeof(Tin) == 4), "staged windows are fp32, 16 per lane");
  using SX = Stage<1, EL>;
  // Look-back dispatch order (see tile_of_block), from timing each workload
  // (packed: C = 1536 x 65536 tokens in 16 sequences): linear rows stream
  // memory best row-major, dense (tile-major cost ~10% at T = 16384; 16-bit
  // rows at T = 65536 7%) and packed alike (backward 5-7%, fp32 forward 4%,
  // 16-bit forward 2% since its boundaries are found without a per-lane
  // search); the log-space kernels resolve their look-back faster tile-major.
  constexpr bool kTileMajor = LOGB || !std::is_same<Ops, LinOps>::value;
  constexpr int NXR = BWD ? (LOGB ? 4 : 3) : 2;  // staged arrays per wave
  __shared__ __attribute__((aligned(16))) float s_x[XP ? WAVES : 1][XP ? NXR * SX::FLOATS : 4];

  __shared__ float s_agg[2][WAVES][NS];
  __shared__ float s_carry[NC];
  __shared__ int32_t s_cu[VARLEN ? kCuSlice : 1];
  __shared__ int32_t s_cu_n, s_cu_k0;

  const int l = lane_id();
  const int w = (int)(threadIdx.x >> 6);

  int64_t r;
  int c_first, c_last;
  if constexpr (MODE == kRowLoop) {
    r = blockIdx.x;
    c_first = c_last = 0;  // the row fits one tile
  } else {
    int c;
    tile_of_block<kTileMajor>(a.rows, a.ntiles, a.blk0, r, c);
    c_first = c_last = c;
  }
  const int64_t T = a.T;
  const int64_t rowoff = r * a.stride;
  const int lead = (int)(rowoff % VEC);
  const int64_t urow = ((T - 1 + lead) / VEC + 1) * VEC;  // padded row length
  const int64_t base = rowoff - lead;                       // element index of padded u = 0
  const Tin* gp = (const Tin*)a.g;
  const float* h0p = a.h0;
  const bool has_h0 = h0p != nullptr;
  // initial state as the backward uses it (h_prev of a sequence's first step)
  auto h0val = [&](int64_t i) -> float { return LOGB ? __expf(h0p[i]) : h0p[i]; };
  float h0row = 0.f;  // loaded with each tile's data (below)

  Workspace ws{};
  if constexpr (MODE == kLookback) ws = ws_view(a.ws);

  // ---- sequence table ------------------------------------------------------
  SegSlice seg{nullptr, 0, 0, false};
  if constexpr (VARLEN) {
    if constexpr (MODE == kRowLoop) {
      // the row's whole table, cached once
      const int n = a.nseg + 1;
      if (n <= kCuSlice) {
        for (int i = threadIdx.x; i < n; i += WAVES * 64) s_cu[i] = a.cu[i];
        __syncthreads();
        seg = SegSlice{nullptr, n, 0, true};
      } else {
        seg = SegSlice{a.cu, n, 0, false};
      }
    }
  }
  // Look-back mode: just the entries that cover this tile. A table of at most
  // 64 entries is read whole into wave 0's lanes (one entry each) before the
  // tile's data loads are issued, and sliced after them, so its only global
  // load overlaps the data; a longer table is searched after the data loads.
  const int ncu = a.nseg + 1;
  int32_t cu_l = 0;
  if constexpr (VARLEN && MODE == kLookback) {
    if (ncu <= 64 && w == 0 && l < ncu) cu_l = a.cu[l];
  }
  auto lookback_slice = [&]() {
    const int64_t jt0 = (int64_t)c_first * TILE;
    const int64_t ut_lo = REV ? urow - jt0 - TILE : jt0;
    const int64_t plo = max(ut_lo - lead, (int64_t)0), phi = min(ut_lo + TILE - lead, T);
    if (ncu <= 64) {
      if (w == 0) {
        int ka = 0, n = 0;
        if (plo < phi) {
          // entries <= key, counted over the lanes' entries
          ka = max(__popcll(__ballot(l < ncu && (int64_t)cu_l <= plo)) - 1, 0);
          const int kb = min(__popcll(__ballot(l < ncu && (int64_t)cu_l <= phi - 1)), a.nseg);
          n = max(kb - ka + 1, 1);
        }
        if (l >= ka && l < ka + n) s_cu[l - ka] = cu_l;
        if (l == 0) { s_cu_n = n; s_cu_k0 = ka; }
      }
      __syncthreads();
      seg = SegSlice{nullptr, s_cu_n, s_cu_k0, true};
      return;
    }
    if (w == 0) {
      int ka = 0, n = 0;
      if (plo < phi) {
        ka = max(wave_count_le(a.cu, ncu, plo) - 1, 0);
        const int kb = min(wave_count_le(a.cu, ncu, phi - 1), a.nseg);
        n = max(kb - ka + 1, 1);
      }
      if (l == 0) { s_cu_n = n; s_cu_k0 = ka; }
    }
    __syncthreads();
    const int n = s_cu_n, k0 = s_cu_k0;
    if (n <= kCuSlice) {
      for (int i = threadIdx.x; i < n; i += WAVES * 64) s_cu[i] = a.cu[k0 + i];
      __syncthreads();
      seg = SegSlice{nullptr, n, k0, true};
    } else {
      seg = SegSlice{a.cu + k0, n, k0, false};
    }
  };
  // entry i of the slice, from LDS (LDS = true) or global memory; code that
  // reads the slice is instantiated for each and chosen by seg.lds (a select
  // between the two arrays would be compiled into one flat load)
  auto segv_in = [&](auto in_lds, int i) -> int64_t {
    if constexpr (decltype(in_lds)::value) return (int64_t)s_cu[i];
    else return (int64_t)seg.g[i];
  };

  C carry = Ops::cident();  // state entering the current tile
  for (int c = c_first; c <= c_last; ++c) {
    const int64_t jt0 = (int64_t)c * TILE;
    const int64_t ut_lo = REV ? urow - jt0 - TILE : jt0;  // tile span in padded coords
    const bool interior = (ut_lo >= lead) && (ut_lo + TILE <= lead + T);
    // padded coordinate of the lowest element of sub-chunk s for this lane
    auto span_lo = [&](int s) -> int64_t {
      const int64_t j0 = jt0 + (int64_t)w * WREG + (int64_t)s * 64 * EL + (int64_t)l * EL;
      return REV ? urow - j0 - EL : j0;
    };

    // ---- load: every vector of the tile is in flight before the first use
    float Lg[SUBS][EL], Lb[SUBS][EL], Lh[BWD ? SUBS : 1][EL], Lx[LOGB ? SUBS : 1][EL];
    // XP: padded coordinate of this wave's window and this lane's block in it
    const int64_t wlo = REV ? urow - jt0 - (int64_t)(w + 1) * WREG : jt0 + (int64_t)w * WREG;
    const int xblk = REV ? 63 - l : l;
    float* xr = s_x[XP ? w : 0];
    // XP: the staged path serves every wave whose whole window lies in the
    // row (a wave-uniform test), so a partial tile sends only its straddling
    // window down the element path (log-space forward, 8192 rows of T = 8000:
    // 209 -> 161 us; of T = 7000: 176 -> 155 us)
    const bool xstage = XP && (interior || (wlo >= lead && wlo + WREG <= lead + T));
    // every array's EL elements of sub-chunk s from vector-aligned padded u0
    auto load_vectors = [&](int s, int64_t u0) {
      load_span<Tin, EL>(gp + base + u0, Lg[s]);
#pragma unroll
      for (int e = 0; e < EL; ++e) Lg[s][e] = gate_value<GATE, LOGB>(Lg[s][e]);
      if constexpr (!BWD) {
        load_span<Tin, EL>((const Tin*)a.b + base + u0, Lb[s]);
      } else {
        load_span<float, EL>((const float*)a.b + base + u0, Lb[s]);
        load_span<float, EL>(a.hs + base + u0, Lh[s]);
        if constexpr (LOGB) load_span<float, EL>(a.lb + base + u0, Lx[s]);
      }
    };
    // Backward halo, one value per wave: the gate before the wave's span and
    // the forward state after it (processing order). Every lane loads the same
    // in-row element (index clamped, result masked), issued ahead of the tile's
    // vectors: loaded where they are used, after the shuffles that wait for
    // the tile, they cost each workgroup a second memory round trip.
    float halo_g = 0.f, halo_h = 0.f;
    bool halo_g_ok = false, halo_h_ok = false;
    if constexpr (BWD) {
      const int64_t jg = jt0 + (int64_t)w * WREG - 1, jh = jt0 + (int64_t)(w + 1) * WREG;
      const int64_t tg = (REV ? urow - 1 - jg : jg) - lead, th = (REV ? urow - 1 - jh : jh) - lead;
      halo_g_ok = jg >= 0 && tg >= 0 && tg < T;
      halo_h_ok = th >= 0 && th < T;
      halo_g = InTraits<Tin>::load1(gp + rowoff + (halo_g_ok ? tg : 0));
      halo_h = a.hs[rowoff + (halo_h_ok ? th : 0)];
    }
    // the row's initial state (a wave-uniform address: a scalar load, which
    // no wait for the tile's vector loads holds back)
    if constexpr (!VARLEN) {
      if (has_h0) h0row = h0val(r);
    }
    if (xstage) {
      if constexpr (XP) {
        SX::load((const float*)gp + base + wlo, xr, SX::FLOATS, true);
        SX::load((const float*)a.b + base + wlo, xr + SX::FLOATS, SX::FLOATS, true);
        if constexpr (BWD) SX::load(a.hs + base + wlo, xr + 2 * SX::FLOATS, SX::FLOATS, true);
        if constexpr (LOGB) SX::load(a.lb + base + wlo, xr + 3 * SX::FLOATS, SX::FLOATS, true);
        wait_stage_loads();
        SX::read_block(xr, xblk, Lg[0]);
#pragma unroll
        for (int e = 0; e < EL; ++e) Lg[0][e] = gate_value<GATE, LOGB>(Lg[0][e]);
        SX::read_block(xr + SX::FLOATS, xblk, Lb[0]);
        if constexpr (BWD) SX::read_block(xr + 2 * SX::FLOATS, xblk, Lh[0]);
        if constexpr (LOGB) SX::read_block(xr + 3 * SX::FLOATS, xblk, Lx[0]);
      }
    } else if (interior) {
      // straight-line: every vector of the tile in flight before the first use
#pragma unroll
      for (int s = 0; s < SUBS; ++s) load_vectors(s, span_lo(s));
    } else {
      // A partial tile (a row end inside it): vector loads for every lane span
      // inside the row, element loads with bounds only for the spans that
      // straddle a row end. (Kept apart from the interior branch: a per-lane
      // condition there cost 5-50% on the look-back kernels.)
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        const int64_t u0 = span_lo(s);
        if (u0 >= lead && u0 + EL <= lead + T) {
          load_vectors(s, u0);
        } else {
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            const int64_t t = u0 + e - lead;
            const bool ok = (t >= 0) && (t < T);
            Lg[s][e] = ok ? gate_value<GATE, LOGB>(InTraits<Tin>::load1(gp + rowoff + t)) : Ops::kMaskA;
            if constexpr (!BWD) {
              Lb[s][e] = ok ? InTraits<Tin>::load1((const Tin*)a.b + rowoff + t) : Ops::kMaskB;
            } else {
              Lb[s][e] = ok ? ((const float*)a.b)[rowoff + t] : 0.f;
              Lh[s][e] = ok ? a.hs[rowoff + t] : 0.f;
              if constexpr (LOGB) Lx[s][e] = ok ? a.lb[rowoff + t] : 0.f;
            }
          }
        }
      }
    }
    // a tile with no sequence start or end inside (its sequence began before
    // it and ends after it) needs no per-lane boundary search below
    bool quiet = false;
    if constexpr (VARLEN && MODE == kLookback) {
      lookback_slice();
      const int64_t plo = max(ut_lo - lead, (int64_t)0), phi = min(ut_lo + TILE - lead, T);
      quiet = seg.n == 2 && seg.lds && segv_in(std::true_type{}, 0) < plo && segv_in(std::true_type{}, 1) > phi;
    }
    if constexpr (LOGB) {
      // b = e^{log b} (a = e^{log a} was taken on load, 0 for log a = -inf)
#pragma unroll
      for (int s = 0; s < SUBS; ++s)
#pragma unroll
        for (int e = 0; e < EL; ++e) Lx[s][e] = __expf(Lx[s][e]);
    }
    // processing order: element e of a lane is physical component P_(e)
    auto P_ = [](int e) { return REV ? EL - 1 - e : e; };
    float A[SUBS][EL], B[SUBS][EL];
    float G[BWD ? SUBS : 1][EL], N[BWD ? SUBS : 1][EL];  // bwd: own gate, next forward state
#pragma unroll
    for (int s = 0; s < SUBS; ++s) {
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        B[s][e] = Lb[s][P_(e)];
        if constexpr (!BWD) {
          A[s][e] = Lg[s][P_(e)];
        } else {
          G[s][e] = Lg[s][P_(e)];
          N[s][e] = Lh[s][P_(e)];
        }
      }
    }

    // ---- backward: shift gates forward and states backward by one element
    if constexpr (BWD) {
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        float gprev = __shfl_up(G[s][EL - 1], 1, 64);
        float hnext = __shfl_down(N[s][0], 1, 64);
        if (s > 0) {
          const float gl = readlane_f(G[s - 1][EL - 1], 63);
          if (l == 0) gprev = gl;
        } else if (l == 0) {
          gprev = halo_g_ok ? gate_value<GATE, LOGB>(halo_g) : 0.f;  // element before this wave's span
        }
        if (s + 1 < SUBS) {
          const float hn = readlane_f(N[s + 1][0], 0);
          if (l == 63) hnext = hn;
        } else if (l == 63) {
          hnext = halo_h_ok ? halo_h : 0.f;  // element after this wave's span
        }
#pragma unroll
        for (int e = EL - 1; e > 0; --e) A[s][e] = G[s][e - 1];
        A[s][0] = gprev;
#pragma unroll
        for (int e = 0; e < EL - 1; ++e) N[s][e] = N[s][e + 1];
        N[s][EL - 1] = hnext;
      }
    }

    // ---- sequence boundaries ------------------------------------------------
    // first: a sequence's first element in processing order; last: its last.
    // few: a forward tile covered by at most kFewBounds table entries (the
    // common packed case: a few sequence starts per tile). Every lane then
    // tests each entry against its span in a wave-uniform loop instead of
    // searching the slice and walking its elements (a per-lane binary search
    // and a divergent walk, both through LDS: 9% of the packed 16-bit
    // forward, C = 1536 x 65536 tokens in 16 sequences, 156 -> 143 us).
    // With initial states it serves the reverse direction only: the lookup of
    // each start's h0 raised the causal kernel to 91 VGPRs (5 waves per SIMD
    // instead of 6, 6% slower without h0) and gained nothing there, while the
    // reverse one kept its registers and ran 8% faster with h0.
    constexpr int kFewBounds = 8;
    const bool few = VARLEN && !BWD && seg.lds && seg.n <= kFewBounds && (REV || !has_h0);
    // the marked positions (starts, or ends when reversed) of the few entries,
    // read once per tile into wave-uniform registers; -1 for none or outside
    // the row
    uint32_t fq[VARLEN && !BWD ? kFewBounds : 1];
    if constexpr (VARLEN && !BWD) {
      if (few) {
#pragma unroll
        for (int i = 0; i < kFewBounds; ++i) {
          const int64_t q = (i < seg.n) ? (int64_t)s_cu[i] - (REV ? 1 : 0) : -1;
          fq[i] = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint64_t)q < (uint64_t)T ? q : -1));
        }
      }
    }
    // cm: bit s EL + ep marks element ep (physical order) of the lane's span
    // in sub-chunk s. A lane's spans lie 64 EL apart, so one pass over the
    // entries places each in its sub-chunk. (Differences of the low 32 bits
    // stand for differences below 2^32 in size: a position before the spans
    // wraps to a value far past them.)
    uint32_t cm = 0;
    if constexpr (VARLEN && !BWD) {
      static_assert(SUBS * EL <= 32, "one bit per element of a lane's spans");
      if (few) {
        constexpr uint32_t kSpanStride = 64 * EL;
        const uint32_t q00 = (uint32_t)(span_lo(0) - lead);
#pragma unroll
        for (int i = 0; i < kFewBounds; ++i) {
          if (i < seg.n && fq[i] != 0xffffffffu) {
            const uint32_t m = REV ? q00 + (uint32_t)(EL - 1) - fq[i] : fq[i] - q00;
            const uint32_t sc = m / kSpanStride, e = m % kSpanStride;
            if (sc < (uint32_t)SUBS && e < (uint32_t)EL) cm |= 1u << (sc * EL + (REV ? EL - 1 - e : e));
          }
        }
      }
    }
    uint32_t lastmask[BWD ? SUBS : 1];
#pragma unroll
    for (int s = 0; s < SUBS; ++s) {
      const int64_t u0 = span_lo(s);
      uint32_t lm = 0;
      if constexpr (!VARLEN) {
        // one sequence per row: first / last are the row's ends, which lie in
        // the spans of at most two lanes of the row. Lanes test their span
        // once before the per-element tests, except in the linear scans'
        // one-tile rows (4-element lanes), where comparing every element was
        // 0.5% faster on the dense fp32 backward; elsewhere the per-element
        // form raised registers past an occupancy step (log-space adjoint 114
        // -> 137 VGPRs, 11% slower; look-back backward 109 -> 138)
        const int64_t tf = REV ? T - 1 : 0, tl = REV ? 0 : T - 1;
        const int64_t q0 = u0 - lead;
        constexpr bool kEachElem = EL < 8 && !LOGB && MODE == kRowLoop;
        const bool ends = kEachElem || (tf >= q0 && tf < q0 + EL) || (BWD && tl >= q0 && tl < q0 + EL);
        if (ends) {
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            const int64_t t = q0 + P_(e);
            if (t == tf) {
              if constexpr (!BWD) Ops::first_ab(A[s][e], B[s][e], h0row, has_h0);
              else A[s][e] = 0.f;
            }
            if constexpr (BWD) {
              if (t == tl) {
                N[s][e] = h0row;
                lm |= 1u << e;
              }
            }
          }
        }
      } else if (few && !quiet) {
        // Position q starts a sequence iff some entry equals q, and ends one
        // iff some entry equals q + 1 (the entries are sorted and the first is
        // at or before the tile's first element). The processing order's
        // first element is the start (forward) or the end (reverse); cm holds
        // the marks.
        const uint32_t q0 = (uint32_t)(u0 - lead);
        const uint32_t fm = (cm >> (s * EL)) & ((1u << EL) - 1u);
        if (fm) {
#pragma unroll
          for (int ep = 0; ep < EL; ++ep) {
            const int e = REV ? EL - 1 - ep : ep;
            if ((fm >> ep) & 1u) {
              float hv = 0.f;
              if constexpr (REV) {
                if (has_h0) {
                  // the sequence this element ends: one before the first
                  // entry equal to its successor (the walk's k)
                  const uint32_t q = q0 + (uint32_t)ep;
                  int k = 0;
#pragma unroll
                  for (int i = kFewBounds - 1; i >= 0; --i)
                    if (i < seg.n && fq[i] == q) k = i;
                  const int sk = min(max(seg.k0 + k - 1, 0), a.nseg - 1);
                  hv = h0val((int64_t)sk * a.rows + r);
                }
              }
              Ops::first_ab(A[s][e], B[s][e], hv, has_h0);
            }
          }
        }
      } else if (seg.n > 0 && !quiet) {
        // walk the elements in physical order against the sequence table
        auto bounds = [&](auto in_lds) {
        auto segv = [&](int i) -> int64_t { return segv_in(in_lds, i); };
        const int64_t q0 = u0 - lead;
        int k = slice_find(seg.n, segv, max(q0, (int64_t)0));
        // a sequence starts or ends inside [q0, q0 + EL) only if the found
        // start is q0 or the next start is at most q0 + EL
        const int64_t next = (k + 1 < seg.n) ? segv(k + 1) : INT64_MAX;
        const bool walk = (segv(k) >= q0) || (next <= q0 + EL);
        if (walk) {
#pragma unroll
          for (int ep = 0; ep < EL; ++ep) {
            const int64_t q = q0 + ep;
            if (q < 0 || q >= T) continue;
            while (k + 1 < seg.n && segv(k + 1) <= q) ++k;
            const bool is_start = segv(k) == q;
            const bool is_end = (k + 1 < seg.n) && (segv(k + 1) - 1 == q);
            const int e = REV ? EL - 1 - ep : ep;
            const bool first = REV ? is_end : is_start;
            const bool last = REV ? is_start : is_end;
            if (first || last) {
              const int sk = min(max(seg.k0 + k, 0), a.nseg - 1);
              const float hv = has_h0 ? h0val((int64_t)sk * a.rows + r) : 0.f;
              if (first) {
                if constexpr (!BWD) Ops::first_ab(A[s][e], B[s][e], hv, has_h0);
                else A[s][e] = 0.f;
              }
              if constexpr (BWD) {
                if (last) {
                  N[s][e] = hv;
                  lm |= 1u << e;
                }
              }
            }
          }
        }
        };
        if (seg.lds) bounds(std::true_type{});
        else bounds(std::false_type{});
      }
      if constexpr (BWD) lastmask[s] = lm;
    }

    // ---- lane-serial summaries and wave scans ---------------------------
    // plain: every step of the wave allows the operator's plain form (log
    // space: all log a and log b finite), decided per wave; the wave's own
    // compositions and applications then skip the -inf selects.
    bool plain = false;
    if constexpr (Ops::kHasPlain) {
      bool ok = true;
#pragma unroll
      for (int s = 0; s < SUBS; ++s)
#pragma unroll
        for (int e = 0; e < EL; ++e) ok = ok && Ops::plain_elem(A[s][e], B[s][e]);
      plain = __ballot(!ok) == 0ull;
    }
    S sum[SUBS];
    auto wave_scan = [&](auto plain_c) {
      constexpr bool PL = decltype(plain_c)::value;
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        S run = Ops::ident();
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          S el = Ops::elem(A[s][e], B[s][e]);
          if constexpr (PL) Ops::compose_plain(run, el);
          else Ops::compose(run, el);
          run = el;
        }
        sum[s] = run;
      }
      // step-major so the SUBS independent scans interleave
      const bool v1 = (l & 15) >= 1, v2 = (l & 15) >= 2, v4 = (l & 15) >= 4, v8 = (l & 15) >= 8;
      const bool v16 = (l & 16) != 0, v32 = l >= 32;
#pragma unroll
      for (int s = 0; s < SUBS; ++s) scan_step<Ops, kRowShr1, 0xf, PL>(sum[s], v1);
#pragma unroll
      for (int s = 0; s < SUBS; ++s) scan_step<Ops, kRowShr2, 0xf, PL>(sum[s], v2);
#pragma unroll
      for (int s = 0; s < SUBS; ++s) scan_step<Ops, kRowShr4, 0xf, PL>(sum[s], v4);
#pragma unroll
      for (int s = 0; s < SUBS; ++s) scan_step<Ops, kRowShr8, 0xf, PL>(sum[s], v8);
#pragma unroll
      for (int s = 0; s < SUBS; ++s) scan_step<Ops, kRowBcast15, 0xa, PL>(sum[s], v16);
#pragma unroll
      for (int s = 0; s < SUBS; ++s) scan_step<Ops, kRowBcast31, 0xc, PL>(sum[s], v32);
    };
    if constexpr (Ops::kHasPlain) {
      if (plain) wave_scan(std::true_type{});
      else wave_scan(std::false_type{});
    } else {
      wave_scan(std::false_type{});
    }
    // wave aggregate = sub-chunk totals (lane 63) in order
    S wagg = Ops::ident();
#pragma unroll
    for (int s = 0; s < SUBS; ++s) {
      S st;
#pragma unroll
      for (int i = 0; i < NS; ++i) st.v[i] = readlane_f(sum[s].v[i], 63);
      Ops::compose(wagg, st);  // (sub-chunks so far, then sub-chunk s)
      wagg = st;
    }

    // ---- across waves ------------------------------------------------------
    S ex = Ops::ident();  // composition of the waves before this one
    S tagg = wagg;        // tile aggregate
    if constexpr (WAVES > 1) {
      const int buf = c & 1;  // alternate buffers: one barrier per tile suffices
      if (l == 0) {
#pragma unroll
        for (int i = 0; i < NS; ++i) s_agg[buf][w][i] = wagg.v[i];
      }
      __syncthreads();
      tagg = Ops::ident();
#pragma unroll
      for (int q = 0; q < WAVES; ++q) {
        if (q == w) ex = tagg;
        S x;
#pragma unroll
        for (int i = 0; i < NS; ++i) x.v[i] = s_agg[buf][q][i];
        Ops::compose(tagg, x);
        tagg = x;
      }
    }

    // ---- across tiles: decoupled look-back ----------------------------------
    if constexpr (MODE == kLookback) {
      uint64_t* rd = ws.desc + (int64_t)ND * ((int64_t)r * a.ntiles);
      uint64_t* my = rd + (int64_t)ND * c;
      if (w == 0) {
        const uint32_t tagA = kTagAgg, tagI = kTagIncl;
        const bool hard = Ops::hard(tagg);
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
        if (c > 0) carry = lookback<Ops, kTileMajor>(ws, rd, c, spin_limit(a.spin));
        stress_pause(2);
        if (l == 0) {
          if (!hard) {
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

    // ---- apply: every element from its exact carry-in ---------------------------
    C hs = Ops::apply(ex, carry);  // state entering this wave's span
    float O[SUBS][EL];
    auto wave_apply = [&](auto plain_c) {
      constexpr bool PL = decltype(plain_c)::value;
#pragma unroll
      for (int s = 0; s < SUBS; ++s) {
        C v;  // state after this lane
        if constexpr (PL) v = Ops::apply_plain(sum[s], hs);
        else v = Ops::apply(sum[s], hs);
        C st;
#pragma unroll
        for (int i = 0; i < NC; ++i) {
          st.v[i] = __shfl_up(v.v[i], 1, 64);
          if (l == 0) st.v[i] = hs.v[i];
          hs.v[i] = readlane_f(v.v[i], 63);
        }
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          if constexpr (PL) {
            st = Ops::step_plain(A[s][e], B[s][e], st);
            O[s][e] = Ops::out_plain(st);
          } else {
            st = Ops::step(A[s][e], B[s][e], st);
            O[s][e] = Ops::out(st);
          }
        }
      }
    };
    if constexpr (Ops::kHasPlain) {
      if (plain) wave_apply(std::true_type{});
      else wave_apply(std::false_type{});
    } else {
      wave_apply(std::false_type{});
    }
    carry = Ops::apply(tagg, carry);  // state at the end of the tile

    // ---- store -------------------------------------------------------------
#pragma unroll
    for (int s = 0; s < SUBS; ++s) {
      const int64_t u0 = span_lo(s);
      float o0[EL], o1[EL];
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        if constexpr (!LOGB) {
          o0[P_(e)] = O[s][e];
          if constexpr (BWD) {
            if constexpr (GATE == kGateSigmoid)
              o1[P_(e)] = (O[s][e] * N[s][e]) * (G[s][e] * (1.f - G[s][e]));  // dz = dg * g (1 - g)
            else
              o1[P_(e)] = O[s][e] * N[s][e];                                    // dg = lam * h_prev
          }
        } else {
          o0[P_(e)] = O[s][e] * Lx[s][P_(e)];             // dlog_b = lam * b
          if constexpr (GATE == kGateNegSoftplus)         // dz = dlog_a * (-sigmoid(z)), sigmoid(z) = 1 - a
            o1[P_(e)] = -((O[s][e] * N[s][e]) * (G[s][e] * (1.f - G[s][e])));
          else
            o1[P_(e)] = (O[s][e] * N[s][e]) * G[s][e];    // dlog_a = lam * h_prev * a
        }
      }
      if (xstage) {
        if constexpr (XP) {
          wave_lds_sync();
          SX::write_block(xr, xblk, o0);
          if constexpr (BWD) SX::write_block(xr + SX::FLOATS, xblk, o1);
          wave_lds_sync();
          SX::store(a.out0 + base + wlo, xr, SX::FLOATS, true);
          if constexpr (BWD) SX::store(a.out1 + base + wlo, xr + SX::FLOATS, SX::FLOATS, true);
        }
      } else if (interior) {
        store_span<EL>(a.out0 + base + u0, o0);
        if constexpr (BWD) store_span<EL>(a.out1 + base + u0, o1);
      } else if (u0 >= lead && u0 + EL <= lead + T) {  // a lane span inside the row
        store_span<EL>(a.out0 + base + u0, o0);
        if constexpr (BWD) store_span<EL>(a.out1 + base + u0, o1);
      } else {
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          const int64_t t = u0 + e - lead;
          if (t >= 0 && t < T) {
            a.out0[rowoff + t] = o0[e];
            if constexpr (BWD) a.out1[rowoff + t] = o1[e];
          }
        }
      }
      if constexpr (BWD) {
        // dh0 = g * lam at each sequence's forward-first element
        if (a.dh0 && lastmask[s]) {
#pragma unroll
          for (int e = 0; e < EL; ++e) {
            if (!(lastmask[s] & (1u << e))) continue;
            const int64_t t = u0 + P_(e) - lead;
            int sk = 0;
            if constexpr (VARLEN) {
              const int kk = seg.lds ? slice_find(seg.n, [&](int i) { return segv_in(std::true_type{}, i); }, t)
                                     : slice_find(seg.n, [&](int i) { return segv_in(std::false_type{}, i); }, t);
              sk = min(max(seg.k0 + kk, 0), a.nseg - 1);
            }
            // dh0 = g * lam; log space: dlog_h0 = a * lam * h0 (N holds h0 there);
            // nothing reaches h0 through a zero gate (a reset)
            const float gl = G[s][e] * O[s][e];
            a.dh0[(int64_t)sk * a.rows + r] = (G[s][e] != 0.f) ? (LOGB ? gl * N[s][e] : gl) : 0.f;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------

template <class Ops, typename Tin, bool BWD, bool REV, int WAVES, int SUBS, int GPL, bool LOGB = false,
          int GATE = kGateNone, bool XP = false>
static hipError_t launch_cfg(const ScalarArgs& a0, hipStream_t st) {
  constexpr int TILE = WAVES * SUBS * 64 * InTraits<Tin>::VEC * GPL;
  ScalarArgs a = a0;
  a.ntiles = (int32_t)scalar_tiles(a.T, a.stride, InTraits<Tin>::VEC, TILE);
  const bool lookback = scalar_uses_lookback(a.rows, a.ntiles);
  const bool varlen = a.cu != nullptr;
  const dim3 block(WAVES * 64);
  if (!lookback) {
    const dim3 grid((unsigned)a.rows);
    if (varlen) hipLaunchKernelGGL((k_scalar<Ops, Tin, BWD, REV, true, kRowLoop, WAVES, SUBS, GPL, LOGB, GATE, XP>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_scalar<Ops, Tin, BWD, REV, false, kRowLoop, WAVES, SUBS, GPL, LOGB, GATE, XP>), grid, block, 0, st, a);
  } else {
    // fresh descriptors for this call (zero tag = not published)
    const size_t words = (size_t)a.rows * (size_t)a.ntiles * (size_t)(Ops::NS + Ops::NC);
    const hipError_t z = launch_zero(a.ws, ws_desc_offset() + words * sizeof(uint64_t), st);
    if (z != hipSuccess) return z;
    const dim3 grid(launch_blocks((uint64_t)a.rows * (uint64_t)a.ntiles, a.nblk));
    if (varlen) hipLaunchKernelGGL((k_scalar<Ops, Tin, BWD, REV, true, kLookback, WAVES, SUBS, GPL, LOGB, GATE, XP>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_scalar<Ops, Tin, BWD, REV, false, kLookback, WAVES, SUBS, GPL, LOGB, GATE, XP>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace mscan
