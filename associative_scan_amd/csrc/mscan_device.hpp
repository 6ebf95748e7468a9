// Device building blocks shared by the libmscan kernels (gfx950 / CDNA4, wave64).
//
// The affine maps h -> P h + Q form a monoid under composition: applying
// (P1, Q1) then (P2, Q2) gives (P2 P1, P2 Q1 + Q2), identity (1, 0) ("Triton
// scan kernels", "One associative-scan family"; "Our RG-LRU GPU audit", "Exact
// real chunk algebra" gives the same per-chunk update P <- a P, Q <- a Q + b).
// Associativity lets every level below regroup the steps freely:
//   lane-serial chunk summary -> 64-lane DPP wave scan -> LDS across waves ->
//   decoupled look-back across tiles -> apply.
//
// Zero transitions. A zero P is treated as "erases everything before": the
// composition keeps the later map unchanged instead of multiplying an earlier
// Q by zero. That is how a reset a_t = 0 is defined ("Our RG-LRU GPU audit",
// "Exact real chunk algebra": a reset is encoded as a zero transition and
// leaves nothing of the prefix), Inf or NaN before it included; for finite
// data it is also the arithmetic result. It makes sequence starts hard
// boundaries too (they enter the scan as P = 0), so a NaN or Inf in one
// packed sequence can never reach the next one. (A product of nonzero gates
// that underflows to 0 is treated the same way; for a finite prefix that is
// again the arithmetic result.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mscan_launch.hpp"

namespace mscan {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// DPP lane movement (GFX9 encodings; gfx950 keeps the wave-wide shifts)
// ---------------------------------------------------------------------------
enum : int {
  kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118,
  kWaveShl1 = 0x130, kWaveShr1 = 0x138, kRowBcast15 = 0x142, kRowBcast31 = 0x143,
};

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float src) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL,
                                                    ROW_MASK, 0xf, false));
}

// DPP move whose value is only used in lanes where the source lane is valid
// (out-of-range sources read zero, lanes outside ROW_MASK are left undefined):
// no register has to be initialised first.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_mov_f(float src) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(src), CTRL, ROW_MASK, 0xf, true));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// ---------------------------------------------------------------------------
// LDS staging of one array over a wave window
// ---------------------------------------------------------------------------
constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x / 2); }

// N floats per step, EL steps per lane, 64 lanes. The window's floats are cut
// into 16-byte units; lane l owns units [l*LU, (l+1)*LU). Unit u is kept at
// LDS unit swz(u) = u ^ ((u >> SH) & MSK): that flips only the low 4 bits (so
// u stays in its aligned group of 16 units, and each group of 16 / 64 units
// is still one contiguous block of memory) and spreads the lanes that read
// unit c of their blocks over 16 different 16-byte bank groups. swz is its
// own inverse.
// Cache policy of the direct loads: nontemporal (nt), as the register loads
// of the streamed arrays are. Every staged array is read exactly once; without
// the hint these loads allocate in the caches and, behind a large write (dirty
// lines left in L2 and the Infinity Cache), spend their time on the evictions:
// log-space forward 8192 rows x T = 8192 after a 1 GiB fill, 204 -> 142 us;
// (2, 1) matrix forward / backward 4096 rows x T = 8192, 266 -> 190 us and
// 389 -> 346 us.
constexpr int kLdsNT = 2;

template <int N, int EL>
struct Stage {
  static constexpr int FLOATS = N * 64 * EL;  // floats per window
  static constexpr int UNITS = FLOATS / 4;
  static constexpr int LU = N * EL / 4;       // units per lane
  static_assert((N * EL) % 4 == 0 && (LU & (LU - 1)) == 0, "lane blocks must be whole powers-of-two of units");
  static constexpr int SH = LU >= 16 ? ilog2c(LU) : 4;
  static constexpr int MSK = (LU >= 16 ? 16 : LU) - 1;
  __device__ static __forceinline__ int swz(int u) { return u ^ ((u >> SH) & MSK); }
  // LDS float index of window float f
  __device__ static __forceinline__ int at(int f) { return swz(f >> 2) * 4 + (f & 3); }

  // window floats [0, nvalid) come from g[0, nvalid); the rest are left as
  // they are (callers mask those steps). vec: g is 16-byte aligned.
  __device__ static __forceinline__ void load(const float* g, float* lds, int nvalid, bool vec) {
    const int l = lane_id();
    if (vec && nvalid == FLOATS) {
#pragma unroll
      for (int i = 0; i < UNITS / 64; ++i) {
        const int u = swz(i * 64 + l);
        __builtin_amdgcn_global_load_lds((const void*)(g + u * 4),
                                         (__attribute__((address_space(3))) void*)(lds + i * 256), 16, 0, kLdsNT);
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < FLOATS / 64; ++i) {
        const int p = i * 64 + l;
        const int f = swz(p >> 2) * 4 + (p & 3);
        if (f < nvalid)
          __builtin_amdgcn_global_load_lds((const void*)(g + f),
                                           (__attribute__((address_space(3))) void*)(lds + i * 64), 4, 0, kLdsNT);
      }
    }
  }
  // window floats [0, nvalid) go to g[0, nvalid)
  __device__ static __forceinline__ void store(float* g, const float* lds, int nvalid, bool vec) {
    const int l = lane_id();
    if (vec && nvalid == FLOATS) {
#pragma unroll
      for (int i = 0; i < UNITS / 64; ++i) {
        const int p = i * 64 + l;
        const v4f t = *(const v4f*)(lds + p * 4);
        __builtin_nontemporal_store(t, (v4f*)(g + swz(p) * 4));
      }
    } else {
#pragma unroll 4
      for (int i = 0; i < FLOATS / 64; ++i) {
        const int p = i * 64 + l;
        const int f = swz(p >> 2) * 4 + (p & 3);
        if (f < nvalid) g[f] = lds[p];
      }
    }
  }
  // the N floats of window step s
  __device__ static __forceinline__ void get(const float* lds, int s, float* o) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int j = 0; j < N / 4; ++j) {
        const v4f t = *(const v4f*)(lds + swz(s * (N / 4) + j) * 4);
        o[4 * j] = t.x; o[4 * j + 1] = t.y; o[4 * j + 2] = t.z; o[4 * j + 3] = t.w;
      }
    } else {
      static_assert(N == 2, "steps of 2 floats or whole units");
      typedef float v2f __attribute__((ext_vector_type(2)));
      const v2f t = *(const v2f*)(lds + swz(s >> 1) * 4 + (s & 1) * 2);
      o[0] = t.x; o[1] = t.y;
    }
  }
  // the LU units (4 LU floats) of lane block `blk`, in order
  __device__ static __forceinline__ void read_block(const float* lds, int blk, float* o) {
#pragma unroll
    for (int j = 0; j < LU; ++j) {
      const v4f t = *(const v4f*)(lds + swz(blk * LU + j) * 4);
      o[4 * j] = t.x; o[4 * j + 1] = t.y; o[4 * j + 2] = t.z; o[4 * j + 3] = t.w;
    }
  }
  __device__ static __forceinline__ void write_block(float* lds, int blk, const float* v) {
#pragma unroll
    for (int j = 0; j < LU; ++j) {
      const v4f t = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
      *(v4f*)(lds + swz(blk * LU + j) * 4) = t;
    }
  }
  __device__ static __forceinline__ void put(float* lds, int s, const float* v) {
    if constexpr (N % 4 == 0) {
#pragma unroll
      for (int j = 0; j < N / 4; ++j) {
        const v4f t = {v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]};
        *(v4f*)(lds + swz(s * (N / 4) + j) * 4) = t;
      }
    } else {
      typedef float v2f __attribute__((ext_vector_type(2)));
      const v2f t = {v[0], v[1]};
      *(v2f*)(lds + swz(s >> 1) * 4 + (s & 1) * 2) = t;
    }
  }
};

// Completion of this wave's direct-to-LDS loads, then of its LDS writes, made
// visible to all of its lanes (the staging areas are private to one wave).
__device__ __forceinline__ void wait_stage_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// Linear affine monoid
// ---------------------------------------------------------------------------
// compose(e, l): e earlier, l later. A zero l.P keeps l (see the file comment).
__device__ __forceinline__ void lin_compose(float eP, float eQ, float& lP, float& lQ) {
  const bool use = (lP != 0.f);
  const float nP = use ? lP * eP : lP;
  const float nQ = use ? __builtin_fmaf(lP, eQ, lQ) : lQ;
  lP = nP;
  lQ = nQ;
}

// value of map (P, Q) applied to h
__device__ __forceinline__ float lin_apply(float P, float Q, float h) {
  return (P != 0.f) ? __builtin_fmaf(P, h, Q) : Q;
}

// ---------------------------------------------------------------------------
// Workspace: a control header followed by the descriptor words of every tile.
//
// Every descriptor word is 64 bits, {tag:32 | value:32}, written and read with
// relaxed agent-scope atomics, so each word is self-validating and no fence is
// needed between words. tag 1 = aggregate of the tile alone, tag 2 = inclusive
// value (the state at the tile's end). The library zero-fills the words a call
// uses (a small kernel on the same stream) right before the scan kernel, so a
// zero tag always means "not published yet" and nothing from an earlier call,
// of any shape, can look valid.
// ---------------------------------------------------------------------------
enum : int { kHdrError = 3, kHdrWords = 32 };
static_assert(kHdrError == kHdrErrorWord && kHdrWords * 4 == kWsHeaderBytes, "workspace header layout");
enum : uint32_t { kTagAgg = 1, kTagIncl = 2 };

__device__ __forceinline__ uint32_t ld_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_u64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t pack_word(uint32_t tag, float v) {
  return ((uint64_t)tag << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ uint32_t word_tag(uint64_t w) { return (uint32_t)(w >> 32); }
__device__ __forceinline__ float word_val(uint64_t w) { return __uint_as_float((uint32_t)w); }

struct Workspace {
  uint32_t* hdr;   // kHdrWords 32-bit control words
  uint64_t* desc;  // per-tile descriptor words
};

// Byte offset of the descriptors (after the control header).
__host__ __device__ __forceinline__ constexpr size_t ws_desc_offset() { return (size_t)kHdrWords * 4; }

__device__ __forceinline__ Workspace ws_view(void* ws) {
  Workspace w;
  w.hdr = (uint32_t*)ws;
  w.desc = (uint64_t*)((char*)ws + ws_desc_offset());
  return w;
}

// Upper bound on look-back polls before a wave gives up. A wait can only run
// out if a predecessor never publishes (a launch that runs part of a grid, or
// a workspace shared by calls that overlap); the wave then sets the header's
// error word and takes a NaN carry, so the kernel still ends and every output
// that depended on the missing carry reads NaN instead of a plausible wrong
// value. A call may ask for a smaller limit (0 = this default).
constexpr uint32_t kSpinLimit = 1u << 22;
__device__ __forceinline__ uint32_t spin_limit(uint32_t requested) { return requested ? requested : kSpinLimit; }

// Race stress (a test build only: the library built with MSCAN_RACE_STRESS
// defined, see the build script): every publish of a look-back descriptor or
// of a chained state first waits a pseudo-random 0 to ~7700 cycles, different
// per workgroup and publish site, so that tiles publish in orders and at
// distances the ordinary timing rarely produces. Without the macro it is
// nothing.
__device__ __forceinline__ void stress_pause(uint32_t site) {
#ifdef MSCAN_RACE_STRESS
  uint32_t x = blockIdx.x * 2654435761u ^ (site + 1u) * 40503u;
  x ^= x >> 15;
  x *= 0x2c1b3c6du;
  x ^= x >> 12;
  const uint32_t n = (x >> 7) & 15u;  // wave-uniform
  for (uint32_t i = 0; i < n; ++i) __builtin_amdgcn_s_sleep(8);
#else
  (void)site;
#endif
}

// ---------------------------------------------------------------------------
// Scan "ops": one summary type S (a map from the state before a span to the
// state after it) and one carry type C (a state), stored as small float arrays
// so the DPP, LDS and look-back code below can move them member by member.
//   compose(e, l) : l := (e then l)          apply(s, c) : state after s from c
//   hard(s)       : s ignores its input      of_carry(c) : hard summary giving c
//   elem(a, b)    : one step                 step(a, b, c): one step applied to c
//   first_ab(a, b, h0, has_h0): turn a sequence's first step into a hard step
//                   with the initial state injected
// ---------------------------------------------------------------------------

// Linear space: h -> P h + Q, carry = h. A zero P is hard.
struct LinOps {
  static constexpr int NS = 2, NC = 1;
  static constexpr float kMaskA = 1.f, kMaskB = 0.f;  // identity step for masked elements
  struct S { float v[NS]; };
  struct C { float v[NC]; };
  __device__ static __forceinline__ S ident() { return S{{1.f, 0.f}}; }
  __device__ static __forceinline__ C cident() { return C{{0.f}}; }
  __device__ static __forceinline__ bool hard(const S& s) { return s.v[0] == 0.f; }
  __device__ static __forceinline__ void compose(const S& e, S& l) { lin_compose(e.v[0], e.v[1], l.v[0], l.v[1]); }
  __device__ static __forceinline__ C apply(const S& s, const C& c) { return C{{lin_apply(s.v[0], s.v[1], c.v[0])}}; }
  __device__ static __forceinline__ S of_carry(const C& c) { return S{{0.f, c.v[0]}}; }
  __device__ static __forceinline__ C carry_of_hard(const S& s) { return C{{s.v[1]}}; }
  __device__ static __forceinline__ S elem(float a, float b) { return S{{a, b}}; }
  // a sequence's first step with h0 injected, as a hard step (a', b'); a
  // zero gate there is a reset and drops h0
  __device__ static __forceinline__ void first_ab(float& a, float& b, float h0, bool) {
    b = (a != 0.f) ? __builtin_fmaf(a, h0, b) : b;
    a = 0.f;
  }
  __device__ static __forceinline__ float out(const C& c) { return c.v[0]; }
  // one step applied to a carry (the per-element apply)
  __device__ static __forceinline__ C step(float a, float b, const C& c) {
    return C{{(a != 0.f) ? __builtin_fmaf(a, c.v[0], b) : b}};
  }
  // No plain path: the linear scans are memory-bound, and dropping their
  // zero-gate selects (a quarter of their VALU work) measured no faster.
  static constexpr bool kHasPlain = false;
  __device__ static __forceinline__ bool plain_elem(float, float) { return false; }
  __device__ static __forceinline__ void compose_plain(const S& e, S& l) { compose(e, l); }
  __device__ static __forceinline__ C apply_plain(const S& s, const C& c) { return apply(s, c); }
  __device__ static __forceinline__ C step_plain(float a, float b, const C& c) { return step(a, b, c); }
  __device__ static __forceinline__ float out_plain(const C& c) { return out(c); }
};

// Log space ("Triton scan kernels", "One associative-scan family": the
// log-space member carries a running log-coefficient sum and an online
// max-shifted log-sum-exp, writing h = exp(.)). A step is (log a, log b).
// Summary S = (P, m, s): P = sum of log a over the span (the running
// log-coefficient sum, local to the span so it stays small), and the span's
// own contribution as a max-shifted sum, log value = m + log s with s >= 1.
// Carry C = (m, s) for log h = m + log s. Composing two pairs needs one exp
// and no log; the output is h = e^m * s. P = -inf (a = 0) is hard.
// Written with selects, not early returns: every lane runs the same
// instructions (branches around the -inf cases cost the log-space kernels an
// exec-mask save, a branch and a restore per call).
__device__ __forceinline__ void lse_pair(float am, float as, float bm, float bs, float& m, float& s) {
  const float M = fmaxf(am, bm);
  const float d = am - bm;
  const float E = __expf(-fabsf(d));
  const bool ge = d >= 0.f;
  const float t = __builtin_fmaf(ge ? bs : as, E, ge ? as : bs);
  s = (M == -__builtin_inff()) ? 0.f : t;
  m = M;
}

struct LogOps {
  static constexpr int NS = 3, NC = 2;
  static constexpr float kMaskA = 0.f, kMaskB = -__builtin_inff();
  struct S { float v[NS]; };
  struct C { float v[NC]; };
  __device__ static __forceinline__ S ident() { return S{{0.f, -__builtin_inff(), 0.f}}; }
  __device__ static __forceinline__ C cident() { return C{{-__builtin_inff(), 0.f}}; }
  __device__ static __forceinline__ bool hard(const S& s) { return s.v[0] == -__builtin_inff(); }
  __device__ static __forceinline__ void compose(const S& e, S& l) {
    const bool hard = l.v[0] == -__builtin_inff();
    float m, s;
    lse_pair(l.v[0] + e.v[1], e.v[2], l.v[1], l.v[2], m, s);
    l.v[0] = hard ? l.v[0] : e.v[0] + l.v[0];
    l.v[1] = hard ? l.v[1] : m;
    l.v[2] = hard ? l.v[2] : s;
  }
  __device__ static __forceinline__ C apply(const S& s, const C& c) {
    const bool hard = s.v[0] == -__builtin_inff();
    C r;
    lse_pair(s.v[0] + c.v[0], c.v[1], s.v[1], s.v[2], r.v[0], r.v[1]);
    return C{{hard ? s.v[1] : r.v[0], hard ? s.v[2] : r.v[1]}};
  }
  __device__ static __forceinline__ S of_carry(const C& c) { return S{{-__builtin_inff(), c.v[0], c.v[1]}}; }
  __device__ static __forceinline__ C carry_of_hard(const S& s) { return C{{s.v[1], s.v[2]}}; }
  __device__ static __forceinline__ S elem(float a, float b) { return S{{a, b, 1.f}}; }
  // a sequence's first step with log h0 injected, as a hard step (-inf, b');
  // log a = -inf there is a reset and drops h0
  __device__ static __forceinline__ void first_ab(float& a, float& b, float h0, bool has_h0) {
    if (has_h0 && a != -__builtin_inff()) {
      float m, s;
      lse_pair(a + h0, 1.f, b, 1.f, m, s);
      b = (m == -__builtin_inff()) ? m : m + __logf(s);
    }
    a = -__builtin_inff();
  }
  __device__ static __forceinline__ float out(const C& c) {
    return c.v[0] == -__builtin_inff() ? 0.f : __expf(c.v[0]) * c.v[1];
  }
  __device__ static __forceinline__ C step(float a, float b, const C& c) {
    return apply(S{{a, b, 1.f}}, c);
  }
  // Plain forms, for a wave whose steps all have finite log a and log b (no
  // a = 0, no b = 0, nothing infinite or NaN): no summary in it is hard and
  // every log-sum-exp has a finite operand, so the -inf selects above never
  // fire and these give the same bits with 11-15 fewer VALU operations per
  // element (the log-space forward is VALU-bound). A carry of (-inf, 0)
  // entering them still gives the step's own value.
  static constexpr bool kHasPlain = true;
  __device__ static __forceinline__ bool plain_elem(float a, float b) {
    return __builtin_fabsf(a) < __builtin_inff() && __builtin_fabsf(b) < __builtin_inff();
  }
  __device__ static __forceinline__ void lse_plain(float am, float as, float bm, float bs, float& m, float& s) {
    const float d = am - bm;
    const float E = __expf(-fabsf(d));
    const bool ge = d >= 0.f;
    s = __builtin_fmaf(ge ? bs : as, E, ge ? as : bs);
    m = fmaxf(am, bm);
  }
  __device__ static __forceinline__ void compose_plain(const S& e, S& l) {
    float m, s;
    lse_plain(l.v[0] + e.v[1], e.v[2], l.v[1], l.v[2], m, s);
    l.v[0] = e.v[0] + l.v[0];
    l.v[1] = m;
    l.v[2] = s;
  }
  __device__ static __forceinline__ C apply_plain(const S& s, const C& c) {
    C r;
    lse_plain(s.v[0] + c.v[0], c.v[1], s.v[1], s.v[2], r.v[0], r.v[1]);
    return r;
  }
  __device__ static __forceinline__ C step_plain(float a, float b, const C& c) {
    return apply_plain(S{{a, b, 1.f}}, c);
  }
  __device__ static __forceinline__ float out_plain(const C& c) { return __expf(c.v[0]) * c.v[1]; }
};

// One DPP scan step on a summary: lanes whose mask bit is set compose the
// summary DPP brings in (earlier) in front of their own. `valid` holds exactly
// in the lanes whose DPP source lies in the wave and inside ROW_MASK, so the
// moved value is never read elsewhere.
// PLAIN: the operator's plain composition (a wave whose steps allow it).
template <class Ops, int CTRL, int ROW_MASK, bool PLAIN = false>
__device__ __forceinline__ void scan_step(typename Ops::S& x, bool valid) {
  typename Ops::S e;
#pragma unroll
  for (int i = 0; i < Ops::NS; ++i) e.v[i] = dpp_mov_f<CTRL, ROW_MASK>(x.v[i]);
  if constexpr (PLAIN) {
    if (valid) Ops::compose_plain(e, x);
  } else {
    if (valid) Ops::compose(e, x);
  }
}

// Row and tile of this workgroup in look-back mode.
//   row-major  (block = r * ntiles + c): the tiles of a row run side by side,
//              so concurrent workgroups stream one contiguous stretch of
//              memory. The dense linear scans use it: their descriptors are
//              3 words and a look-back window costs little.
//   tile-major (block = c * rows + r): every row's tile c is dispatched before
//              any row's tile c + 1, so by the time a tile looks back its
//              predecessor has usually published its inclusive value and one
//              descriptor read settles the carry. The matrix kernels (up to
//              48-word descriptors, where reading back through a window cost
//              more than the data), the packed and the log-space scans use it.
//              (On dense linear rows it made concurrent workgroups read the
//              same offset of rows a power of two apart and cost ~10% at
//              T >= 16384.)
// Either way a tile waits only on lower-numbered blocks of its own row, which
// were dispatched earlier, so the look-back always makes progress.
// blk0: index of this launch's first block in the call's numbering (nonzero
// only when a launch runs part of the grid).
template <bool TILE_MAJOR>
__device__ __forceinline__ void tile_of_block(int64_t rows, int ntiles, uint32_t blk0, int64_t& r, int& c) {
  const uint32_t b = blockIdx.x + blk0;
  if constexpr (TILE_MAJOR) {
    const uint32_t q = b / (uint32_t)rows;
    c = (int)q;
    r = (int64_t)(b - q * (uint32_t)rows);
  } else {
    const uint32_t q = b / (uint32_t)ntiles;
    r = (int64_t)q;
    c = (int)(b - q * (uint32_t)ntiles);
  }
}

// Row and tile of this workgroup in grouped order: a row's tiles in groups of
// K consecutive tiles (the last group of a row may be shorter), the groups
// tile-major (group g of every row before group g + 1 of any row) and the K
// tiles of a group row-major, dispatched one after another. K = 1 is
// tile-major, K >= ntiles row-major. A tile's predecessor in its row is always
// an earlier block.
__device__ __forceinline__ void tile_of_block_grouped(int64_t rows, int ntiles, uint32_t blk0, int K, int64_t& r,
                                                      int& c) {
  const uint64_t b = (uint64_t)blockIdx.x + blk0;
  const int nfull = ntiles / K;                // full groups per row
  const uint64_t per = (uint64_t)K * (uint64_t)rows;  // blocks per full group index
  const uint64_t g = b / per;
  if (g < (uint64_t)nfull) {
    const uint64_t w = b - g * per;
    const uint64_t q = w / (uint64_t)K;
    r = (int64_t)q;
    c = (int)(g * (uint64_t)K + (w - q * (uint64_t)K));
  } else {
    const uint64_t Kt = (uint64_t)(ntiles - nfull * K);  // the short last group
    const uint64_t w = b - (uint64_t)nfull * per;
    const uint64_t q = w / Kt;
    r = (int64_t)q;
    c = (int)((uint64_t)nfull * (uint64_t)K + (w - q * Kt));
  }
}

// ---------------------------------------------------------------------------
// Decoupled look-back. Descriptor set of tile i = NS aggregate words followed
// by NC inclusive words (the state at the tile's end). Run by one whole wave;
// returns the state entering tile `c` of the row whose first descriptor set
// is `row_desc`.
// ---------------------------------------------------------------------------
template <class Ops, bool FAST = false>
__device__ __forceinline__ typename Ops::C lookback(Workspace w, const uint64_t* row_desc, int c, uint32_t limit) {
  using S = typename Ops::S;
  constexpr int ND = Ops::NS + Ops::NC;
  const int l = lane_id();
  const uint32_t tagA = kTagAgg, tagI = kTagIncl;
  // fast path (FAST: tile-major dispatch, where it usually succeeds): the
  // immediate predecessor has published its inclusive value
  if constexpr (FAST) {
    bool ok = true;
    typename Ops::C cc;
#pragma unroll
    for (int i = 0; i < Ops::NC; ++i) cc.v[i] = 0.f;
    if (l == 0) {
      const uint64_t* d = row_desc + (int64_t)ND * (c - 1);
#pragma unroll
      for (int i = 0; i < Ops::NC; ++i) {
        const uint64_t wi = ld_u64(d + Ops::NS + i);
        ok = ok && (word_tag(wi) == tagI);
        cc.v[i] = word_val(wi);
      }
    }
    if (__builtin_amdgcn_readfirstlane((int)ok)) {
#pragma unroll
      for (int i = 0; i < Ops::NC; ++i) cc.v[i] = readlane_f(cc.v[i], 0);
      return cc;
    }
  }
  S acc = Ops::ident();  // composition of the tiles already passed (later ones)
  bool found = false;    // acc already ends on an inclusive value
  int j = c - 1;
  uint32_t spins = 0;
  while (true) {
    const int jt = j - l;
    const bool inrow = jt >= 0;
    S e = Ops::ident();
    bool is_incl = false;
    int stop = 64;
    while (true) {
      bool ready = !inrow;
      is_incl = false;
      if (inrow) {
        const uint64_t* d = row_desc + (int64_t)ND * jt;
        bool ok = true;
        typename Ops::C cc;
#pragma unroll
        for (int i = 0; i < Ops::NC; ++i) {
          const uint64_t wi = ld_u64(d + Ops::NS + i);
          ok = ok && (word_tag(wi) == tagI);
          cc.v[i] = word_val(wi);
        }
        if (ok) {
          is_incl = true;
          ready = true;
          e = Ops::of_carry(cc);
        } else {
          bool okA = true;
          S ea;
#pragma unroll
          for (int i = 0; i < Ops::NS; ++i) {
            const uint64_t wa = ld_u64(d + i);
            okA = okA && (word_tag(wa) == tagA);
            ea.v[i] = word_val(wa);
          }
          if (okA) {
            ready = true;
            if (jt == 0) {
              // the row's first tile starts from the initial state, so its
              // inclusive value follows from its aggregate: a window that
              // reaches the row start always ends on an inclusive value
              e = Ops::of_carry(Ops::apply(ea, Ops::cident()));
              is_incl = true;
            } else {
              e = ea;
            }
          }
        }
      }
      const uint64_t incl_mask = __ballot(is_incl);
      stop = incl_mask ? __builtin_ctzll(incl_mask) : 64;
      const uint64_t need = (stop >= 63) ? ~0ull : ((2ull << stop) - 1ull);
      const uint64_t not_ready = __ballot(!ready) & need;
      if (not_ready == 0) break;
      if (++spins > limit) {
        if (l == 0) st_u32(w.hdr + kHdrError, 1u);
        typename Ops::C bad;
#pragma unroll
        for (int i = 0; i < Ops::NC; ++i) bad.v[i] = __builtin_nanf("");
        return bad;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (!found) {
      if (l > stop) e = Ops::ident();
      // reduce lanes stop..0 in time order (higher lane = earlier tile)
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        S o;
#pragma unroll
        for (int i = 0; i < Ops::NS; ++i) o.v[i] = __shfl_down(e.v[i], off, 64);
        if (l + off < 64) Ops::compose(o, e);
      }
      S win;
#pragma unroll
      for (int i = 0; i < Ops::NS; ++i) win.v[i] = readlane_f(e.v[i], 0);
      Ops::compose(win, acc);
      found = stop < 64;
    }
    if (found || j < 64) break;  // an inclusive value, or the row's first tile, closes it
    j -= 64;
  }
  return Ops::carry_of_hard(acc);  // acc ends on an inclusive value: it is hard
}

}  // namespace mscan
