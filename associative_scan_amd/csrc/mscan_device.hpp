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
// Q by zero. For finite data this is exactly the arithmetic result. It also
// makes sequence starts hard boundaries (they enter the scan as P = 0), so a
// NaN or Inf in one packed sequence can never reach the next one.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mscan {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

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

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

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

// One scan step: lanes whose mask bit is set combine with the value DPP brings in.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void lin_scan_step(float& P, float& Q, bool valid) {
  const float pe = dpp_f<CTRL, ROW_MASK>(1.f, P);
  const float qe = dpp_f<CTRL, ROW_MASK>(0.f, Q);
  const bool use = valid && (P != 0.f);
  const float nP = use ? P * pe : P;
  const float nQ = use ? __builtin_fmaf(P, qe, Q) : Q;
  P = nP;
  Q = nQ;
}

// Inclusive scan over the 64 lanes of a wave (lane 0 earliest):
// four row shifts within rows of 16, then the two row broadcasts.
__device__ __forceinline__ void lin_wave_scan(float& P, float& Q) {
  const int l = lane_id();
  lin_scan_step<kRowShr1, 0xf>(P, Q, (l & 15) >= 1);
  lin_scan_step<kRowShr2, 0xf>(P, Q, (l & 15) >= 2);
  lin_scan_step<kRowShr4, 0xf>(P, Q, (l & 15) >= 4);
  lin_scan_step<kRowShr8, 0xf>(P, Q, (l & 15) >= 8);
  lin_scan_step<kRowBcast15, 0xa>(P, Q, (l & 16) != 0);
  lin_scan_step<kRowBcast31, 0xc>(P, Q, l >= 32);
}

// ---------------------------------------------------------------------------
// Workspace: control header, one epoch word per row, descriptor words per tile.
//
// Every descriptor word is 64 bits, {tag:32 | value:32}, written and read with
// relaxed agent-scope atomics, so each word is self-validating and no fence is
// needed between words. tag = (epoch << 2) | kind, kind 1 = aggregate of the
// tile alone, 2 = inclusive value (the state at the tile's end). Each row has
// its own epoch, which the row's last tile advances once its look-back has
// finished (by then every tile of the row has read the epoch), so words from
// earlier calls never look valid, nothing needs clearing between calls and no
// atomic read-modify-write touches a shared address.
// ---------------------------------------------------------------------------
enum : int { kHdrError = 3, kHdrWords = 32 };
enum : uint32_t { kKindAgg = 1, kKindIncl = 2 };

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
  uint32_t* hdr;    // kHdrWords 32-bit control words
  uint32_t* epoch;  // one word per row
  uint64_t* desc;   // per-tile descriptor words
};

// Byte offset of the descriptors: header + per-row epochs rounded up to 16 bytes.
__host__ __device__ __forceinline__ size_t ws_desc_offset(int64_t rows) {
  return (size_t)kHdrWords * 4 + (((size_t)rows * 4 + 15) & ~(size_t)15);
}

__device__ __forceinline__ Workspace ws_view(void* ws, int64_t rows) {
  Workspace w;
  w.hdr = (uint32_t*)ws;
  w.epoch = (uint32_t*)((char*)ws + kHdrWords * 4);
  w.desc = (uint64_t*)((char*)ws + ws_desc_offset(rows));
  return w;
}

// Upper bound on look-back polls before a wave gives up (then the header's
// error word is set and the carry is taken as zero, so the kernel still ends).
constexpr uint32_t kSpinLimit = 1u << 22;

// ---------------------------------------------------------------------------
// Decoupled look-back for scalar linear descriptors.
// Descriptor set of tile i: agg P at desc[3i], agg Q at desc[3i+1], inclusive
// value at desc[3i+2]. Run by one whole wave; returns the state entering tile
// `c` of the row whose first descriptor set is `row_desc`.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float lin_lookback(Workspace w, const uint64_t* row_desc, int c,
                                              uint32_t epoch) {
  const int l = lane_id();
  const uint32_t tagA = (epoch << 2) | kKindAgg, tagI = (epoch << 2) | kKindIncl;
  float accP = 1.f, accQ = 0.f;  // composition of the tiles already passed (later ones)
  int j = c - 1;
  uint32_t spins = 0;
  while (true) {
    const int jt = j - l;
    const bool inrow = jt >= 0;
    float eP = 1.f, eQ = 0.f;
    bool is_incl = false;
    while (true) {
      bool ready = !inrow;
      is_incl = false;
      if (inrow) {
        const uint64_t wi = ld_u64(row_desc + 3 * jt + 2);
        if (word_tag(wi) == tagI) {
          is_incl = true;
          ready = true;
          eP = 0.f;
          eQ = word_val(wi);
        } else {
          const uint64_t wp = ld_u64(row_desc + 3 * jt);
          const uint64_t wq = ld_u64(row_desc + 3 * jt + 1);
          if (word_tag(wp) == tagA && word_tag(wq) == tagA) {
            ready = true;
            eP = word_val(wp);
            eQ = word_val(wq);
          }
        }
      }
      const uint64_t incl_mask = __ballot(is_incl);
      const int stop = incl_mask ? __builtin_ctzll(incl_mask) : 64;
      const uint64_t need = (stop >= 63) ? ~0ull : ((2ull << stop) - 1ull);
      const uint64_t not_ready = __ballot(!ready) & need;
      if (not_ready == 0) break;
      if (++spins > kSpinLimit) {
        if (l == 0) st_u32(w.hdr + kHdrError, 1u);
        return 0.f;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const uint64_t incl_mask = __ballot(is_incl);
    const int stop = incl_mask ? __builtin_ctzll(incl_mask) : 64;
    if (l > stop) { eP = 1.f; eQ = 0.f; }
    // reduce lanes stop..0 in time order (higher lane = earlier tile)
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float pe = __shfl_down(eP, off, 64);
      const float qe = __shfl_down(eQ, off, 64);
      if (l + off < 64) lin_compose(pe, qe, eP, eQ);
    }
    const float wP = readlane_f(eP, 0), wQ = readlane_f(eQ, 0);
    lin_compose(wP, wQ, accP, accQ);
    if (stop < 64) break;
    j -= 64;
  }
  return accQ;  // accP is 0: the window ended on an inclusive value
}

}  // namespace mscan
