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
// Layout: one lane owns EL consecutive time steps; a step's k x k and k x v
// blocks are contiguous, loaded as 16-byte vectors. A tile is WAVES waves x 64
// lanes x EL steps. Inside a tile the steps are summarised per lane as
// (P, Q) = (product of the A's, accumulated B's), scanned across the wave with
// DPP, and across waves through LDS; across tiles the row-loop / look-back
// modes of the scalar kernels apply unchanged (see scan_scalar.hip).
//
// Backward: processing order is the reverse of the forward's; element j is
// (A of the step before it in that order, transposed; dy_j), a sequence's
// first element is (0, dy). Outputs dB = lam, dA_t = lam_t h_prev^T with
// h_prev the forward state before t (h0 at a sequence start), and
// dh0 = A_s^T lam_s at each sequence's forward-first step s.
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
  // out = M * X for M k x k and X k x n (row-major), plus optional addend
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
  // l := (e then l); a zero l.P keeps l (a reset or a sequence start)
  __device__ static __forceinline__ void compose(const S& e, S& l) {
    if (zero_k(l.v)) return;
    S r;
    mul<K>(l.v, e.v, nullptr, r.v);
    mul<V>(l.v, e.v + KK, l.v + KK, r.v + KK);
    l = r;
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

// n floats from a 16-byte (n % 4 == 0) or 8-byte (n == 2) aligned address.
// Cached accesses on purpose: the lanes of a wave touch lane-strided parts of
// the same lines over several instructions, and those lines must stay in L1/L2
// between them (non-temporal accesses measured several times slower here).
template <int N>
__device__ __forceinline__ void vload(const float* p, float* o) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const v4f t = *(const v4f*)(p + 4 * i);
      o[4 * i] = t.x; o[4 * i + 1] = t.y; o[4 * i + 2] = t.z; o[4 * i + 3] = t.w;
    }
  } else if constexpr (N == 2) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f t = *(const v2f*)p;
    o[0] = t.x; o[1] = t.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = p[i];
  }
}

template <int N>
__device__ __forceinline__ void vstore(float* p, const float* v) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      const v4f t = {v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
      *(v4f*)(p + 4 * i) = t;
    }
  } else if constexpr (N == 2) {
    typedef float v2f __attribute__((ext_vector_type(2)));
    const v2f t = {v[0], v[1]};
    *(v2f*)p = t;
  } else {
#pragma unroll
    for (int i = 0; i < N; ++i) p[i] = v[i];
  }
}

// Largest i in [0, n) with v[i] <= q (0 if none).
__device__ __forceinline__ int seg_find(const int32_t* v, int n, int64_t q) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)v[mid] <= q) lo = mid; else hi = mid;
  }
  return lo;
}

constexpr int kMatCuLds = 1024;  // cu_seqlens entries cached in LDS per workgroup
enum : int { kMatRowLoop = 0, kMatLookback = 1 };

// ---------------------------------------------------------------------------
// the kernel
// ---------------------------------------------------------------------------
template <int K, int V, bool BWD, bool REV, bool VARLEN, int MODE, int WAVES, int EL>
__global__ __launch_bounds__(WAVES * 64) void k_matrix(const MatArgs a) {
  using Ops = MatOps<K, V>;
  using S = typename Ops::S;
  using C = typename Ops::C;
  constexpr int KK = K * K, KV = K * V, NS = Ops::NS, NC = Ops::NC, ND = NS + NC;
  constexpr int WSTEPS = 64 * EL;      // steps per wave
  constexpr int TILE = WAVES * WSTEPS;  // steps per tile

  __shared__ float s_agg[2][WAVES][NS];
  __shared__ float s_carry[NC];
  __shared__ int32_t s_cu[VARLEN ? kMatCuLds : 1];

  const int l = lane_id();
  const int w = (int)(threadIdx.x >> 6);
  int64_t r;
  int c_first, c_last;
  if constexpr (MODE == kMatRowLoop) {
    r = blockIdx.x;
    c_first = 0;
    c_last = a.ntiles - 1;
  } else {
    r = blockIdx.x / (uint32_t)a.ntiles;
    c_first = c_last = (int)(blockIdx.x - (uint32_t)r * (uint32_t)a.ntiles);
  }
  const int64_t T = a.T;
  const int64_t row0 = r * a.stride;  // first step of the row
  const bool has_h0 = a.h0 != nullptr;

  Workspace ws{};
  if constexpr (MODE == kMatLookback) ws = ws_view(a.ws);

  // sequence table: cached whole in LDS when it fits, else read from memory
  const int32_t* cuv = a.cu;
  const int ncu = a.nseg + 1;
  if constexpr (VARLEN) {
    if (ncu <= kMatCuLds) {
      for (int i = threadIdx.x; i < ncu; i += WAVES * 64) s_cu[i] = a.cu[i];
      __syncthreads();
      cuv = s_cu;
    }
  }
  // h0 of sequence k for this row (zero when absent)
  auto load_h0 = [&](int k, float* o) {
    if (has_h0) vload<KV>(a.h0 + ((int64_t)k * a.rows + r) * KV, o);
    else {
#pragma unroll
      for (int i = 0; i < KV; ++i) o[i] = 0.f;
    }
  };

  C carry = Ops::cident();
  for (int c = c_first; c <= c_last; ++c) {
    const int64_t j0 = (int64_t)c * TILE + (int64_t)w * WSTEPS + (int64_t)l * EL;  // processing index of step 0
    auto phys = [&](int64_t j) -> int64_t { return REV ? T - 1 - j : j; };

    // ---- load ---------------------------------------------------------------
    // fwd: Am = A_t, Bm = B_t. bwd: Am = A_t (own), Bm = dy_t, Hm = h_t.
    float Am[EL][KK], Bm[EL][KV], Hm[BWD ? EL : 1][KV];
    // a tile wholly inside the row issues every load unconditionally, so all
    // of them are in flight together; only a row's last tile checks steps
    const bool interior = (int64_t)(c + 1) * TILE <= T;
    if (interior) {
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int64_t t = phys(j0 + e);
        vload<KK>(a.A + (row0 + t) * KK, Am[e]);
        vload<KV>(a.B + (row0 + t) * KV, Bm[e]);
        if constexpr (BWD) vload<KV>(a.hs + (row0 + t) * KV, Hm[e]);
      }
    } else {
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int64_t t = phys(j0 + e);
      if (t >= 0 && t < T) {
        vload<KK>(a.A + (row0 + t) * KK, Am[e]);
        vload<KV>(a.B + (row0 + t) * KV, Bm[e]);
        if constexpr (BWD) vload<KV>(a.hs + (row0 + t) * KV, Hm[e]);
      } else {
        // identity step for positions outside the row
#pragma unroll
        for (int i = 0; i < KK; ++i) Am[e][i] = (i % (K + 1) == 0) ? 1.f : 0.f;
#pragma unroll
        for (int i = 0; i < KV; ++i) Bm[e][i] = 0.f;
        if constexpr (BWD) {
#pragma unroll
          for (int i = 0; i < KV; ++i) Hm[e][i] = 0.f;
        }
      }
    }
    }

    // ---- sequence boundaries ----------------------------------------------------
    // first: a sequence's first step in processing order; last: its last one
    uint32_t firstm = 0, lastm = 0;
    int segk[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) segk[e] = 0;
    if constexpr (!VARLEN) {
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int64_t j = j0 + e;
        if (j == 0) firstm |= 1u << e;
        if (j == T - 1) lastm |= 1u << e;
      }
    } else {
      // physical range of the lane's steps, walked upward
      const int64_t tlo = REV ? T - (j0 + EL) : j0;
      int k = seg_find(cuv, ncu, max(tlo, (int64_t)0));
#pragma unroll
      for (int ep = 0; ep < EL; ++ep) {
        const int64_t q = tlo + ep;
        if (q < 0 || q >= T) continue;
        while (k + 1 < ncu && (int64_t)cuv[k + 1] <= q) ++k;
        const bool is_start = (int64_t)cuv[k] == q;
        const bool is_end = (k + 1 < ncu) && ((int64_t)cuv[k + 1] - 1 == q);
        const int e = REV ? EL - 1 - ep : ep;
        segk[e] = min(max(k, 0), a.nseg - 1);
        if (REV ? is_end : is_start) firstm |= 1u << e;
        if (REV ? is_start : is_end) lastm |= 1u << e;
      }
    }

    // ---- elements (X, Y) of the scan in processing order -------------------------
    // fwd: X = A_t, Y = B_t (sequence start: X = 0, Y = A h0 + B)
    // bwd: X = (A of the previous step in processing order)^T, Y = dy_t
    //      (sequence start: X = 0), N = forward state before t (h0 at the
    //      sequence's forward-first step)
    // (the forward keeps X in Am itself; the backward needs A_t for dh0)
    float Xb[BWD ? EL : 1][KK], N[BWD ? EL : 1][KV];
    auto X = [&](int e) -> float* {
      if constexpr (BWD) return Xb[e];
      else return Am[e];
    };
    if constexpr (!BWD) {
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        if (firstm & (1u << e)) {
          float h0v[KV], y[KV];
          load_h0(segk[e], h0v);
          Ops::template mul<V>(Am[e], h0v, Bm[e], y);
#pragma unroll
          for (int i = 0; i < KV; ++i) Bm[e][i] = y[i];
#pragma unroll
          for (int i = 0; i < KK; ++i) Am[e][i] = 0.f;
        }
      }
    } else {
      // previous step's A (lane before / wave before) and next step's h
      float Ap[KK], Hn[KV];
#pragma unroll
      for (int i = 0; i < KK; ++i) Ap[i] = __shfl_up(Am[EL - 1][i], 1, 64);
#pragma unroll
      for (int i = 0; i < KV; ++i) Hn[i] = __shfl_down(Hm[0][i], 1, 64);
      if (l == 0) {
        const int64_t t = phys(j0 - 1);
        if (j0 - 1 >= 0 && t >= 0 && t < T) vload<KK>(a.A + (row0 + t) * KK, Ap);
      }
      if (l == 63) {
        const int64_t t = phys(j0 + EL);
        if (t >= 0 && t < T) vload<KV>(a.hs + (row0 + t) * KV, Hn);
        else {
#pragma unroll
          for (int i = 0; i < KV; ++i) Hn[i] = 0.f;
        }
      }
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const float* src = (e == 0) ? Ap : Am[e - 1];
        const bool first = firstm & (1u << e);
#pragma unroll
        for (int p = 0; p < K; ++p)
#pragma unroll
          for (int q = 0; q < K; ++q) Xb[e][p * K + q] = first ? 0.f : src[q * K + p];
        const float* hn = (e == EL - 1) ? Hn : Hm[e + 1];
        if (lastm & (1u << e)) {
          load_h0(segk[e], N[e]);
        } else {
#pragma unroll
          for (int i = 0; i < KV; ++i) N[e][i] = hn[i];
        }
      }
    }

    // ---- lane-serial summary ------------------------------------------------------
    S sum = Ops::ident();
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      if (Ops::zero_k(X(e))) {
#pragma unroll
        for (int i = 0; i < KK; ++i) sum.v[i] = 0.f;
#pragma unroll
        for (int i = 0; i < KV; ++i) sum.v[KK + i] = Bm[e][i];
      } else {
        S nx;
        Ops::template mul<K>(X(e), sum.v, nullptr, nx.v);
        Ops::template mul<V>(X(e), sum.v + KK, Bm[e], nx.v + KK);
        sum = nx;
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
    S ex = Ops::ident(), tagg = wagg;
    if constexpr (WAVES > 1) {
      const int buf = c & 1;
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

    // ---- across tiles: decoupled look-back ------------------------------------------
    if constexpr (MODE == kMatLookback) {
      uint64_t* rd = ws.desc + (int64_t)ND * ((int64_t)r * a.ntiles);
      uint64_t* my = rd + (int64_t)ND * c;
      if (w == 0) {
        const uint32_t tagA = kTagAgg, tagI = kTagIncl;
        const bool hard = Ops::hard(tagg);
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
        if (c > 0) carry = lookback<Ops>(ws, rd, c);
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

    // ---- apply and store ---------------------------------------------------------
    {
      const C hw = Ops::apply(ex, carry);  // state entering this wave's span
      const C v = Ops::apply(sum, hw);     // state after this lane
      C st;
#pragma unroll
      for (int i = 0; i < NC; ++i) {
        st.v[i] = __shfl_up(v.v[i], 1, 64);
        if (l == 0) st.v[i] = hw.v[i];
      }
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        if (Ops::zero_k(X(e))) {
#pragma unroll
          for (int i = 0; i < KV; ++i) st.v[i] = Bm[e][i];
        } else {
          C nx;
          Ops::template mul<V>(X(e), st.v, Bm[e], nx.v);
          st = nx;
        }
        const int64_t t = phys(j0 + e);
        if (t >= 0 && t < T) {
          vstore<KV>(a.out0 + (row0 + t) * KV, st.v);
          if constexpr (BWD) {
            // dA_t = lam_t h_prev^T (k x k)
            float dA[KK];
#pragma unroll
            for (int p = 0; p < K; ++p)
#pragma unroll
              for (int q = 0; q < K; ++q) {
                float acc = 0.f;
#pragma unroll
                for (int u = 0; u < V; ++u) acc = __builtin_fmaf(st.v[p * V + u], N[e][q * V + u], acc);
                dA[p * K + q] = acc;
              }
            vstore<KK>(a.out1 + (row0 + t) * KK, dA);
            if (a.dh0 && (lastm & (1u << e))) {
              // dh0 = A_s^T lam_s
              float d[KV];
#pragma unroll
              for (int p = 0; p < K; ++p)
#pragma unroll
                for (int u = 0; u < V; ++u) {
                  float acc = 0.f;
#pragma unroll
                  for (int q = 0; q < K; ++q) acc = __builtin_fmaf(Am[e][q * K + p], st.v[q * V + u], acc);
                  d[p * V + u] = acc;
                }
              float* dst = a.dh0 + ((int64_t)segk[e] * a.rows + r) * KV;
#pragma unroll
              for (int i = 0; i < KV; ++i) dst[i] = d[i];
            }
          }
        }
      }
    }
    carry = Ops::apply(tagg, carry);  // state at the end of the tile
  }
}

// ---------------------------------------------------------------------------
// host launch
// ---------------------------------------------------------------------------
template <int K, int V>
struct MatCfg;
// (waves per workgroup, steps per lane) for forward / backward
template <> struct MatCfg<2, 1> { static constexpr int W = 4, EF = 8, EB = 4; };
template <> struct MatCfg<2, 2> { static constexpr int W = 4, EF = 4, EB = 4; };
template <> struct MatCfg<4, 1> { static constexpr int W = 4, EF = 4, EB = 2; };
template <> struct MatCfg<4, 4> { static constexpr int W = 4, EF = 4, EB = 2; };

template <int K, int V>
int64_t matrix_tile_steps(bool bwd) {
  return (int64_t)MatCfg<K, V>::W * 64 * (bwd ? MatCfg<K, V>::EB : MatCfg<K, V>::EF);
}

template <int K, int V, bool BWD, bool REV>
static hipError_t launch_mat(const MatArgs& a0, hipStream_t st) {
  constexpr int W = MatCfg<K, V>::W, E = BWD ? MatCfg<K, V>::EB : MatCfg<K, V>::EF;
  MatArgs a = a0;
  a.ntiles = (int32_t)((a.T + W * 64 * E - 1) / (W * 64 * E));
  const bool lookback = scalar_uses_lookback(a.rows, a.ntiles);
  const bool varlen = a.cu != nullptr;
  const dim3 block(W * 64);
  if (!lookback) {
    const dim3 grid((unsigned)a.rows);
    if (varlen) hipLaunchKernelGGL((k_matrix<K, V, BWD, REV, true, kMatRowLoop, W, E>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((k_matrix<K, V, BWD, REV, false, kMatRowLoop, W, E>), grid, block, 0, st, a);
  } else {
    // fresh descriptors for this call (zero tag = not published)
    const size_t words = (size_t)a.rows * (size_t)a.ntiles * (size_t)(MatOps<K, V>::NS + MatOps<K, V>::NC);
    const hipError_t z = launch_zero(a.ws, ws_desc_offset() + words * sizeof(uint64_t), st);
    if (z != hipSuccess) return z;
    const dim3 grid((unsigned)((uint64_t)a.rows * (uint64_t)a.ntiles));
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

int64_t matrix_tiles(int64_t T, int k, int v, bool bwd) {
  int64_t tile = 0;
  if (k == 2 && v == 1) tile = matrix_tile_steps<2, 1>(bwd);
  else if (k == 2 && v == 2) tile = matrix_tile_steps<2, 2>(bwd);
  else if (k == 4 && v == 1) tile = matrix_tile_steps<4, 1>(bwd);
  else if (k == 4 && v == 4) tile = matrix_tile_steps<4, 4>(bwd);
  else return 0;
  return (T + tile - 1) / tile;
}

hipError_t launch_matrix(const MatArgs& a, int k, int v, bool bwd, hipStream_t st) {
  if (k == 2 && v == 1) return launch_kv<2, 1>(a, bwd, st);
  if (k == 2 && v == 2) return launch_kv<2, 2>(a, bwd, st);
  if (k == 4 && v == 1) return launch_kv<4, 1>(a, bwd, st);
  if (k == 4 && v == 4) return launch_kv<4, 4>(a, bwd, st);
  return hipErrorInvalidValue;
}

}  // namespace mscan
