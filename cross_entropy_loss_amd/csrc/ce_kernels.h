// ce_kernels.h -- gfx950 device code for token-level softmax cross-entropy.
//
// What is computed (per logit row x[0..V) with label y; the pages' "Fast
// Cross Entropy" kernel, PyPI page "fms-acceleration-foak 0.7.4", kernel
// list): the softmax cross-entropy loss lse - x_y, its token mean over rows
// whose label is not ignore_index (fms-hf-tuning PR #280, "Early Version Of
// This Plugin": per-token averaging), and the gradient
// (softmax - onehot) * dloss / n_valid.
//
// Shape of the work on CDNA4.  The path is a streaming row reduction bound by
// HBM bandwidth, not a contraction, so there is no MFMA here.  One workgroup
// owns one row (or one vocabulary slab of a row).  Every lane issues all of
// its 16-byte loads of the row up front (VPL loads per lane, NT lanes, held
// in VGPRs: 64 VGPRs for a 64000-byte bf16 row at NT=256), so the row is read
// from HBM once and the gradient is computed from registers and written once.
//
// Numerics for 16-bit inputs (fp32 arithmetic, v_exp_f32 on base 2):
//   pass 0  per-lane max m_l (bf16: also a lower bound of the lane minimum)
//   pass 1  per-lane s_l = sum_{j != y} 2^{(x_j - m_l) log2 e}; the label
//           element is set to -inf in registers first, so the sum excludes it
//           without a subtraction
//   merge   (m, s) pairs across the workgroup -> M, S_excl
//   row     e_y = exp(x_y - M), S = S_excl + e_y, lse = M + log S,
//           q = S_excl / S  (= 1 - p_y, no cancellation)
//           loss = lse - x_y when q >= 1/2, else log1p(S_excl / e_y)
//   pass 2  g_j = 2^{(x_j - lse) log2 e} * s  (s = dloss / n_valid),
//           g_y = -s q, rounded once to the storage format (nearest-even).
// fp32 inputs run the same steps in fp64 and round once to fp32.
//
// The valid-token count.  The gradient scale needs n_valid of the whole
// batch before any row is written.  The first K workgroups of the launch
// each count a slice of the labels and publish an epoch-tagged partial count
// (one 64-bit relaxed agent-scope atomic store: tag << 32 | bad << 31 |
// count); every row polls the K words with a bounded wait.  Workgroups are
// dispatched in increasing id order on each XCD, so the K counters are
// resident before any poller can fill the machine; the wait is bounded
// anyway (CE_STATUS_SYNC_TIMEOUT) so a wave never spins forever.
//
// The mean.  Each row publishes its loss into its own epoch-tagged 64-bit
// slot of the workspace (tag << 32 | loss bits: one relaxed agent-scope
// store, so no fence and no shared counter).  The last workgroup of the grid
// polls the N slots, sums the losses in row order in fp64 (deterministic),
// writes L, n_valid and the status word, then bumps the epoch so the
// workspace is ready for the next call.  No workgroup ever waits for the
// finisher, so the wait cannot deadlock.  (Same-address device-scope atomics,
// one per workgroup, serialise at the memory side at tens of ns each, and an
// agent-scope release writes back the whole L2: both cost more than the
// kernel itself at these sizes.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ce_buffer.h"

namespace cek {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kStatusLabelRange = 0x1u;
constexpr uint32_t kStatusSyncTimeout = 0x2u;
constexpr int kMaxCounters = 64;
constexpr int kSpinLimit = 1 << 18;  // default polls (each a memory round trip plus s_sleep): ~0.5 s

// ---------------------------------------------------------------------------
// Workspace header (device memory owned by the caller, zero-filled once).
// ---------------------------------------------------------------------------
struct WsHeader {
  uint32_t epoch;  // bumped by the finishing workgroup of every call
  uint32_t flags;  // status bits raised by workgroups of the running call
  uint32_t pad0[14];
  uint64_t part[kMaxCounters];  // tagged partial label counts
};
constexpr size_t kWsHeaderBytes = 1024;
static_assert(sizeof(WsHeader) <= kWsHeaderBytes, "header too large");

__device__ __forceinline__ uint64_t ld_agent(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Reinterpret one 32-bit lane word.  The word is taken by value: clang's
// __builtin_bit_cast applied directly to an ext-vector element expression
// (v[i]) reads element 0 whatever i is, so element accesses never go into a
// bit cast directly.
template <typename T>
__device__ __forceinline__ T as(uint32_t w) {
  return __builtin_bit_cast(T, w);
}

// ---------------------------------------------------------------------------
// Element formats.  A 16-byte vector holds EPV elements.
// ---------------------------------------------------------------------------
struct BF16 {
  static constexpr int ESZ = 2, EPV = 8;
  static constexpr bool kBF = true;
  typedef uint16_t bits_t;
  typedef float acc_t;
  // smallest |scale| at which a flushed 2^t (t < -126) could change a rounded
  // output: scale * 2^-126 reaches half of the smallest subnormal 2^-133
  static constexpr float kSlowScale = 0x1p-8f;
  __device__ static float lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
  __device__ static float hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
  __device__ static float load1(uint16_t b) { return __builtin_bit_cast(float, (uint32_t)b << 16); }
  __device__ static uint32_t pack(float a, float b) {
    f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
  }
  __device__ static uint16_t store1(float a) { return (uint16_t)(pack(a, 0.0f) & 0xffffu); }
  __device__ static void kill(u32x4& v, int e) {  // element e := -inf
    const uint32_t mask = (e & 1) ? 0xffff0000u : 0x0000ffffu;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      if (d == (e >> 1)) v[d] = (v[d] & ~mask) | (0xff80ff80u & mask);
  }
};

struct F16 {
  static constexpr int ESZ = 2, EPV = 8;
  static constexpr bool kBF = false;
  typedef uint16_t bits_t;
  typedef float acc_t;
  // fp16's smallest subnormal is 2^-24, so flushed 2^t below 2^-126 matter
  // only for |scale| above 2^101
  static constexpr float kSlowScale = 0x1p101f;
  __device__ static float lo(uint32_t u) { return (float)__builtin_bit_cast(h2, u).x; }
  __device__ static float hi(uint32_t u) { return (float)__builtin_bit_cast(h2, u).y; }
  __device__ static float load1(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
  __device__ static uint32_t pack(float a, float b) {
    f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  }
  __device__ static uint16_t store1(float a) { return (uint16_t)(pack(a, 0.0f) & 0xffffu); }
  __device__ static void kill(u32x4& v, int e) {
    const uint32_t mask = (e & 1) ? 0xffff0000u : 0x0000ffffu;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      if (d == (e >> 1)) v[d] = (v[d] & ~mask) | (0xfc00fc00u & mask);
  }
};

struct F32 {
  static constexpr int ESZ = 4, EPV = 4;
  typedef uint32_t bits_t;
  typedef double acc_t;
  __device__ static float load1(uint32_t b) { return __builtin_bit_cast(float, b); }
  __device__ static uint32_t store1(float a) { return __builtin_bit_cast(uint32_t, a); }
  __device__ static void kill(u32x4& v, int e) {
#pragma unroll
    for (int d = 0; d < 4; ++d)
      if (d == e) v[d] = 0xff800000u;
  }
};

// ---------------------------------------------------------------------------
// Cache policy of the streaming loads and stores (bit 0: nontemporal loads,
// bit 1: nontemporal stores).
// ---------------------------------------------------------------------------
template <int POL>
__device__ __forceinline__ u32x4 ldv(const u32x4* p) {
  if constexpr (POL & 1) return __builtin_nontemporal_load(p);
  else return *p;
}
template <int POL>
__device__ __forceinline__ void stv(u32x4* p, u32x4 v) {
  if constexpr (POL & 2) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---------------------------------------------------------------------------
// Reductions.
// ---------------------------------------------------------------------------
template <typename F>
__device__ __forceinline__ F wave_sum(F v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v |= __shfl_xor(v, o, 64);
  return v;
}

// Merge of two (max, sum-relative-to-max) pairs; a pair with m = -inf is empty.
__device__ __forceinline__ void ms_merge(double& m, double& s, double m2, double s2) {
  const double M = fmax(m, m2);
  const double a = (m == -INFINITY) ? 0.0 : s * exp(m - M);
  const double b = (m2 == -INFINITY) ? 0.0 : s2 * exp(m2 - M);
  m = M;
  s = a + b;
}
// e^d in fp64 for the per-element passes over fp32 rows.  t = d log2(e) is
// split as n + f with n = rint(t) and |f| <= 1/2, so e^d = 2^n e^(f ln 2); the
// second factor is the Taylor series of the exponential at 0 in f ln 2 to
// degree 11, whose truncation error is below 7e-15 relative for
// |f ln 2| <= 0.35, and 2^n is applied exactly by ldexp.  The relative error is
// a few 1e-15 wherever the result is a normal fp64 number, far inside the
// 6e-8 that one rounding to fp32 leaves for a 1-ulp gradient.  t below -1100
// (d = -inf included) gives +0; NaN stays NaN.  About 21 VALU instructions,
// against about twice that for the library exp with its special-case
// handling; the library exp and log remain in use for per-row quantities.
constexpr double kLn2d = 0.69314718055994530942;
constexpr double kLog2ed = 1.44269504088896340736;
constexpr double taylor_coef(int k) {  // (ln 2)^k / k!
  double r = 1.0;
  for (int i = 1; i <= k; ++i) r = r * kLn2d / i;
  return r;
}
__device__ __forceinline__ double exp_f64(double d) {
  constexpr double c[12] = {taylor_coef(0), taylor_coef(1), taylor_coef(2),  taylor_coef(3),
                            taylor_coef(4), taylor_coef(5), taylor_coef(6),  taylor_coef(7),
                            taylor_coef(8), taylor_coef(9), taylor_coef(10), taylor_coef(11)};
  const double t = d * kLog2ed;
  const double n = __builtin_rint(t);
  const double f = t - n;
  double p = c[11];
#pragma unroll
  for (int k = 10; k >= 0; --k) p = fma(p, f, c[k]);
  const int ni = (int)fmin(fmax(n, -2000.0), 2000.0);  // NaN -> -2000 (p is NaN then)
  const double r = ldexp(p, ni);
  return (t < -1100.0) ? 0.0 : r;
}

__device__ __forceinline__ float first_lane(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// Reductions on DPP lane moves (no LDS traffic).  A step combines each lane
// with the lane a DPP control selects; lanes a row mask leaves out combine
// with the identity.  After quad_perm [1,0,3,2], [2,3,0,1], row_half_mirror
// and row_mirror every lane of a 16-lane row holds the row's result;
// row_bcast15 (rows 1, 3) and row_bcast31 (rows 2, 3) then leave the
// wave's result in lane 63.
struct OpMax {
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
  __device__ float operator()(float a, float b) const { return fminf(a, b); }
};
struct OpAdd {
  __device__ float operator()(float a, float b) const { return a + b; }
};
template <int CTRL, int ROWS, typename Op>
__device__ __forceinline__ float dpp_step(float v, float ident, Op op) {
  const int t = __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, ident), __builtin_bit_cast(int, v), CTRL, ROWS,
                                            0xf, false);
  return op(v, __builtin_bit_cast(float, t));
}
// Result of the first N lanes (N = 1, 2, 4, 8 or 16) in each of them.
template <int N, typename Op>
__device__ __forceinline__ float row_reduce(float v, float ident, Op op) {
  if constexpr (N >= 2) v = dpp_step<0xb1, 0xf>(v, ident, op);   // quad_perm [1,0,3,2]
  if constexpr (N >= 4) v = dpp_step<0x4e, 0xf>(v, ident, op);   // quad_perm [2,3,0,1]
  if constexpr (N >= 8) v = dpp_step<0x141, 0xf>(v, ident, op);  // row_half_mirror
  if constexpr (N >= 16) v = dpp_step<0x140, 0xf>(v, ident, op); // row_mirror
  return v;
}
// Result of the whole wave, the same in every lane.
template <typename Op>
__device__ __forceinline__ float wave_reduce(float v, float ident, Op op) {
  v = row_reduce<16>(v, ident, op);
  v = dpp_step<0x142, 0xa>(v, ident, op);  // row_bcast15
  v = dpp_step<0x143, 0xc>(v, ident, op);  // row_bcast31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Row statistics of a workgroup from each lane's (max m, sum s relative to
// m, min mn): every wave reduces its maxima, rescales each lane's sum once
// and adds, then the NW wave triples (LDS) are reduced the same way in the
// first NW lanes of every wave, so all waves hold the same M, S, MN.
template <int NW>
__device__ __forceinline__ void row_stats(float m, float s, float mn, float* lm, float* ls, float* lmn, float& M,
                                          float& S, float& MN) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const float mw = wave_reduce(m, -INFINITY, OpMax());
  float sw = (m == -INFINITY) ? 0.0f : s * __builtin_amdgcn_exp2f((m - mw) * kLog2e);
  sw = wave_reduce(sw, 0.0f, OpAdd());
  const float nw = wave_reduce(mn, INFINITY, OpMin());
  if (lane == 0) {
    lm[wid] = mw;
    ls[wid] = sw;
    lmn[wid] = nw;
  }
  __syncthreads();
  float pm = -INFINITY, ps = 0.0f, pn = INFINITY;
  if (lane < NW) {
    pm = lm[lane];
    ps = ls[lane];
    pn = lmn[lane];
  }
  const float mb = row_reduce<NW>(pm, -INFINITY, OpMax());
  ps = (pm == -INFINITY) ? 0.0f : ps * __builtin_amdgcn_exp2f((pm - mb) * kLog2e);
  ps = row_reduce<NW>(ps, 0.0f, OpAdd());
  pn = row_reduce<NW>(pn, INFINITY, OpMin());
  M = first_lane(mb);
  S = first_lane(ps);
  MN = first_lane(pn);
}



// (max, sum) statistics of a workgroup whose lanes hold a max m (an input
// value) and a sum s relative to it, for the fp64 sums of fp32 rows and for
// slab partials: the workgroup max first (DPP within each wave, the waves'
// maxima through LDS), then one rescale per lane, then the sum (shuffles
// within each wave, the waves' sums added in wave order).  Deterministic;
// every thread returns the same M and S.  (Merging (max, sum) pairs at every
// shuffle step instead costs two exponentials per step and lane.)
__device__ __forceinline__ float rescale(float s, float m, float M) {
  return s * __builtin_amdgcn_exp2f((m - M) * kLog2e);
}
__device__ __forceinline__ double rescale(double s, float m, float M) { return s * exp_f64((double)m - (double)M); }
template <int NW, typename A>
__device__ __forceinline__ void block_ms(float m, A s, float* lm, A* ls, float& M, A& S) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const float mw = wave_reduce(m, -INFINITY, OpMax());
  if (lane == 0) lm[wid] = mw;
  __syncthreads();
  float mb = lm[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) mb = fmaxf(mb, lm[w]);
  A r = (m == -INFINITY) ? (A)0 : rescale(s, m, mb);
  r = wave_sum(r);
  if (lane == 0) ls[wid] = r;
  __syncthreads();
  A t = ls[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) t += ls[w];
  M = mb;
  S = t;
}

// ---------------------------------------------------------------------------
// Per-call arguments.
// ---------------------------------------------------------------------------
struct Args {
  char* logits;  // row i at logits + i * ld * ESZ
  int64_t ld;    // row stride in elements
  char* grad;    // gradient rows (== logits for in-place)
  int64_t grad_ld;
  const int64_t* labels;
  int64_t N, V, ignore;
  const float* dloss;  // NULL = 1
  float* loss_mean;
  float* loss_rows;
  double* lse_rows;    // nullable
  double* pcomp_rows;  // nullable
  int32_t* n_valid_out;
  const int32_t* n_valid_in;  // backward
  const double* lse_in;       // backward
  const double* pcomp_in;     // backward
  uint32_t* status;           // nullable
  WsHeader* ws;
  uint64_t* slots;   // [N] tagged per-row losses for the finisher
  double2* slab_ms;  // [N * C] (max, label-excluded sum) per vocabulary slab
  float* slab_xy;    // [N] label logit, written by the slab that holds it
  int64_t chunk;     // slab width in elements (chunked kernels)
  int C;             // slabs per row
  int K;             // counter workgroups (each publishes one partial count)
  int Kpoll;         // partial-count words a poller waits for (K; more only
                     // when a host-side test forces the bounded wait to expire)
  int spin_limit;    // polls before a wait gives up (CE_STATUS_SYNC_TIMEOUT)
};

// Geometry of V elements starting at `base`: `head` elements before the first
// 16-byte boundary, `nvec` aligned 16-byte vectors, then `tail` elements.
struct Geom {
  int head, tail, nvec;
};
template <int ESZ, int EPV>
__device__ __forceinline__ Geom geom(const char* base, int64_t V) {
  Geom g;
  const uintptr_t a = (uintptr_t)base;
  int64_t h = (int64_t)(((16 - (a & 15)) & 15) / ESZ);
  if (h > V) h = V;
  g.head = (int)h;
  g.nvec = (int)((V - h) / EPV);
  g.tail = (int)((V - h) % EPV);
  return g;
}

// Where element j (0 <= j < V, or -1 for none) of a geometry lives, as seen by
// lane `tid` of NT: in this lane's head slot, tail slot, or body vector k,
// element e.  Fields are -1 when this lane does not hold it.
struct Owner {
  int head, tail, k, e;
};
template <int NT, int EPV>
__device__ __forceinline__ Owner owner(const Geom& g, int64_t j, int tid) {
  Owner o = {-1, -1, -1, 0};
  if (j < 0) return o;
  if (j < g.head) {
    if (tid == (int)j) o.head = 1;
  } else if (j - g.head < (int64_t)g.nvec * EPV) {
    const int vy = (int)((j - g.head) / EPV);
    if (tid == vy % NT) {
      o.k = vy / NT;
      o.e = (int)((j - g.head) % EPV);
    }
  } else if (tid == (int)(j - g.head - (int64_t)g.nvec * EPV)) {
    o.tail = 1;
  }
  return o;
}

// ---------------------------------------------------------------------------
// Label counting, the poll, loss publication and the call's finish.
// ---------------------------------------------------------------------------
// Counter workgroup j of K counts labels [N*j/K, N*(j+1)/K) and publishes.
template <int NT>
__device__ void count_and_publish(const Args& a, int j, uint32_t tag, uint32_t* lds_u32) {
  const int tid = threadIdx.x;
  const int64_t i0 = a.N * j / a.K, i1 = a.N * (j + 1) / a.K;
  uint32_t cnt = 0, bad = 0;
  for (int64_t i = i0 + tid; i < i1; i += NT) {
    const int64_t y = a.labels[i];
    if (y != a.ignore) {
      cnt += 1;
      bad |= (y < 0 || y >= a.V) ? 1u : 0u;
    }
  }
  cnt = wave_sum(cnt);
  bad = wave_or(bad);
  const int w = tid >> 6;
  if ((tid & 63) == 0) {
    lds_u32[2 * w] = cnt;
    lds_u32[2 * w + 1] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    uint32_t c = 0, b = 0;
    for (int k = 0; k < NT / 64; ++k) {
      c += lds_u32[2 * k];
      b |= lds_u32[2 * k + 1];
    }
    st_agent(&a.ws->part[j], ((uint64_t)tag << 32) | ((uint64_t)(b & 1u) << 31) | (uint64_t)(c & 0x7fffffffu));
  }
  __syncthreads();
}

// Raises a status bit (rare error paths only) and waits until it has landed,
// so that it is visible before this workgroup publishes its row.
__device__ __forceinline__ void raise_flag(const Args& a, uint32_t bit) {
  __hip_atomic_fetch_or(&a.ws->flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wave 0 polls the partial counts and leaves n_valid, the bad-label bit and
// the timeout bit in lds_u[0..2] (read them after a barrier).  A wait that
// gives up raises CE_STATUS_SYNC_TIMEOUT; the count is then unknown, and the
// gradient scale of this workgroup becomes NaN (call_scale), so an expired
// wait can never pass for a valid result.
__device__ void poll_to_lds(const Args& a, uint32_t tag, uint32_t* lds_u) {
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63;
  uint64_t w = 0;
  uint32_t to = 0;
  if (lane < a.Kpoll) {
    for (int it = 0;; ++it) {
      w = ld_agent(&a.ws->part[lane]);
      if ((uint32_t)(w >> 32) == tag) break;
      if (it >= a.spin_limit) {
        to = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  uint32_t c = (lane < a.Kpoll) ? (uint32_t)(w & 0x7fffffffu) : 0u;
  uint32_t b = (lane < a.Kpoll) ? (uint32_t)((w >> 31) & 1u) : 0u;
  c = wave_sum(c);
  b = wave_or(b);
  to = wave_or(to);
  if (lane == 0) {
    lds_u[0] = c;
    lds_u[1] = b;
    lds_u[2] = to;
    if (to) raise_flag(a, kStatusSyncTimeout);
  }
}

// The same sums when the counts were published by an earlier launch of the
// call (already complete, so nothing to wait for).  Kernels whose workgroups
// are not all waited on by the finisher must use this form: a workgroup that
// polls with the epoch it read could start after the finisher has bumped the
// epoch and wait for a tag that never comes.
__device__ void counts_to_lds(const Args& a, uint32_t* lds_u) {
  if ((threadIdx.x >> 6) != 0) return;
  const int lane = threadIdx.x & 63;
  const uint64_t w = (lane < a.K) ? ld_agent(&a.ws->part[lane]) : 0ull;
  uint32_t c = (uint32_t)(w & 0x7fffffffu);
  uint32_t b = (uint32_t)((w >> 31) & 1u);
  c = wave_sum(c);
  b = wave_or(b);
  if (lane == 0) {
    lds_u[0] = c;
    lds_u[1] = b;
    lds_u[2] = 0u;
  }
}

// The gradient scale dloss / n_valid from the count in lds_u (NaN when this
// workgroup's wait for the count gave up).
__device__ __forceinline__ double call_scale(const Args& a, const uint32_t* lds_u) {
  if (lds_u[2]) return __builtin_nan("");
  return (a.dloss ? (double)a.dloss[0] : 1.0) / (double)lds_u[0];
}

// A row's loss, published for the finisher (one thread).
__device__ __forceinline__ void publish_loss(const Args& a, int64_t row, float loss, uint32_t tag) {
  st_agent(&a.slots[row], ((uint64_t)tag << 32) | (uint64_t)__builtin_bit_cast(uint32_t, loss));
}

// Run by the last workgroup of the grid, after its own row: waits for every
// row's tagged loss, sums in row order (fp64), writes L, n_valid and status,
// and bumps the epoch.  n, bad and the poll's timeout bit come from this
// workgroup's poll (lds_u[0..2]).  After any expired wait L is NaN.
template <int NT>
__device__ void finish_call(const Args& a, uint32_t epoch, const uint32_t* lds_u, double* lds_d) {
  const int tid = threadIdx.x;
  const uint32_t n = lds_u[0], bad = lds_u[1], poll_to = lds_u[2];
  const uint32_t tag = epoch + 1u;
  constexpr int B = 8;  // slot loads in flight per lane
  double acc = 0.0;
  uint32_t to = 0;
  for (int64_t base = 0; base < a.N; base += (int64_t)NT * B) {
    uint64_t w[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      if (i < a.N) w[j] = ld_agent(&a.slots[i]);
    }
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int64_t i = base + (int64_t)j * NT + tid;
      if (i < a.N) {
        // once one wait has expired the call is already invalid: stop waiting
        for (int it = 0; (uint32_t)(w[j] >> 32) != tag; ++it) {
          if (to || it >= a.spin_limit) {
            to = 1;
            break;
          }
          __builtin_amdgcn_s_sleep(2);
          w[j] = ld_agent(&a.slots[i]);
        }
        acc += (double)__builtin_bit_cast(float, (uint32_t)(w[j] & 0xffffffffu));
      }
    }
  }
  lds_d[tid] = acc;
  __syncthreads();
#pragma unroll
  for (int s = NT / 2; s >= 1; s >>= 1) {
    if (tid < s) lds_d[tid] += lds_d[tid + s];
    __syncthreads();
  }
  const int any_to = __syncthreads_or((int)to);
  if (tid == 0) {
    const uint32_t flags = ld_agent(&a.ws->flags) | (any_to ? kStatusSyncTimeout : 0u);
    a.loss_mean[0] = (any_to || poll_to) ? __builtin_nanf("") : (float)(lds_d[0] / (double)n);
    a.n_valid_out[0] = (int32_t)n;
    if (a.status) a.status[0] = (bad ? kStatusLabelRange : 0u) | flags;
    st_agent(&a.ws->flags, 0u);
    st_agent(&a.ws->epoch, epoch + 1u);
  }
}

// ---------------------------------------------------------------------------
// Lane passes over the staged vectors (16-bit formats, fp32 arithmetic).
// ---------------------------------------------------------------------------
// pass 0: lane max; for bf16 also the lane min.  Both bf16 elements of a
// dword are widened exactly (reading the high one as the whole dword would
// turn a -inf next to a nonzero low half into a signalling NaN, which the
// three-input max does not skip).
// K0..K1: the vector slots taken (all by default; a vocabulary chunk of the
// row otherwise).  MIN = false leaves mn alone (callers that need no min).
// The bf16 max and min take one three-input instruction per dword (the
// compiler left most of them as two two-input ones).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
template <typename T, int NT, int VPL, int K0 = 0, int K1 = VPL, bool MIN = true>
__device__ __forceinline__ void pass0_16(const u32x4 (&v)[VPL], int nvec, int tid, float& m, float& mn) {
#pragma unroll
  for (int k = K0; k < K1; ++k) {
    if (k * NT + tid < nvec) {
      if constexpr (T::kBF) {
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t u = v[k][d];
          const float a0 = T::hi(u), a1 = T::lo(u);
          m = max3f(m, a0, a1);
          if constexpr (MIN) mn = min3f(mn, a0, a1);
        }
      } else {
        h2 hm = as<h2>(v[k][0]);
#pragma unroll
        for (int d = 1; d < 4; ++d) hm = __builtin_elementwise_max(hm, as<h2>(v[k][d]));
        m = fmaxf(m, fmaxf((float)hm.x, (float)hm.y));
      }
    }
  }
}

// The label element (vector slot kx, element ex of this lane; kx = -1 in
// the other lanes) set to -inf in the staged registers, once per row after
// pass 0: pass 1 then sums without it (2^-inf = 0) and pass 2 writes 0 there,
// which the owner lane overwrites with the label's gradient after the row's
// stores.  No per-element select remains in either pass.
template <typename T, int VPL>
__device__ __forceinline__ void kill_label(u32x4 (&v)[VPL], int kx, int ex) {
  if (kx < 0) return;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
    if (k == kx) T::kill(v[k], ex);
}

// pass 1: sum of 2^{x log2 e - mc} over the lane's elements (the label
// already set to -inf by kill_label; or, with kx >= 0, its term zeroed here:
// the persistent wide-row and slab-statistics kernels keep the staged data
// untouched, where the register kill cost them 20-30 VGPRs and spills).
template <typename T, int NT, int VPL, int K0 = 0, int K1 = VPL>
__device__ __forceinline__ float pass1_16(const u32x4 (&v)[VPL], int nvec, int tid, float mc, float xh, float xt,
                                         int kx = -1, int ex = 0) {
  float s0 = __builtin_amdgcn_exp2f(__builtin_fmaf(xh, kLog2e, -mc));
  float s1 = __builtin_amdgcn_exp2f(__builtin_fmaf(xt, kLog2e, -mc));
#pragma unroll
  for (int k = K0; k < K1; ++k) {
    if (k * NT + tid < nvec) {
      float t[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t u = v[k][d];
        t[2 * d] = __builtin_amdgcn_exp2f(__builtin_fmaf(T::lo(u), kLog2e, -mc));
        t[2 * d + 1] = __builtin_amdgcn_exp2f(__builtin_fmaf(T::hi(u), kLog2e, -mc));
      }
      if (k == kx) {
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = (e == ex) ? 0.0f : t[e];
      }
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        s0 += t[2 * d];
        s1 += t[2 * d + 1];
      }
    }
  }
  return s0 + s1;
}

// One gradient element of a 16-bit row: with u = (x - lse) log2e <= 0 and
// s = dloss / n_valid, g = 2^u s.  MODE selects the arithmetic:
//   kFold    g = 2^(x log2e - b),  b = lse log2e - log2 s      (s > 0)
//   kScaled  g = 2^(x log2e - (lse log2e - c)) * (s 2^-c),  c = ilogb(s) + 9
//   kMul     g = 2^(x log2e - lse log2e) * s                   (other s)
// v_exp_f32 flushes results below 2^-126 to zero, while bf16 keeps
// subnormals down to 2^-133.  In kScaled the factor s 2^-c lies in
// [2^-9, 2^-8), so every output that rounds to a nonzero 16-bit value has
// its power of two at or above 2^-126 (and at most 2^127 for |s| < 2^118):
// the flush never decides a result and the product rounds once more to fp32
// (a subnormal fp32 product is kept; the final 16-bit rounding then differs
// from a single rounding by at most one unit of the last place).
enum { kFold = 0, kMul = 1, kScaled = 2 };
constexpr float kScaledMax = 0x1p118f;  // |s| range served by kScaled
struct GradConsts {
  float b;      // kFold exponent offset
  float lc;     // lse log2e (kMul)
  float lcs;    // lse log2e - c (kScaled)
  float scale;  // s (kMul)
  float ss;     // s 2^-c (kScaled)
  float gy;     // the label element's gradient, -s (1 - p_y)
};
template <int MODE>
__device__ __forceinline__ float gelem(float x, const GradConsts& k) {
  if constexpr (MODE == kFold) return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -k.b));
  else if constexpr (MODE == kMul) return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -k.lc)) * k.scale;
  else return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -k.lcs)) * k.ss;
}

// A row's 16-byte-aligned body to load: its first vector and vector count.
struct Prefetch {
  const u32x4* body;  // NULL: nothing to load
  int nvec;
};

// pass 2: gradient of the staged vectors, stored to gbody (the label element
// is written afterwards by grad_row_16).
template <typename T, int NT, int VPL, int POL, int MODE>
__device__ __forceinline__ void pass2_16(const u32x4 (&v)[VPL], int nvec, int tid, u32x4* gbody, const GradConsts& kc) {
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int idx = k * NT + tid;
    if (idx < nvec) {
      float gv[8];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        gv[2 * d] = gelem<MODE>(T::lo(v[k][d]), kc);
        gv[2 * d + 1] = gelem<MODE>(T::hi(v[k][d]), kc);
      }
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) o[d] = T::pack(gv[2 * d], gv[2 * d + 1]);
      stv<POL>(gbody + idx, o);
    }
    // one vector's arithmetic and store at a time: left to itself the
    // scheduler interleaves vectors and holds more values live (this shape
    // is tuned with the barrier in place)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Issues the loads of a row's body into v.
template <int NT, int VPL, int POL>
__device__ __forceinline__ void load_body(u32x4 (&v)[VPL], const Prefetch& pf, int tid) {
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int idx = k * NT + tid;
    if (pf.body && idx < pf.nvec) v[k] = ldv<POL>(pf.body + idx);
  }
}

// Head / tail elements of a 16-bit row (one per lane at most).
template <typename T, int MODE>
__device__ __forceinline__ float gscalar(float x, bool is_label, const GradConsts& kc) {
  return is_label ? kc.gy : gelem<MODE>(x, kc);
}

// Picks the pass-2 arithmetic for a row.  tmin: a lower bound of
// min_j (x_j - lse) log2e over the row (only used for bf16).  kFold computes
// 2^t with t = u + log2 s, flushed below 2^-126, which matters only for bf16
// (its subnormals reach 2^-133); kMul's 2^u is flushed below 2^-126, which
// matters once |s| exceeds T::kSlowScale.  Those rows take kScaled.  (Scales
// of 2^118 and beyond, which no loss gradient reaches, keep kFold / kMul.)
template <typename T>
__device__ __forceinline__ int grad_mode(float scale, float tmin) {
  const float as = fabsf(scale);
  const bool scalable = as > 0.0f && as < kScaledMax;  // false for NaN
  if (scale > 0.0f && scale <= 3.0e38f) {
    if (T::kBF && scalable && tmin + log2f(scale) < -125.0f) return kScaled;
    return kFold;
  }
  if (scalable && as > T::kSlowScale && (!T::kBF || tmin < -125.0f)) return kScaled;
  return kMul;
}

template <typename T>
__device__ __forceinline__ GradConsts grad_consts(float lse, float scale, double scale_d, double pcomp) {
  GradConsts k;
  k.lc = lse * kLog2e;
  k.b = k.lc - log2f(scale);  // used only when scale > 0
  const float as = fabsf(scale);
  const int c = (as > 0.0f && as < kScaledMax) ? ilogbf(scale) + 9 : 0;
  k.lcs = k.lc - (float)c;
  k.ss = ldexpf(scale, -c);
  k.scale = scale;
  k.gy = (float)(-scale_d * pcomp);
  return k;
}

// Writes NaN over a row whose label is out of range.
template <typename T, int NT, int VPL, int POL>
__device__ __forceinline__ void nan_row(char* gbase, const Geom& g, int tid, int v0) {
  u32x4* gbody = (u32x4*)(gbase + g.head * T::ESZ);
  const uint32_t q = (T::ESZ == 2) ? 0x7fc07fc0u : 0x7fc00000u;
  const u32x4 z = {q, q, q, q};
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int idx = v0 + k * NT + tid;
    if (idx < g.nvec) stv<POL>(gbody + idx, z);
  }
  if (v0 == 0) {
    typedef typename T::bits_t B;
    if (tid < g.head) ((B*)gbase)[tid] = (B)q;
    if (tid < g.tail) ((B*)gbase)[g.head + (int64_t)g.nvec * T::EPV + tid] = (B)q;
  }
}

// Whole pass 2 of a 16-bit row (or slab): nvec staged body vectors written
// to gbody, plus this lane's head element (to *ph) and tail element (to *pt)
// when it has them.
template <typename T, int NT, int VPL, int POL>
__device__ __forceinline__ void grad_row_16(u32x4 (&v)[VPL], int nvec, int tid, u32x4* gbody, int mode,
                                            const GradConsts& kc, const Owner& own, float xh, float xt,
                                            typename T::bits_t* ph, typename T::bits_t* pt) {
  float gh = 0.0f, gt = 0.0f;
  if (mode == kFold) {
    pass2_16<T, NT, VPL, POL, kFold>(v, nvec, tid, gbody, kc);
    gh = gscalar<T, kFold>(xh, own.head > 0, kc);
    gt = gscalar<T, kFold>(xt, own.tail > 0, kc);
  } else if (mode == kMul) {
    pass2_16<T, NT, VPL, POL, kMul>(v, nvec, tid, gbody, kc);
    gh = gscalar<T, kMul>(xh, own.head > 0, kc);
    gt = gscalar<T, kMul>(xt, own.tail > 0, kc);
  } else {
    pass2_16<T, NT, VPL, POL, kScaled>(v, nvec, tid, gbody, kc);
    gh = gscalar<T, kScaled>(xh, own.head > 0, kc);
    gt = gscalar<T, kScaled>(xt, own.tail > 0, kc);
  }
  if (ph) *ph = T::store1(gh);
  if (pt) *pt = T::store1(gt);
  // the label element: after the vector store that covered it (same lane,
  // same address, program order)
  if (own.k >= 0) ((typename T::bits_t*)gbody)[(int64_t)(own.k * NT + tid) * T::EPV + own.e] = T::store1(kc.gy);
}

// Lane minimum of 16-bit staged vectors (bf16 only; a lower bound within one
// bf16 ulp, as in pass 0).
template <typename T, int NT, int VPL>
__device__ __forceinline__ float lane_min_16(const u32x4 (&v)[VPL], int nvec, int tid, float mn) {
#pragma unroll
  for (int k = 0; k < VPL; ++k)
    if (k * NT + tid < nvec)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t u = v[k][d];
        mn = fminf(mn, fminf(__builtin_bit_cast(float, u), __builtin_bit_cast(float, u << 16)));
      }
  return mn;
}

// grad_mode for a workgroup whose lanes each know only their own minimum:
// kScaled is agreed with one barrier (bf16 only).
template <typename T>
__device__ __forceinline__ int block_grad_mode(float scale, float tmin_lane) {
  const float as = fabsf(scale);
  const bool pos = scale > 0.0f && scale <= 3.0e38f;
  const bool scalable = as > 0.0f && as < kScaledMax;
  if constexpr (T::kBF) {
    const bool lane = pos ? (tmin_lane + log2f(scale) < -125.0f) : (as > T::kSlowScale && tmin_lane < -125.0f);
    const int any = __syncthreads_or(lane ? 1 : 0);
    if (scalable && any) return kScaled;
    return pos ? kFold : kMul;
  } else {
    if (pos) return kFold;
    return (scalable && as > T::kSlowScale) ? kScaled : kMul;
  }
}

// Writes +0 over the row's elements (ignored rows are not read).
template <typename T, int NT, int VPL, int POL>
__device__ __forceinline__ void zero_row(char* gbase, const Geom& g, int tid, int v0) {
  u32x4* gbody = (u32x4*)(gbase + g.head * T::ESZ);
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int idx = v0 + k * NT + tid;
    if (idx < g.nvec) stv<POL>(gbody + idx, z);
  }
  if (v0 == 0) {
    typedef typename T::bits_t B;
    if (tid < g.head) ((B*)gbase)[tid] = 0;
    if (tid < g.tail) ((B*)gbase)[g.head + (int64_t)g.nvec * T::EPV + tid] = 0;
  }
}

// ---------------------------------------------------------------------------
// Whole-row kernel for 16-bit formats (bf16, fp16).
//   FUSED: forward + gradient written over the row.   !FUSED: forward only.
// One workgroup of NT lanes per row; row capacity NT * VPL vectors.  (A
// persistent variant that loops over rows measured no faster at these row
// sizes: the hardware refills a finished workgroup's slot within ~2 us.)
// ---------------------------------------------------------------------------
// Waves per SIMD the register budget must allow: 8 for 512- and 1024-lane
// shapes of at most 8 vectors per lane (64 VGPRs: four 512-lane rows per
// CU), 4 otherwise (128 VGPRs).  Without a bound the compiler may take up to
// 256 VGPRs for a 512-lane shape and fit one row per CU.
template <int NT, int VPL>
constexpr int row_min_waves() { return (NT >= 512 && VPL <= 8) ? 8 : 4; }

// The statistics pass holds no gradient state: 64 VGPRs for up to 8 vectors
// per lane.  (With a 128-VGPR budget the scheduler has been seen to build up
// more than 128 live values in the 256 x 8 shape and spill.)
template <int VPL>
constexpr int stats_min_waves() { return VPL <= 8 ? 8 : 4; }

template <typename T, int NT, int VPL, int POL, bool FUSED>
__global__ __launch_bounds__(NT, (row_min_waves<NT, VPL>())) void row_kernel_16(Args a) {
  constexpr int ESZ = T::ESZ, EPV = T::EPV, NW = NT / 64;
  typedef typename T::bits_t B;
  __shared__ float lds_m[NW], lds_s[NW], lds_mn[NW];
  __shared__ uint32_t lds_u[2 * NW + 4];
  __shared__ double lds_d[NT];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;

  const uint32_t epoch = ld_agent(&a.ws->epoch);  // unchanged until the finisher's last store
  const uint32_t tag = epoch + 1u;
  if (row < a.K) count_and_publish<NT>(a, (int)row, tag, lds_u + 4);

  char* rbase = a.logits + row * a.ld * ESZ;
  const int64_t y = a.labels[row];
  const bool ignored = (y == a.ignore);
  const bool badlab = !ignored && (y < 0 || y >= a.V);
  const Geom g = geom<ESZ, EPV>(rbase, a.V);

  // ---- issue every load of the row -------------------------------------
  u32x4 v[VPL];
  float xh = -INFINITY, xt = -INFINITY;  // this lane's head / tail element
  const bool has_h = tid < g.head, has_t = tid < g.tail;
  if (!ignored) {
    load_body<NT, VPL, POL>(v, Prefetch{(const u32x4*)(rbase + g.head * ESZ), g.nvec}, tid);
    if (has_h) xh = T::load1(((const B*)rbase)[tid]);
    if (has_t) xt = T::load1(((const B*)rbase)[g.head + (int64_t)g.nvec * EPV + tid]);
  }
  const float xy = (!ignored && !badlab) ? T::load1(((const B*)rbase)[y]) : 0.0f;
  poll_to_lds(a, tag, lds_u);

  float lse = 0.0f, loss = 0.0f, pcomp = 0.0f;
  if (!ignored) {
    float m = fmaxf(xh, xt);
    float mn = INFINITY;
    if (has_h) mn = xh;
    if (has_t) mn = fminf(mn, xt);
    pass0_16<T, NT, VPL, 0, VPL, FUSED>(v, g.nvec, tid, m, mn);  // the min serves only the gradient
    const Owner own = owner<NT, EPV>(g, badlab ? -1 : y, tid);
    // the label element is left out of the sum: -inf in the registers of the
    // lane that holds it (kill_label), or in the head / tail element
    const float xh1 = (own.head > 0) ? -INFINITY : xh, xt1 = (own.tail > 0) ? -INFINITY : xt;
    const float mc = (m == -INFINITY) ? 0.0f : m * kLog2e;
    kill_label<T, VPL>(v, own.k, own.e);
    const float s = pass1_16<T, NT, VPL>(v, g.nvec, tid, mc, xh1, xt1);
    float M, S_ex, MN;
    row_stats<NW>(m, s, mn, lds_m, lds_s, lds_mn, M, S_ex, MN);
    if (badlab) {
      lse = loss = pcomp = __builtin_nanf("");
    } else {
      const float ey = __builtin_amdgcn_exp2f((xy - M) * kLog2e);
      const float S = S_ex + ey;
      lse = M + logf(S);
      pcomp = S_ex / S;
      loss = (pcomp >= 0.5f) ? (lse - xy) : log1pf(S_ex / ey);
    }
    if constexpr (FUSED) {
      char* gbase = a.grad + row * a.grad_ld * ESZ;
      if (badlab) {
        nan_row<T, NT, VPL, POL>(gbase, g, tid, 0);
      } else {
        const double scale_d = call_scale(a, lds_u);
        const float scale = (float)scale_d;
        const GradConsts kc = grad_consts<T>(lse, scale, scale_d, (double)pcomp);
        // lower bound of (x - lse) log2e over the row (the lane minima are
        // exact; the 2^-7 relative widening is a margin)
        const float tmin = (MN - fabsf(MN) * 0x1p-7f - lse) * kLog2e;
        const int64_t jt = g.head + (int64_t)g.nvec * EPV + tid;
        grad_row_16<T, NT, VPL, POL>(v, g.nvec, tid, (u32x4*)(gbase + g.head * ESZ), grad_mode<T>(scale, tmin), kc,
                                     own, xh, xt, has_h ? (B*)gbase + tid : nullptr,
                                     has_t ? (B*)gbase + jt : nullptr);
      }
    }
  } else {
    if constexpr (FUSED) zero_row<T, NT, VPL, POL>(a.grad + row * a.grad_ld * ESZ, g, tid, 0);
  }
  if (tid == 0) {
    a.loss_rows[row] = loss;
    if (a.lse_rows) a.lse_rows[row] = (double)lse;
    if (a.pcomp_rows) a.pcomp_rows[row] = (double)pcomp;
    publish_loss(a, row, loss, tag);
  }
  if (blockIdx.x == gridDim.x - 1) {
    __syncthreads();
    finish_call<NT>(a, epoch, lds_u, lds_d);
  }
}

// ---------------------------------------------------------------------------
// Fused kernel for 16-byte-aligned 16-bit rows (vocab a multiple of 8 and a
// 16-byte row stride), persistent, with buffer loads and stores.
//
// A buffer resource per row (SGPRs: base, byte size) lets every access use
// one per-lane VGPR offset (lane * 16) plus a per-vector SGPR offset, so no
// per-vector 64-bit addresses are held in VGPRs.  The descriptor's size also
// bounds every access: loads past the row return 0 and stores past it are
// dropped, so only the reductions of pass 0 / pass 1 need lane predicates.
// ---------------------------------------------------------------------------
// row_rsrc, aux_load / aux_store and buf_store: ce_buffer.h

template <int NT, int VPL, int POL>
__device__ __forceinline__ void buf_load_row(u32x4 (&v)[VPL], __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
#pragma unroll
  for (int k = 0; k < VPL; ++k)
    v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k * NT * 16, aux_load<POL>()));
}
template <int NT, int VPL, int POL>
__device__ __forceinline__ void buf_fill_row(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t word) {
  const u32x4 z = {word, word, word, word};
#pragma unroll
  for (int k = 0; k < VPL; ++k) buf_store<aux_store<POL>()>(z, rs, voff, k * NT * 16);
}

// pass 2 on buffer stores.  Lanes past the row compute garbage that their
// dropped stores discard.
template <typename T, int NT, int VPL, int POL, int MODE>
__device__ __forceinline__ void pass2_buf(const u32x4 (&v)[VPL], __amdgpu_buffer_rsrc_t out, uint32_t voff,
                                          const GradConsts& kc, int kx, int ex) {
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    float gv[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      gv[2 * d] = gelem<MODE>(T::lo(v[k][d]), kc);
      gv[2 * d + 1] = gelem<MODE>(T::hi(v[k][d]), kc);
    }
    if (k == kx) {
#pragma unroll
      for (int e = 0; e < 8; ++e) gv[e] = (e == ex) ? kc.gy : gv[e];
    }
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = T::pack(gv[2 * d], gv[2 * d + 1]);
    buf_store<aux_store<POL>()>(o, out, voff, k * NT * 16);
  }
}

//
// KB > 0: the vocabulary is taken as two chunks, vector slots [0, KB) and
// [KB, VPL) of every lane (chunk width KB * NT * 8 elements): each chunk's
// (max, label-excluded sum) is reduced over the workgroup on its own and the
// two are merged, the per-chunk log-sum-exp merge of a chunked loss done
// on chip with no second read of the row.
template <typename T, int NT, int VPL, int POL, int KB = 0>
__global__ __launch_bounds__(NT, 4) void row_fused_aligned(Args a) {
  constexpr int ESZ = T::ESZ, EPV = T::EPV, NW = NT / 64;
  __shared__ float lds_m[2][NW], lds_s[2][NW], lds_mn[2][NW];
  __shared__ uint32_t lds_u[2 * NW + 4];
  __shared__ double lds_d[NT];
  const int tid = threadIdx.x;
  const int64_t G = gridDim.x;
  const int nvec = (int)(a.V / EPV);
  const uint32_t rbytes = (uint32_t)nvec * 16u;
  const uint32_t voff = (uint32_t)tid * 16u;

  const uint32_t epoch = ld_agent(&a.ws->epoch);
  const uint32_t tag = epoch + 1u;
  if ((int)blockIdx.x < a.K) count_and_publish<NT>(a, (int)blockIdx.x, tag, lds_u + 4);

  poll_to_lds(a, tag, lds_u);
  int par = 0;
  for (int64_t row = blockIdx.x; row < a.N; row += G) {
    char* base = a.logits + row * a.ld * ESZ;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(base, rbytes);
    const int64_t y = a.labels[row];
    const bool ignored = (y == a.ignore);
    const bool bad = !ignored && (y < 0 || y >= a.V);
    u32x4 v[VPL];
    if (!ignored) buf_load_row<NT, VPL, POL>(v, rs, voff);

    float lse = 0.0f, loss = 0.0f, pcomp = 0.0f;
    if (!ignored) {
      const float xy = bad ? 0.0f : T::load1(((const typename T::bits_t*)base)[y]);
      int kx = -1, ex = 0;
      if (!bad) {
        const int vy = (int)(y / EPV);
        if (tid == vy % NT) {
          kx = vy / NT;
          ex = (int)(y % EPV);
        }
      }
      float M, S_ex, MN;
      float m = -INFINITY, mn = INFINITY;
      if constexpr (KB == 0) {
        pass0_16<T, NT, VPL>(v, nvec, tid, m, mn);
        const float mc = (m == -INFINITY) ? 0.0f : m * kLog2e;
        const float s = pass1_16<T, NT, VPL>(v, nvec, tid, mc, -INFINITY, -INFINITY, kx, ex);
        row_stats<NW>(m, s, mn, lds_m[par], lds_s[par], lds_mn[par], M, S_ex, MN);
        par ^= 1;
      } else {
        // chunk by chunk (each its own max), then the two (max, sum) merged;
        // the two reductions take both LDS slots, so par is left as it is
        float m1 = -INFINITY, mn1 = INFINITY;
        pass0_16<T, NT, VPL, 0, KB>(v, nvec, tid, m, mn);
        pass0_16<T, NT, VPL, KB, VPL>(v, nvec, tid, m1, mn1);
        const float mc0 = (m == -INFINITY) ? 0.0f : m * kLog2e, mc1 = (m1 == -INFINITY) ? 0.0f : m1 * kLog2e;
        const float s0 = pass1_16<T, NT, VPL, 0, KB>(v, nvec, tid, mc0, -INFINITY, -INFINITY, kx, ex);
        const float s1 = pass1_16<T, NT, VPL, KB, VPL>(v, nvec, tid, mc1, -INFINITY, -INFINITY, kx, ex);
        float M0, S0, MN0, M1, S1, MN1;
        row_stats<NW>(m, s0, mn, lds_m[par], lds_s[par], lds_mn[par], M0, S0, MN0);
        row_stats<NW>(m1, s1, mn1, lds_m[par ^ 1], lds_s[par ^ 1], lds_mn[par ^ 1], M1, S1, MN1);
        M = fmaxf(M0, M1);
        S_ex = ((M0 == -INFINITY) ? 0.0f : S0 * __builtin_amdgcn_exp2f((M0 - M) * kLog2e)) +
               ((M1 == -INFINITY) ? 0.0f : S1 * __builtin_amdgcn_exp2f((M1 - M) * kLog2e));
        MN = fminf(MN0, MN1);
      }
      if (bad) {
        lse = loss = pcomp = __builtin_nanf("");
        buf_fill_row<NT, VPL, POL>(rs, voff, (T::ESZ == 2) ? 0x7fc07fc0u : 0x7fc00000u);
      } else {
        const float ey = __builtin_amdgcn_exp2f((xy - M) * kLog2e);
        const float S = S_ex + ey;
        lse = M + logf(S);
        pcomp = S_ex / S;
        loss = (pcomp >= 0.5f) ? (lse - xy) : log1pf(S_ex / ey);
        const double scale_d = call_scale(a, lds_u);
        const float scale = (float)scale_d;
        const GradConsts kc = grad_consts<T>(lse, scale, scale_d, (double)pcomp);
        const float tmin = (MN - fabsf(MN) * 0x1p-7f - lse) * kLog2e;
        const int mode = grad_mode<T>(scale, tmin);
        if (mode == kFold) pass2_buf<T, NT, VPL, POL, kFold>(v, rs, voff, kc, kx, ex);
        else if (mode == kScaled) pass2_buf<T, NT, VPL, POL, kScaled>(v, rs, voff, kc, kx, ex);
        else pass2_buf<T, NT, VPL, POL, kMul>(v, rs, voff, kc, kx, ex);
      }
    } else {
      buf_fill_row<NT, VPL, POL>(rs, voff, 0u);
    }
    if (tid == 0) {
      a.loss_rows[row] = loss;
      if (a.lse_rows) a.lse_rows[row] = (double)lse;
      if (a.pcomp_rows) a.pcomp_rows[row] = (double)pcomp;
      publish_loss(a, row, loss, tag);
    }
  }
  if (blockIdx.x == G - 1) {
    __syncthreads();
    finish_call<NT>(a, epoch, lds_u, lds_d);
  }
}

// ---------------------------------------------------------------------------
// Whole-row kernel for fp32 inputs: the same steps in fp64, rounded once.
// ---------------------------------------------------------------------------
template <int NT, int VPL, int POL, bool FUSED>
__global__ __launch_bounds__(NT) void row_kernel_32(Args a) {
  constexpr int ESZ = 4, EPV = 4, NW = NT / 64;
  __shared__ float lds_m[NW];
  __shared__ double lds_s[NW];
  __shared__ uint32_t lds_u[2 * NW + 4];
  __shared__ double lds_d[NT];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint32_t epoch = ld_agent(&a.ws->epoch);
  const uint32_t tag = epoch + 1u;
  if (row < a.K) count_and_publish<NT>(a, (int)row, tag, lds_u + 4);

  char* rbase = a.logits + row * a.ld * ESZ;
  const int64_t y = a.labels[row];
  const bool ignored = (y == a.ignore);
  const bool badlab = !ignored && (y < 0 || y >= a.V);
  const Geom g = geom<ESZ, EPV>(rbase, a.V);
  const u32x4* body = (const u32x4*)(rbase + g.head * ESZ);
  u32x4 v[VPL];
  float xh = -INFINITY, xt = -INFINITY;
  const bool has_h = tid < g.head, has_t = tid < g.tail;
  if (!ignored) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int idx = k * NT + tid;
      if (idx < g.nvec) v[k] = ldv<POL>(body + idx);
    }
    if (has_h) xh = ((const float*)rbase)[tid];
    if (has_t) xt = ((const float*)rbase)[g.head + (int64_t)g.nvec * EPV + tid];
  }
  const double xy = (!ignored && !badlab) ? (double)((const float*)rbase)[y] : 0.0;
  poll_to_lds(a, tag, lds_u);

  double lse = 0.0, loss = 0.0, pcomp = 0.0;
  if (!ignored) {
    float mf = fmaxf(xh, xt);
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (k * NT + tid < g.nvec)
#pragma unroll
        for (int d = 0; d < 4; ++d) mf = fmaxf(mf, as<float>(v[k][d]));
    const Owner own = owner<NT, EPV>(g, badlab ? -1 : y, tid);
    if (own.head > 0) xh = -INFINITY;
    if (own.tail > 0) xt = -INFINITY;
    if (own.k >= 0) {
#pragma unroll
      for (int k = 0; k < VPL; ++k)
        if (k == own.k) F32::kill(v[k], own.e);
    }
    const double mm = (mf == -INFINITY) ? 0.0 : (double)mf;
    double s4[4] = {exp_f64((double)xh - mm), exp_f64((double)xt - mm), 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (k * NT + tid < g.nvec)
#pragma unroll
        for (int d = 0; d < 4; ++d) s4[d] += exp_f64((double)as<float>(v[k][d]) - mm);
    float Mf;
    double S_ex;
    block_ms<NW>(mf, (s4[0] + s4[1]) + (s4[2] + s4[3]), lds_m, lds_s, Mf, S_ex);
    const double M = (double)Mf;
    if (badlab) {
      lse = loss = pcomp = __builtin_nan("");
    } else {
      const double ey = exp(xy - M);
      const double S = S_ex + ey;
      lse = M + log(S);
      pcomp = S_ex / S;
      loss = (pcomp >= 0.5) ? (lse - xy) : log1p(S_ex / ey);
    }
    if constexpr (FUSED) {
      const double scale = call_scale(a, lds_u);
      char* gbase = a.grad + row * a.grad_ld * ESZ;
      u32x4* gbody = (u32x4*)(gbase + g.head * ESZ);
      if (badlab) {
        nan_row<F32, NT, VPL, POL>(gbase, g, tid, 0);
      } else {
#pragma unroll
        for (int k = 0; k < VPL; ++k) {
          const int idx = k * NT + tid;
          if (idx < g.nvec) {
            u32x4 o;
#pragma unroll
            for (int d = 0; d < 4; ++d)
              o[d] = __builtin_bit_cast(uint32_t, (float)(exp_f64((double)as<float>(v[k][d]) - lse) * scale));
            stv<POL>(gbody + idx, o);
          }
        }
        float* grow = (float*)gbase;
        const int64_t jt = g.head + (int64_t)g.nvec * EPV + tid;
        if (has_h) grow[tid] = (float)(exp_f64((double)xh - lse) * scale);
        if (has_t) grow[jt] = (float)(exp_f64((double)xt - lse) * scale);
        // the label's gradient overwrites the value just stored for it (same
        // lane, same address: program order)
        const float gy = (float)(-scale * pcomp);
        if (own.k >= 0) ((float*)gbody)[(int64_t)(own.k * NT + tid) * EPV + own.e] = gy;
        if (own.head > 0) grow[tid] = gy;
        if (own.tail > 0) grow[jt] = gy;
      }
    }
  } else {
    if constexpr (FUSED) zero_row<F32, NT, VPL, POL>(a.grad + row * a.grad_ld * ESZ, g, tid, 0);
  }
  if (tid == 0) {
    a.loss_rows[row] = (float)loss;
    if (a.lse_rows) a.lse_rows[row] = lse;
    if (a.pcomp_rows) a.pcomp_rows[row] = pcomp;
    publish_loss(a, row, (float)loss, tag);
  }
  if (blockIdx.x == gridDim.x - 1) {
    __syncthreads();
    finish_call<NT>(a, epoch, lds_u, lds_d);
  }
}

// ---------------------------------------------------------------------------
// Backward from saved statistics, elementwise:
//   grad_j = s 2^{(x_j - lse) log2 e} (j != y),  grad_y = -s pcomp,  s = dloss/n.
// blockIdx.x = row * C + slab, a slab being NT*VPL vectors of the row.  16-bit
// rows take fp64 exponentials only when |s| is large enough for a flushed
// 2^t to change a rounded output; fp32 rows always compute in fp64.
//
// The vectors are those of the gradient row (its 16-byte-aligned body, with
// head and tail elements before and after it), so every store is a whole
// aligned vector.  When the logits row has another 16-byte phase than the
// gradient row (an out-of-place gradient buffer laid out differently), the
// input of each vector is assembled from the two aligned 16-byte blocks it
// straddles: both hold at least one byte of the row, and an aligned 16-byte
// block never crosses a page, so neither load can leave mapped memory; the
// bytes outside the row are discarded.
// ---------------------------------------------------------------------------
// 16 bytes starting r bytes (r in 1..15, even) past the aligned block p.
template <int POL>
__device__ __forceinline__ u32x4 ld_shifted(const u32x4* p, uint32_t r) {
  const u32x4 lo = ldv<POL>(p), hi = ldv<POL>(p + 1);
  const uint32_t w = r >> 2, b = r & 3u;
  const uint32_t c[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  uint32_t t[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const uint32_t c0 = c[i], c1 = c[i + 1], c2 = c[i + 2], c3 = (i + 3 < 8) ? c[i + 3] : 0u;
    t[i] = (w == 0) ? c0 : (w == 1) ? c1 : (w == 2) ? c2 : c3;
  }
  u32x4 o;
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = __builtin_amdgcn_alignbyte(t[d + 1], t[d], b);
  return o;
}

template <int NT, int VPL, int POL>
__device__ __forceinline__ void load_slab(u32x4 (&v)[VPL], const char* in, int nvec, int v0, int tid) {
  const uint32_t r = (uint32_t)((uintptr_t)in & 15u);
  if (r == 0) {
    const u32x4* body = (const u32x4*)in;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int idx = v0 + k * NT + tid;
      if (idx < nvec) v[k] = ldv<POL>(body + idx);
    }
  } else {
    const u32x4* blk = (const u32x4*)(in - r);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int idx = v0 + k * NT + tid;
      if (idx < nvec) v[k] = ld_shifted<POL>(blk + idx, r);
    }
  }
}

template <typename T, int NT, int VPL, int POL>
__global__ __launch_bounds__(NT) void grad_kernel(Args a) {
  constexpr int ESZ = T::ESZ, EPV = T::EPV;
  typedef typename T::bits_t B;
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x / a.C;
  const int slab = (int)(blockIdx.x % a.C);
  const int v0 = slab * NT * VPL;
  const char* rbase = a.logits + row * a.ld * ESZ;
  char* gbase = a.grad + row * a.grad_ld * ESZ;
  const Geom g = geom<ESZ, EPV>(gbase, a.V);  // the gradient row's vectors
  u32x4* gbody = (u32x4*)(gbase + g.head * ESZ);
  const int64_t y = a.labels[row];
  if (y == a.ignore) {
    zero_row<T, NT, VPL, POL>(gbase, g, tid, v0);
    return;
  }
  const bool badlab = (y < 0 || y >= a.V);
  if (badlab) {
    nan_row<T, NT, VPL, POL>(gbase, g, tid, v0);
    return;
  }
  const double lse_d = a.lse_in[row];
  const double scale_d = (a.dloss ? (double)a.dloss[0] : 1.0) / (double)a.n_valid_in[0];
  const double gy_d = -scale_d * a.pcomp_in[row];
  u32x4 v[VPL];
  load_slab<NT, VPL, POL>(v, rbase + g.head * ESZ, g.nvec, v0, tid);
  if constexpr (ESZ == 2) {
    const bool hh = slab == 0 && tid < g.head, ht = slab == 0 && tid < g.tail;
    const int64_t jt = g.head + (int64_t)g.nvec * EPV + tid;
    const float xh = hh ? T::load1(((const B*)rbase)[tid]) : 0.0f;
    const float xt = ht ? T::load1(((const B*)rbase)[jt]) : 0.0f;
    const float scale = (float)scale_d, lse = (float)lse_d;
    float tmin = INFINITY;
    if constexpr (T::kBF) {
      float mn = lane_min_16<T, NT, VPL>(v, g.nvec - v0, tid, INFINITY);
      if (hh) mn = fminf(mn, xh);
      if (ht) mn = fminf(mn, xt);
      tmin = (mn - fabsf(mn) * 0x1p-7f - lse) * kLog2e;
    }
    const int mode = block_grad_mode<T>(scale, tmin);
    const GradConsts kc = grad_consts<T>(lse, scale, scale_d, a.pcomp_in[row]);
    Owner own = owner<NT, EPV>(g, y, tid);
    if (own.k >= 0) own.k -= slab * VPL;  // vector index within this slab
    if (own.k >= VPL) own.k = -1;
    grad_row_16<T, NT, VPL, POL>(v, g.nvec - v0, tid, gbody + v0, mode, kc, own, xh, xt,
                                 hh ? (B*)gbase + tid : nullptr, ht ? (B*)gbase + jt : nullptr);
  } else {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int idx = v0 + k * NT + tid;
      if (idx < g.nvec) {
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d)
          o[d] = __builtin_bit_cast(uint32_t, (float)(exp_f64((double)as<float>(v[k][d]) - lse_d) * scale_d));
        stv<POL>(gbody + idx, o);
      }
    }
    float* grow = (float*)gbase;
    const float* xrow = (const float*)rbase;
    if (slab == 0) {
      if (tid < g.head) grow[tid] = (float)(exp_f64((double)xrow[tid] - lse_d) * scale_d);
      if (tid < g.tail) {
        const int64_t j = g.head + (int64_t)g.nvec * EPV + tid;
        grow[j] = (float)(exp_f64((double)xrow[j] - lse_d) * scale_d);
      }
    }
    // the label's gradient overwrites the value this lane just stored for it
    // (same lane, same address: program order)
    const Owner own = owner<NT, EPV>(g, y, tid);
    const float gy = (float)gy_d;
    if (own.k >= v0 / NT && own.k < v0 / NT + VPL) ((float*)gbody)[(int64_t)(own.k * NT + tid) * EPV + own.e] = gy;
    if (slab == 0 && own.head > 0) grow[tid] = gy;
    if (slab == 0 && own.tail > 0) grow[g.head + (int64_t)g.nvec * EPV + tid] = gy;
  }
}

// ---------------------------------------------------------------------------
// Chunked forward, step 1: per (row, vocabulary slab) max and label-excluded
// sum.  blockIdx.x = row * C + c; slab c covers elements [c*chunk, ...).
// ---------------------------------------------------------------------------
template <typename T, int NT, int VPL, int POL>
__global__ __launch_bounds__(NT, (stats_min_waves<VPL>())) void slab_stats_kernel(Args a) {
  constexpr int ESZ = T::ESZ, EPV = T::EPV, NW = NT / 64;
  typedef typename T::acc_t A;
  typedef typename T::bits_t B;
  __shared__ float lds_m[NW];
  __shared__ A lds_s[NW];
  __shared__ uint32_t lds_u[2 * NW + 4];
  const int tid = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / a.C;
  const int c = (int)(bid % a.C);
  const uint32_t tag = ld_agent(&a.ws->epoch) + 1u;
  if (bid < a.K) count_and_publish<NT>(a, (int)bid, tag, lds_u + 4);
  const int64_t j0 = (int64_t)c * a.chunk;
  const int64_t Vc = (a.V - j0 < a.chunk) ? (a.V - j0) : a.chunk;
  const char* sbase = a.logits + (row * a.ld + j0) * ESZ;
  const int64_t y = a.labels[row];
  const bool ignored = (y == a.ignore);
  const bool badlab = !ignored && (y < 0 || y >= a.V);
  if (ignored || badlab) {
    if (tid == 0) a.slab_ms[bid] = make_double2(badlab ? __builtin_nan("") : -INFINITY, 0.0);
    return;
  }
  const bool mine = y >= j0 && y < j0 + Vc;
  const Geom g = geom<ESZ, EPV>(sbase, Vc);
  const u32x4* body = (const u32x4*)(sbase + g.head * ESZ);
  u32x4 v[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int idx = k * NT + tid;
    if (idx < g.nvec) v[k] = ldv<POL>(body + idx);
  }
  const bool has_h = tid < g.head, has_t = tid < g.tail;
  float xh = -INFINITY, xt = -INFINITY;
  if (has_h) xh = T::load1(((const B*)sbase)[tid]);
  if (has_t) xt = T::load1(((const B*)sbase)[g.head + (int64_t)g.nvec * EPV + tid]);
  if (mine && tid == 0) a.slab_xy[row] = T::load1(((const B*)sbase)[y - j0]);
  const Owner own = owner<NT, EPV>(g, mine ? y - j0 : -1, tid);
  float m;
  A s;
  if constexpr (ESZ == 2) {
    float mf = fmaxf(xh, xt), mn = INFINITY;
    pass0_16<T, NT, VPL>(v, g.nvec, tid, mf, mn);
    if (own.head > 0) xh = -INFINITY;
    if (own.tail > 0) xt = -INFINITY;
    const float mc = (mf == -INFINITY) ? 0.0f : mf * kLog2e;
    s = pass1_16<T, NT, VPL>(v, g.nvec, tid, mc, xh, xt, own.k, own.e);
    m = mf;
  } else {
    float mf = fmaxf(xh, xt);
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (k * NT + tid < g.nvec)
#pragma unroll
        for (int d = 0; d < 4; ++d) mf = fmaxf(mf, as<float>(v[k][d]));
    if (own.head > 0) xh = -INFINITY;
    if (own.tail > 0) xt = -INFINITY;
    const double mm = (mf == -INFINITY) ? 0.0 : (double)mf;
    if (own.k >= 0) {  // the label is left out of the sum
#pragma unroll
      for (int k = 0; k < VPL; ++k)
        if (k == own.k) F32::kill(v[k], own.e);
    }
    double s4[4] = {exp_f64((double)xh - mm), exp_f64((double)xt - mm), 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < VPL; ++k)
      if (k * NT + tid < g.nvec)
#pragma unroll
        for (int d = 0; d < 4; ++d) s4[d] += exp_f64((double)as<float>(v[k][d]) - mm);
    s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
    m = mf;
  }
  float M;
  A S;
  block_ms<NW>(m, s, lds_m, lds_s, M, S);
  if (tid == 0) a.slab_ms[bid] = make_double2((double)M, (double)S);
}

// Merge of the C slab partials of a row (fp64): lse, loss, pcomp.
struct RowStats {
  double lse, loss, pcomp;
  bool bad;
};
__device__ __forceinline__ RowStats merge_slabs(const Args& a, int64_t row) {
  RowStats r;
  double M = -INFINITY, S_ex = 0.0;
  r.bad = false;
  for (int c = 0; c < a.C; ++c) {
    const double2 p = a.slab_ms[row * a.C + c];
    if (p.x != p.x) r.bad = true;
    ms_merge(M, S_ex, p.x, p.y);
  }
  if (r.bad) {
    r.lse = r.loss = r.pcomp = __builtin_nan("");
    return r;
  }
  const double xy = (double)a.slab_xy[row];
  const double ey = exp(xy - M);
  const double S = S_ex + ey;
  r.lse = M + log(S);
  r.pcomp = S_ex / S;
  r.loss = (r.pcomp >= 0.5) ? (r.lse - xy) : log1p(S_ex / ey);
  return r;
}

// ---------------------------------------------------------------------------
// Chunked forward, step 2: per-row merge, row outputs and the mean.
// ---------------------------------------------------------------------------
template <int NT>
__global__ __launch_bounds__(NT) void slab_merge_kernel(Args a) {
  constexpr int NW = NT / 64;
  __shared__ uint32_t lds_u[2 * NW + 4];
  __shared__ double lds_d[NT];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const uint32_t epoch = ld_agent(&a.ws->epoch);
  counts_to_lds(a, lds_u);  // published by the statistics launch
  if (tid == 0) {
    const int64_t y = a.labels[row];
    RowStats r = {0.0, 0.0, 0.0, false};
    if (y != a.ignore) r = merge_slabs(a, row);
    a.loss_rows[row] = (float)r.loss;
    if (a.lse_rows) a.lse_rows[row] = r.lse;
    if (a.pcomp_rows) a.pcomp_rows[row] = r.pcomp;
    publish_loss(a, row, (float)r.loss, epoch + 1u);
  }
  if (blockIdx.x == gridDim.x - 1) {
    __syncthreads();
    finish_call<NT>(a, epoch, lds_u, lds_d);
  }
}

// ---------------------------------------------------------------------------
// Chunked fused path (16-bit formats), step 2: merge the row's slab partials,
// re-read the slab and write its gradient in place; row outputs from slab 0;
// the mean at the end.  blockIdx.x = row * C + c.
// ---------------------------------------------------------------------------
template <typename T, int NT, int VPL, int POL>
__global__ __launch_bounds__(NT, 4) void slab_grad_kernel(Args a) {
  constexpr int ESZ = T::ESZ, EPV = T::EPV, NW = NT / 64;
  typedef typename T::bits_t B;
  __shared__ uint32_t lds_u[2 * NW + 4];
  __shared__ double lds_d[NT];
  __shared__ double lds_r[4];
  const int tid = threadIdx.x;
  const int64_t bid = blockIdx.x;
  const int64_t row = bid / a.C;
  const int c = (int)(bid % a.C);
  const uint32_t epoch = ld_agent(&a.ws->epoch);
  const int64_t j0 = (int64_t)c * a.chunk;
  const int64_t Vc = (a.V - j0 < a.chunk) ? (a.V - j0) : a.chunk;
  char* sbase = a.logits + (row * a.ld + j0) * ESZ;
  const int64_t y = a.labels[row];
  const bool ignored = (y == a.ignore);
  const Geom g = geom<ESZ, EPV>(sbase, Vc);
  u32x4* body = (u32x4*)(sbase + g.head * ESZ);
  u32x4 v[VPL];
  if (!ignored) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int idx = k * NT + tid;
      if (idx < g.nvec) v[k] = ldv<POL>(body + idx);
    }
  }
  // published by the statistics launch; slabs c > 0 publish no loss slot, so
  // the finisher does not wait for them and they must not wait on the epoch
  counts_to_lds(a, lds_u);
  if (tid == 0 && !ignored) {
    const RowStats r = merge_slabs(a, row);
    lds_r[0] = r.lse;
    lds_r[1] = r.loss;
    lds_r[2] = r.pcomp;
    lds_r[3] = r.bad ? 1.0 : 0.0;
  }
  __syncthreads();
  if (ignored) {
    zero_row<T, NT, VPL, POL>(sbase, g, tid, 0);
  } else {
    const bool badlab = lds_r[3] != 0.0;
    if (badlab) {
      nan_row<T, NT, VPL, POL>(sbase, g, tid, 0);
    } else {
      const double scale_d = call_scale(a, lds_u);
      const float scale = (float)scale_d, lse = (float)lds_r[0];
      const bool hh = tid < g.head, ht = tid < g.tail;
      const int64_t jt = g.head + (int64_t)g.nvec * EPV + tid;
      const float xh = hh ? T::load1(((const B*)sbase)[tid]) : 0.0f;
      const float xt = ht ? T::load1(((const B*)sbase)[jt]) : 0.0f;
      float tmin = INFINITY;
      if constexpr (T::kBF) {
        float mn = lane_min_16<T, NT, VPL>(v, g.nvec, tid, INFINITY);
        if (hh) mn = fminf(mn, xh);
        if (ht) mn = fminf(mn, xt);
        tmin = (mn - fabsf(mn) * 0x1p-7f - lse) * kLog2e;
      }
      const int mode = block_grad_mode<T>(scale, tmin);
      const GradConsts kc = grad_consts<T>(lse, scale, scale_d, lds_r[2]);
      const Owner own = owner<NT, EPV>(g, (y >= j0 && y < j0 + Vc) ? y - j0 : -1, tid);
      grad_row_16<T, NT, VPL, POL>(v, g.nvec, tid, body, mode, kc, own, xh, xt, hh ? (B*)sbase + tid : nullptr,
                                   ht ? (B*)sbase + jt : nullptr);
    }
  }
  if (c == 0 && tid == 0) {
    const float loss = ignored ? 0.0f : (float)lds_r[1];
    a.loss_rows[row] = loss;
    if (a.lse_rows) a.lse_rows[row] = ignored ? 0.0 : lds_r[0];
    if (a.pcomp_rows) a.pcomp_rows[row] = ignored ? 0.0 : lds_r[2];
    publish_loss(a, row, loss, epoch + 1u);
  }
  if (blockIdx.x == gridDim.x - 1) {
    __syncthreads();
    finish_call<NT>(a, epoch, lds_u, lds_d);
  }
}

// Writes the outputs of a call with no rows (L = NaN, n_valid = 0).
__global__ void empty_call_kernel(float* loss_mean, int32_t* n_valid, uint32_t* status) {
  if (threadIdx.x == 0) {
    loss_mean[0] = __builtin_nanf("");
    n_valid[0] = 0;
    if (status) status[0] = 0u;
  }
}

// Zero-fills a workspace with plain stores.
__global__ void ws_fill_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

}  // namespace cek
