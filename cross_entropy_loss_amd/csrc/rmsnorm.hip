// rmsnorm.hip -- RMS layer normalisation, forward and backward, for gfx950
// (the C ABI in include/ce_mi355x.h: ce_rmsnorm_workspace_bytes,
// ce_rmsnorm_forward, ce_rmsnorm_backward).
//
// The pages list "Fast RMS LayerNorm" among the package's kernels (PyPI page
// "fms-acceleration-foak 0.7.4", kernel list) and patch it in for a model's
// RMSNorm class (same page, the model-patcher rule that replaces
// GraniteRMSNorm's forward; fms-hf-tuning PR #280, "Notes on FastKernels").
// Per row x[0..H) with weight w:
//   rstd = 1 / sqrt(mean x^2 + eps),  y = w x rstd
//   dx = rstd (w dy - x^ mean(x^ w dy)),  dw = sum over rows of dy x^,
// with x^ = x rstd.  16-bit formats compute in fp32 and round once; fp32
// computes y and dx in fp64 (dw accumulates in fp32 over a workgroup's rows
// and in fp64 across workgroups).
//
// Shape of the work.  HBM-bound rows of a few KB (Mistral-7B: H = 4096 bf16,
// 8 KB): one wave per row, the row in VGPRs (VPL 16-byte vectors per lane),
// sums of squares and dot products reduced with DPP lane moves, no barrier on
// the row path.  Rows are read and written through buffer resources (one per
// row, in SGPRs): loads past the row return 0 and stores past it are dropped,
// so the row path has no per-vector branches (a branch per vector made the
// compiler wait for every earlier store before each store).  The backward's
// dw is summed without atomics: each wave keeps per-lane fp32 sums over the
// rows it handles, the workgroup's waves are added in a fixed order through
// LDS, and a second launch adds the workgroups' partials in a fixed order
// (deterministic).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ce_buffer.h"
#include "ce_mi355x.h"
#include "row_formats.h"

namespace {

using cek::buf_store;
using cek::row_rsrc;
using cek::u32x4;
using rowfmt::as_f;
using rowfmt::BF16;
using rowfmt::F16;

constexpr int kWaves = 4;          // forward: waves (rows in flight) per workgroup
#ifndef RMS_BWD_WAVES
#define RMS_BWD_WAVES 8
#endif
#ifndef RMS_BWD_GROUPS
#define RMS_BWD_GROUPS 256
#endif
constexpr int kBwdWaves = RMS_BWD_WAVES;       // backward: waves per workgroup (one per row in flight)
constexpr int kMaxBwdGroups = RMS_BWD_GROUPS;  // backward workgroups: partial rows of dw
constexpr int kMaxVPL = 32;     // forward: rows up to 32 KB (16384 bf16 / 8192 fp32)
constexpr int kMaxBwdVPL = 8;   // backward: vectors per wave (the per-lane dw sums, 8 VPL floats, stay in
                                // VGPRs); wider rows are split over 2 or 4 waves
constexpr int kNT = 2;          // buffer instruction aux bits: nontemporal (streamed rows)

// Waves per SIMD the register budget must allow (without a bound the
// compiler has taken up to 256 VGPRs for these shapes, one wave per SIMD).
template <int VPL>
constexpr int fwd_min_waves() { return VPL <= 4 ? 8 : (VPL <= 8 ? 6 : (VPL <= 16 ? 4 : 2)); }
template <int VPL, int R = 1>
constexpr int bwd_min_waves() { return R >= 2 ? 2 : (VPL <= 4 ? 4 : 3); }  // R >= 2: LDS allows 2 per SIMD

// Makes the compiler treat v as redefined here, so that values it derived
// from v earlier (unpacked floats) are recomputed rather than kept live
// across the two passes over the row.
__device__ __forceinline__ void fence_regs(u32x4& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ u32x4 ld_vec(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int k) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, k * 1024, kNT));
}
// A row of `bytes` bytes at p; p is wave-uniform.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const char* p, uint32_t bytes) {
  return row_rsrc(p, bytes);
}
// The weight row into LDS, once per workgroup, zero past its nvec vectors (so
// lanes past the row read a zero weight); ends with a barrier.  LDS reads
// count on their own counter, so reading the weight between a row's stores
// does not make each store wait for the ones before it, as a global load
// there would.
template <int VPL>
__device__ __forceinline__ void stage_weight(const char* w, int nvec, u32x4 (&lw)[VPL * 64]) {
  const u32x4* wr = (const u32x4*)w;
  for (int i = threadIdx.x; i < VPL * 64; i += blockDim.x) lw[i] = i < nvec ? wr[i] : u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
}

// The row index of this wave, in a scalar register.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Wave sum on DPP lane moves (quad_perm, row mirrors, row broadcasts); the
// wave's sum is read from lane 63.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROWS, 0xf,
                                                                   false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = dpp_add<0xb1, 0xf>(v);
  v = dpp_add<0x4e, 0xf>(v);
  v = dpp_add<0x141, 0xf>(v);
  v = dpp_add<0x140, 0xf>(v);
  v = dpp_add<0x142, 0xa>(v);
  v = dpp_add<0x143, 0xc>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// Forward, 16-bit formats: one wave per row.
// ---------------------------------------------------------------------------
template <typename T, int VPL>
__global__ __launch_bounds__(64 * kWaves, (fwd_min_waves<VPL>())) void rms_fwd16(const char* x, int64_t ldx,
                                                                                const char* w, int64_t N, int H,
                                                                                float eps, char* y, int64_t ldy,
                                                                                float* rstd_out) {
  __shared__ u32x4 lw[VPL * 64];
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave_id();
  stage_weight<VPL>(w, H / 8, lw);
  if (row >= N) return;  // the whole wave
  const uint32_t rb = (uint32_t)H * 2, voff = (uint32_t)lane * 16;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + row * ldx * 2, rb), ry = rsrc(y + row * ldy * 2, rb);
  u32x4 v[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) v[k] = ld_vec(rx, voff, k);
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const float a = T::lo(v[k][d]), b = T::hi(v[k][d]);
      ss = __builtin_fmaf(a, a, ss);
      ss = __builtin_fmaf(b, b, ss);
    }
  ss = wave_sum(ss);
  double ssd = (double)ss;
  if (!(ss <= 0x1p+120f) || ss < 0x1p-100f) {
    // wave-uniform and rare: a square overflowed fp32 (|x| beyond ~2^60) or
    // the sum sits low enough for subnormal squares to matter; redo in fp64
    double s2 = 0.0;
#pragma unroll
    for (int k = 0; k < VPL; ++k)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const double a = (double)T::lo(v[k][d]), b = (double)T::hi(v[k][d]);
        s2 = fma(a, a, s2);
        s2 = fma(b, b, s2);
      }
    ssd = wave_sum(s2);
  }
  const float r = (float)(1.0 / sqrt(ssd / (double)H + (double)eps));
#pragma unroll
  for (int k = 0; k < VPL; ++k) fence_regs(v[k]);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const u32x4 wv = lw[k * 64 + lane];
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      o[d] = T::pack(T::lo(v[k][d]) * r * T::lo(wv[d]), T::hi(v[k][d]) * r * T::hi(wv[d]));
    buf_store<kNT>(o, ry, voff, k * 1024);
  }
  if (lane == 0) rstd_out[row] = r;
}

// Forward, fp32 rows: fp64 arithmetic, one rounding.
template <int VPL>
__global__ __launch_bounds__(64 * kWaves, (fwd_min_waves<VPL>())) void rms_fwd32(const char* x, int64_t ldx,
                                                                                const char* w, int64_t N, int H,
                                                                                float eps, char* y, int64_t ldy,
                                                                                float* rstd_out) {
  __shared__ u32x4 lw[VPL * 64];
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + wave_id();
  stage_weight<VPL>(w, H / 4, lw);
  if (row >= N) return;
  const uint32_t rb = (uint32_t)H * 4, voff = (uint32_t)lane * 16;
  const __amdgpu_buffer_rsrc_t rx = rsrc(x + row * ldx * 4, rb), ry = rsrc(y + row * ldy * 4, rb);
  u32x4 v[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) v[k] = ld_vec(rx, voff, k);
  __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const double a = (double)as_f(v[k][d]);
      ss = fma(a, a, ss);
    }
  ss = wave_sum(ss);
  const double r = 1.0 / sqrt(ss / (double)H + (double)eps);
#pragma unroll
  for (int k = 0; k < VPL; ++k) fence_regs(v[k]);
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const u32x4 wv = lw[k * 64 + lane];
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d)
      o[d] = __builtin_bit_cast(uint32_t, (float)((double)as_f(v[k][d]) * r * (double)as_f(wv[d])));
    buf_store<kNT>(o, ry, voff, k * 1024);
  }
  if (lane == 0) rstd_out[row] = (float)r;
}

// ---------------------------------------------------------------------------
// Backward: each wave takes rows blockIdx.x * kBwdWaves + wave, + gridDim.x *
// kBwdWaves, ...; dx is written per row; per-lane fp32 sums of dy x^ over
// those rows are added across the workgroup's waves in a fixed order through
// LDS and written as the workgroup's partial row of dw.  Lanes past the row
// load zeros (and a zero weight), so they add nothing to the sums.
//
// LDS: the weight row (static, staged once), and slots for the row groups' dw
// sums laid out [slot][wave share][vector k][quad][lane][4] with compile-time
// strides, so a wave moves its sums with 16-byte LDS accesses that the
// compiler can batch (with a runtime stride it could not prove the addresses
// apart and waited out every read-add-write in turn).  The row groups' sums
// meet in a pairwise tree (log2 of the groups' count steps, a fixed order);
// group 0 writes the workgroup's partial row straight from its registers.
// ---------------------------------------------------------------------------
template <int VPL, int EPV>
constexpr size_t bwd_lds_floats() { return (size_t)VPL * 64 * EPV; }

template <int EPV, int VPL, int R>
__device__ __forceinline__ void merge_store(float (&acc)[VPL][EPV], float* la, int nvec, float* partial_row,
                                            int lane, int rgi, int q) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  constexpr int Q = EPV / 4, RG = kBwdWaves / R;
  f4* l4 = (f4*)la;
  // pairwise tree over the row groups: at stride st, group rgi + st hands its
  // sums to group rgi (rgi a multiple of 2 st) through LDS slot rgi / (2 st),
  // which adds them to its own: ((s0 + s1) + (s2 + s3)) + ..., a fixed order
  for (int st = 1; st < RG; st *= 2) {
    const int slot = rgi / (2 * st);
    if (rgi % (2 * st) == st) {
#pragma unroll
      for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int u = 0; u < Q; ++u)
          l4[(((slot * R + q) * VPL + k) * Q + u) * 64 + lane] =
              f4{acc[k][4 * u], acc[k][4 * u + 1], acc[k][4 * u + 2], acc[k][4 * u + 3]};
    }
    __syncthreads();
    if (rgi % (2 * st) == 0) {
#pragma unroll
      for (int k = 0; k < VPL; ++k)
#pragma unroll
        for (int u = 0; u < Q; ++u) {
          const f4 b = l4[(((slot * R + q) * VPL + k) * Q + u) * 64 + lane];
          acc[k][4 * u] += b.x;
          acc[k][4 * u + 1] += b.y;
          acc[k][4 * u + 2] += b.z;
          acc[k][4 * u + 3] += b.w;
        }
    }
    __syncthreads();
  }
  if (rgi == 0) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = (q * VPL + k) * 64 + lane;
#pragma unroll
      for (int u = 0; u < Q; ++u)
        if (i < nvec)
          *(f4*)(partial_row + (size_t)i * EPV + 4 * u) =
              f4{acc[k][4 * u], acc[k][4 * u + 1], acc[k][4 * u + 2], acc[k][4 * u + 3]};
    }
  }
}

// The row's dot product from the partial sums of its R waves, in wave order
// (R > 1: through LDS, one barrier per row; the slot alternates with the
// iteration so a wave still reading the last row's sums is never overwritten).
template <int R>
__device__ __forceinline__ float group_sum(float part, float (&dp)[2][kBwdWaves], int it, int rgi, int q, int lane) {
  if constexpr (R == 1) {
    return part;
  } else {
    if (lane == 0) dp[it & 1][rgi * R + q] = part;
    __syncthreads();
    float s = dp[it & 1][rgi * R];
#pragma unroll
    for (int u = 1; u < R; ++u) s += dp[it & 1][rgi * R + u];
    return s;
  }
}

template <typename T, int VPL, int R>
__global__ __launch_bounds__(64 * kBwdWaves, (bwd_min_waves<VPL, R>())) void rms_bwd16(
    const char* dy, int64_t lddy, const char* x, int64_t ldx, const char* w, const float* rstd, int64_t N, int H,
    char* dx, int64_t lddx, float* partial) {
  constexpr int RG = kBwdWaves / R;  // rows in flight per workgroup
  __shared__ float lds_acc[bwd_lds_floats<VPL * kBwdWaves / 2, 8>()];  // the tree's slots
  __shared__ u32x4 lw[VPL * R * 64];
  __shared__ float dp[2][kBwdWaves];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int rgi = wid / R, q = wid % R;  // row group, and this wave's share of the row
  const int nvec = H / 8;
  const uint32_t rb = (uint32_t)H * 2, voff = (uint32_t)lane * 16;
  const int sb = q * VPL * 1024;  // byte offset of this wave's columns
  stage_weight<VPL * R>(w, nvec, lw);
  const u32x4* lwq = lw + q * VPL * 64;
  float acc[VPL][8];
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.0f;
  // the same trip count for every wave of the workgroup (R > 1 has a barrier
  // per row); a row past the end has empty buffer resources: loads give 0 and
  // stores are dropped
  int it = 0;
  for (int64_t r0 = (int64_t)blockIdx.x * RG; r0 < N; r0 += (int64_t)gridDim.x * RG, ++it) {
    const int64_t row = r0 + rgi;
    const uint32_t nb = row < N ? rb : 0u;
    const __amdgpu_buffer_rsrc_t rg = rsrc(dy + row * lddy * 2, nb), rx = rsrc(x + row * ldx * 2, nb);
    u32x4 g[VPL], xv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      g[k] = ld_vec(rg, voff, sb / 1024 + k);
      xv[k] = ld_vec(rx, voff, sb / 1024 + k);
    }
    __builtin_amdgcn_sched_barrier(0);
    const float r = row < N ? rstd[row] : 0.0f;
    float dot = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const u32x4 wv = lwq[k * 64 + lane];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        dot = __builtin_fmaf(T::lo(xv[k][d]) * r, T::lo(wv[d]) * T::lo(g[k][d]), dot);
        dot = __builtin_fmaf(T::hi(xv[k][d]) * r, T::hi(wv[d]) * T::hi(g[k][d]), dot);
      }
    }
    const float c = group_sum<R>(wave_sum(dot), dp, it, rgi, q, lane) / (float)H;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      fence_regs(g[k]);
      fence_regs(xv[k]);
    }
    const __amdgpu_buffer_rsrc_t ro = rsrc(dx + row * lddx * 2, nb);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const u32x4 wv = lwq[k * 64 + lane];
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float xl = T::lo(xv[k][d]) * r, xh = T::hi(xv[k][d]) * r;
        const float gl = T::lo(g[k][d]), gh = T::hi(g[k][d]);
        o[d] = T::pack(r * (T::lo(wv[d]) * gl - xl * c), r * (T::hi(wv[d]) * gh - xh * c));
        acc[k][2 * d] = __builtin_fmaf(gl, xl, acc[k][2 * d]);
        acc[k][2 * d + 1] = __builtin_fmaf(gh, xh, acc[k][2 * d + 1]);
      }
      buf_store<kNT>(o, ro, voff, sb + k * 1024);
    }
  }
  merge_store<8, VPL, R>(acc, lds_acc, nvec, partial + (int64_t)blockIdx.x * H, lane, rgi, q);
}

// Backward, fp32 rows: y-side arithmetic in fp64, the dw sums in fp32.
template <int VPL, int R>
__global__ __launch_bounds__(64 * kBwdWaves, (bwd_min_waves<VPL, R>())) void rms_bwd32(
    const char* dy, int64_t lddy, const char* x, int64_t ldx, const char* w, const float* rstd, int64_t N, int H,
    char* dx, int64_t lddx, float* partial) {
  constexpr int RG = kBwdWaves / R;
  __shared__ float lds_acc[bwd_lds_floats<VPL * kBwdWaves / 2, 4>()];
  __shared__ u32x4 lw[VPL * R * 64];
  __shared__ double dpd[2][kBwdWaves];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int rgi = wid / R, q = wid % R;
  const int nvec = H / 4;
  const uint32_t rb = (uint32_t)H * 4, voff = (uint32_t)lane * 16;
  const int sb = q * VPL * 1024;
  stage_weight<VPL * R>(w, nvec, lw);
  const u32x4* lwq = lw + q * VPL * 64;
  float acc[VPL][4];
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[k][e] = 0.0f;
  int it = 0;
  for (int64_t r0 = (int64_t)blockIdx.x * RG; r0 < N; r0 += (int64_t)gridDim.x * RG, ++it) {
    const int64_t row = r0 + rgi;
    const uint32_t nb = row < N ? rb : 0u;
    const __amdgpu_buffer_rsrc_t rg = rsrc(dy + row * lddy * 4, nb), rx = rsrc(x + row * ldx * 4, nb);
    u32x4 g[VPL], xv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      g[k] = ld_vec(rg, voff, sb / 1024 + k);
      xv[k] = ld_vec(rx, voff, sb / 1024 + k);
    }
    __builtin_amdgcn_sched_barrier(0);
    const double r = row < N ? (double)rstd[row] : 0.0;
    double dot = 0.0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const u32x4 wv = lwq[k * 64 + lane];
#pragma unroll
      for (int d = 0; d < 4; ++d)
        dot = fma((double)as_f(xv[k][d]) * r, (double)as_f(wv[d]) * (double)as_f(g[k][d]), dot);
    }
    dot = wave_sum(dot);
    if constexpr (R > 1) {  // the row's R partial sums, in wave order
      if (lane == 0) dpd[it & 1][rgi * R + q] = dot;
      __syncthreads();
      dot = dpd[it & 1][rgi * R];
#pragma unroll
      for (int u = 1; u < R; ++u) dot += dpd[it & 1][rgi * R + u];
    }
    const double c = dot / (double)H;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      fence_regs(g[k]);
      fence_regs(xv[k]);
    }
    const __amdgpu_buffer_rsrc_t ro = rsrc(dx + row * lddx * 4, nb);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const u32x4 wv = lwq[k * 64 + lane];
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const double xh = (double)as_f(xv[k][d]) * r, gd = (double)as_f(g[k][d]);
        o[d] = __builtin_bit_cast(uint32_t, (float)(r * ((double)as_f(wv[d]) * gd - xh * c)));
        acc[k][d] = __builtin_fmaf((float)gd, (float)xh, acc[k][d]);
      }
      buf_store<kNT>(o, ro, voff, sb + k * 1024);
    }
  }
  merge_store<4, VPL, R>(acc, lds_acc, nvec, partial + (int64_t)blockIdx.x * H, lane, rgi, q);
}

// dw[j] = sum over the G partial rows in fp64, rounded once.  A workgroup
// takes 64 columns as 16 column quads; its 16 row slices (contiguous ranges
// of the G rows) are summed by separate threads with all their 16-byte loads
// in flight together, then added in slice order through LDS: a fixed order,
// whatever the timing.  H is a multiple of 4.
#ifndef RMS_RED_QUADS
#define RMS_RED_QUADS 16
#endif
constexpr int kRedQuads = RMS_RED_QUADS, kRedSlices = 256 / kRedQuads, kRedUnroll = 16;
template <typename TO>
__global__ __launch_bounds__(kRedQuads * kRedSlices) void rms_dw_reduce(const float* partial, int G, int H, TO* dw) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  __shared__ double part[kRedSlices][kRedQuads * 4];
  const int cq = threadIdx.x % kRedQuads, sl = threadIdx.x / kRedQuads;
  const int j = (blockIdx.x * kRedQuads + cq) * 4;
  const int per = (G + kRedSlices - 1) / kRedSlices;
  const int g0 = sl * per, g1 = min(G, g0 + per);
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  if (j < H) {
    for (int g = g0; g < g1; g += kRedUnroll) {
      f4 v[kRedUnroll];
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u)
        v[u] = g + u < g1 ? *(const f4*)(partial + (int64_t)(g + u) * H + j) : f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) {
        s0 += (double)v[u].x;
        s1 += (double)v[u].y;
        s2 += (double)v[u].z;
        s3 += (double)v[u].w;
      }
    }
  }
  part[sl][cq * 4 + 0] = s0;
  part[sl][cq * 4 + 1] = s1;
  part[sl][cq * 4 + 2] = s2;
  part[sl][cq * 4 + 3] = s3;
  __syncthreads();
  const int c = threadIdx.x;  // one output column per thread of the first 4 kRedQuads
  const int jc = blockIdx.x * kRedQuads * 4 + c;
  if (c < kRedQuads * 4 && jc < H) {
    double t = part[0][c];
#pragma unroll
    for (int q = 1; q < kRedSlices; ++q) t += part[q][c];
    dw[jc] = (TO)t;
  }
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------
bool valid_dtype(int d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16 || d == CE_DTYPE_F16; }
int esize(int d) { return d == CE_DTYPE_F32 ? 4 : 2; }

// Vectors per lane for a row of H elements (0: not served).
int vpl_for(int64_t H, int dtype) {
  const int epv = 16 / esize(dtype);
  if (H < 1 || H % epv) return 0;
  const int64_t nvec = H / epv;
  for (int v = 1; v <= kMaxVPL; v *= 2)
    if ((int64_t)v * 64 >= nvec) return v;
  return 0;
}

int bwd_groups(int64_t N) {
  const int64_t g = (N + kBwdWaves - 1) / kBwdWaves;
  return (int)(g < 1 ? 1 : (g > kMaxBwdGroups ? kMaxBwdGroups : g));
}

typedef void (*FwdFn)(const char*, int64_t, const char*, int64_t, int, float, char*, int64_t, float*);
typedef void (*BwdFn)(const char*, int64_t, const char*, int64_t, const char*, const float*, int64_t, int, char*,
                      int64_t, float*);

#define RMS_VPL_CASES(MAKE) MAKE(1) MAKE(2) MAKE(4) MAKE(8) MAKE(16) MAKE(32)
// backward: total vectors per lane -> (vectors per wave, waves per row)
#define RMS_BWD_CASES(MAKE) MAKE(1, 1) MAKE(2, 1) MAKE(4, 1) MAKE(8, 1) MAKE(8, 2) MAKE(8, 4)

FwdFn fwd_fn(int dtype, int vpl) {
#define MAKE(V)                                          \
  if (vpl == V) {                                        \
    if (dtype == CE_DTYPE_BF16) return rms_fwd16<BF16, V>; \
    if (dtype == CE_DTYPE_F16) return rms_fwd16<F16, V>;   \
    return rms_fwd32<V>;                                 \
  }
  RMS_VPL_CASES(MAKE)
#undef MAKE
  return nullptr;
}
BwdFn bwd_fn(int dtype, int vpl) {
  const int r = vpl > kMaxBwdVPL ? vpl / kMaxBwdVPL : 1, v = vpl / r;
#define MAKE(V, R)                                             \
  if (v == V && r == R) {                                      \
    if (dtype == CE_DTYPE_BF16) return rms_bwd16<BF16, V, R>;  \
    if (dtype == CE_DTYPE_F16) return rms_bwd16<F16, V, R>;    \
    return rms_bwd32<V, R>;                                    \
  }
  RMS_BWD_CASES(MAKE)
#undef MAKE
  return nullptr;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

size_t ce_rmsnorm_workspace_bytes(int64_t n_rows, int64_t hidden, int dtype) {
  if (!valid_dtype(dtype) || n_rows < 0 || vpl_for(hidden, dtype) == 0) return 0;
  return ((size_t)bwd_groups(n_rows) * (size_t)hidden * 4 + 255) & ~(size_t)255;
}

int ce_rmsnorm_forward(const void* x, int64_t ld_x, const void* weight, int64_t n_rows, int64_t hidden, int dtype,
                       float eps, void* y, int64_t ld_y, float* rstd, void* stream) {
  if (!valid_dtype(dtype)) return CE_ERR_DTYPE;
  const int64_t N = n_rows, H = hidden;
  if (N < 0 || H < 1 || ld_x < H || ld_y < H || !(eps >= 0.0f)) return CE_ERR_INVALID_ARG;
  if (N > 0 && (x == nullptr || weight == nullptr || y == nullptr || rstd == nullptr)) return CE_ERR_INVALID_ARG;
  const int es = esize(dtype), vpl = vpl_for(H, dtype);
  if (vpl == 0 || H > ((int64_t)1 << 30)) return CE_ERR_UNSUPPORTED;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(y) || (ld_x * es) % 16 || (ld_y * es) % 16)
    return CE_ERR_UNSUPPORTED;
  // y may be x itself (same stride): each row is read whole before it is written
  if (y == x && ld_y != ld_x) return CE_ERR_INVALID_ARG;
  if (N == 0) return CE_OK;
  const int64_t grid = (N + kWaves - 1) / kWaves;
  if (grid > 0x7fffffff) return CE_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(fwd_fn(dtype, vpl), dim3((unsigned)grid), dim3(64 * kWaves), 0, (hipStream_t)stream,
                     (const char*)x, ld_x, (const char*)weight, N, (int)H, eps, (char*)y, ld_y, rstd);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

int ce_rmsnorm_backward(const void* dy, int64_t ld_dy, const void* x, int64_t ld_x, const void* weight,
                        const float* rstd, int64_t n_rows, int64_t hidden, int dtype, void* dx, int64_t ld_dx,
                        void* dweight, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return CE_ERR_DTYPE;
  const int64_t N = n_rows, H = hidden;
  if (N < 0 || H < 1 || ld_dy < H || ld_x < H || ld_dx < H) return CE_ERR_INVALID_ARG;
  if (dweight == nullptr || weight == nullptr) return CE_ERR_INVALID_ARG;
  if (N > 0 && (dy == nullptr || x == nullptr || rstd == nullptr || dx == nullptr)) return CE_ERR_INVALID_ARG;
  const int es = esize(dtype), vpl = vpl_for(H, dtype);
  if (vpl == 0 || bwd_fn(dtype, vpl) == nullptr) return CE_ERR_UNSUPPORTED;
  if (!aligned16(dy) || !aligned16(x) || !aligned16(weight) || !aligned16(dx) || (ld_dy * es) % 16 ||
      (ld_x * es) % 16 || (ld_dx * es) % 16)
    return CE_ERR_UNSUPPORTED;
  if ((uintptr_t)dweight % es) return CE_ERR_INVALID_ARG;
  // dx may be dy itself (same stride): each row is read whole before it is written
  if (dx == dy && ld_dx != ld_dy) return CE_ERR_INVALID_ARG;
  const size_t need = ce_rmsnorm_workspace_bytes(N, H, dtype);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 255)) return CE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* partial = (float*)workspace;
  const int G = bwd_groups(N);
  if (N > 0) {
    hipLaunchKernelGGL(bwd_fn(dtype, vpl), dim3((unsigned)G), dim3(64 * kBwdWaves), 0, st, (const char*)dy,
                       ld_dy, (const char*)x, ld_x, (const char*)weight, rstd, N, (int)H, (char*)dx, ld_dx, partial);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  const int gsum = N > 0 ? G : 0;
  const unsigned rb = (unsigned)((H + kRedQuads * 4 - 1) / (kRedQuads * 4));
  const dim3 rt(kRedQuads * kRedSlices);
  if (dtype == CE_DTYPE_BF16)
    hipLaunchKernelGGL(rms_dw_reduce<__bf16>, dim3(rb), rt, 0, st, partial, gsum, (int)H, (__bf16*)dweight);
  else if (dtype == CE_DTYPE_F16)
    hipLaunchKernelGGL(rms_dw_reduce<_Float16>, dim3(rb), rt, 0, st, partial, gsum, (int)H, (_Float16*)dweight);
  else
    hipLaunchKernelGGL(rms_dw_reduce<float>, dim3(rb), rt, 0, st, partial, gsum, (int)H, (float*)dweight);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

}  // extern "C"
