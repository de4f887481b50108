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
// sums of squares and dot products reduced with DPP lane moves, no LDS and no
// barrier on the row path.  The backward's dw is summed without atomics: each
// wave keeps per-lane fp32 sums over the rows it handles, the four waves of a
// workgroup are added in a fixed order through LDS, and a second launch adds
// the workgroups' partials in a fixed order (deterministic).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "ce_mi355x.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;          // waves (rows in flight) per workgroup
constexpr int kMaxBwdGroups = 256; // backward workgroups: partial rows of dw
constexpr int kMaxVPL = 32;     // forward: rows up to 32 KB (16384 bf16 / 8192 fp32)
constexpr int kMaxBwdVPL = 8;   // backward: the per-lane dw sums (8 VPL floats) stay in VGPRs

// Waves per SIMD the register budget must allow (without a bound the
// compiler has taken up to 256 VGPRs for these shapes, one wave per SIMD).
template <int VPL>
constexpr int fwd_min_waves() { return VPL <= 8 ? 8 : (VPL <= 16 ? 4 : 2); }
template <int VPL>
constexpr int bwd_min_waves() { return VPL <= 4 ? 4 : 3; }

// Makes the compiler treat v as redefined here, so that values it derived
// from v earlier (unpacked floats) are recomputed rather than kept live
// across the two passes over the row.
__device__ __forceinline__ void fence_regs(u32x4& v) { asm volatile("" : "+v"(v)); }

struct BF16 {
  static constexpr int EPV = 8;
  __device__ static float lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
  __device__ static float hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
  __device__ static uint32_t pack(float a, float b) {
    f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
  }
};
struct F16 {
  static constexpr int EPV = 8;
  __device__ static float lo(uint32_t u) { return (float)__builtin_bit_cast(h2, u).x; }
  __device__ static float hi(uint32_t u) { return (float)__builtin_bit_cast(h2, u).y; }
  __device__ static uint32_t pack(float a, float b) {
    f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  }
};

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }

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
__global__ __launch_bounds__(64 * kWaves, (fwd_min_waves<VPL>())) void rms_fwd16(const char* x, int64_t ldx, const char* w, int64_t N, int H,
                                                         float eps, char* y, int64_t ldy, float* rstd_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= N) return;  // the whole wave
  const u32x4* xr = (const u32x4*)(x + row * ldx * 2);
  const u32x4* wr = (const u32x4*)w;
  u32x4* yr = (u32x4*)(y + row * ldy * 2);
  const int nvec = H / 8;
  u32x4 v[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int i = k * 64 + lane;
    if (i < nvec) v[k] = __builtin_nontemporal_load(xr + i);
  }
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
    if (k * 64 + lane < nvec)
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
      if (k * 64 + lane < nvec)
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
    const int i = k * 64 + lane;
    if (i < nvec) {
      const u32x4 wv = wr[i];
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = T::pack(T::lo(v[k][d]) * r * T::lo(wv[d]), T::hi(v[k][d]) * r * T::hi(wv[d]));
      __builtin_nontemporal_store(o, yr + i);
    }
  }
  if (lane == 0) rstd_out[row] = r;
}

// Forward, fp32 rows: fp64 arithmetic, one rounding.
template <int VPL>
__global__ __launch_bounds__(64 * kWaves, (fwd_min_waves<VPL>())) void rms_fwd32(const char* x, int64_t ldx, const char* w, int64_t N, int H,
                                                         float eps, char* y, int64_t ldy, float* rstd_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  if (row >= N) return;
  const u32x4* xr = (const u32x4*)(x + row * ldx * 4);
  const u32x4* wr = (const u32x4*)w;
  u32x4* yr = (u32x4*)(y + row * ldy * 4);
  const int nvec = H / 4;
  u32x4 v[VPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    const int i = k * 64 + lane;
    if (i < nvec) v[k] = __builtin_nontemporal_load(xr + i);
  }
  double ss = 0.0;
#pragma unroll
  for (int k = 0; k < VPL; ++k)
    if (k * 64 + lane < nvec)
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
    const int i = k * 64 + lane;
    if (i < nvec) {
      const u32x4 wv = wr[i];
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = __builtin_bit_cast(uint32_t, (float)((double)as_f(v[k][d]) * r * (double)as_f(wv[d])));
      __builtin_nontemporal_store(o, yr + i);
    }
  }
  if (lane == 0) rstd_out[row] = (float)r;
}

// ---------------------------------------------------------------------------
// Backward: each wave takes rows blockIdx.x * kWaves + wave, + gridDim.x *
// kWaves, ...; dx is written per row; per-lane fp32 sums of dy x^ over those
// rows are added across the four waves in a fixed order (LDS, H floats) and
// written as the workgroup's partial row of dw.
// ---------------------------------------------------------------------------
template <typename T, int VPL>
__global__ __launch_bounds__(64 * kWaves, (bwd_min_waves<VPL>())) void rms_bwd16(const char* dy, int64_t lddy, const char* x, int64_t ldx,
                                                         const char* w, const float* rstd, int64_t N, int H,
                                                         char* dx, int64_t lddx, float* partial) {
  extern __shared__ float lds_acc[];  // H floats
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nvec = H / 8;
  const u32x4* wr = (const u32x4*)w;
  float acc[VPL][8];
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[k][e] = 0.0f;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wid; row < N; row += (int64_t)gridDim.x * kWaves) {
    const u32x4* gr = (const u32x4*)(dy + row * lddy * 2);
    const u32x4* xr = (const u32x4*)(x + row * ldx * 2);
    u32x4 g[VPL], xv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = k * 64 + lane;
      if (i < nvec) {
        g[k] = __builtin_nontemporal_load(gr + i);
        xv[k] = __builtin_nontemporal_load(xr + i);
      }
    }
    const float r = rstd[row];
    float dot = 0.0f;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = k * 64 + lane;
      if (i < nvec) {
        const u32x4 wv = wr[i];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          dot = __builtin_fmaf(T::lo(xv[k][d]) * r, T::lo(wv[d]) * T::lo(g[k][d]), dot);
          dot = __builtin_fmaf(T::hi(xv[k][d]) * r, T::hi(wv[d]) * T::hi(g[k][d]), dot);
        }
      }
    }
    const float c = wave_sum(dot) / (float)H;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      fence_regs(g[k]);
      fence_regs(xv[k]);
    }
    u32x4* outr = (u32x4*)(dx + row * lddx * 2);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = k * 64 + lane;
      if (i < nvec) {
        const u32x4 wv = wr[i];
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float xl = T::lo(xv[k][d]) * r, xh = T::hi(xv[k][d]) * r;
          const float gl = T::lo(g[k][d]), gh = T::hi(g[k][d]);
          o[d] = T::pack(r * (T::lo(wv[d]) * gl - xl * c), r * (T::hi(wv[d]) * gh - xh * c));
          acc[k][2 * d] = __builtin_fmaf(gl, xl, acc[k][2 * d]);
          acc[k][2 * d + 1] = __builtin_fmaf(gh, xh, acc[k][2 * d + 1]);
        }
        __builtin_nontemporal_store(o, outr + i);
      }
    }
  }
  // the four waves' sums, added in wave order
  for (int wv = 0; wv < kWaves; ++wv) {
    if (wid == wv) {
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const int i = k * 64 + lane;
        if (i < nvec)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int j = i * 8 + e;
            lds_acc[j] = (wv == 0 ? 0.0f : lds_acc[j]) + acc[k][e];
          }
      }
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < H; j += 64 * kWaves) partial[(int64_t)blockIdx.x * H + j] = lds_acc[j];
}

// Backward, fp32 rows: y-side arithmetic in fp64, the dw sums in fp32.
template <int VPL>
__global__ __launch_bounds__(64 * kWaves, (bwd_min_waves<VPL>())) void rms_bwd32(const char* dy, int64_t lddy, const char* x, int64_t ldx,
                                                         const char* w, const float* rstd, int64_t N, int H,
                                                         char* dx, int64_t lddx, float* partial) {
  extern __shared__ float lds_acc[];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int nvec = H / 4;
  const u32x4* wr = (const u32x4*)w;
  float acc[VPL][4];
#pragma unroll
  for (int k = 0; k < VPL; ++k)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[k][e] = 0.0f;
  for (int64_t row = (int64_t)blockIdx.x * kWaves + wid; row < N; row += (int64_t)gridDim.x * kWaves) {
    const u32x4* gr = (const u32x4*)(dy + row * lddy * 4);
    const u32x4* xr = (const u32x4*)(x + row * ldx * 4);
    u32x4 g[VPL], xv[VPL];
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = k * 64 + lane;
      if (i < nvec) {
        g[k] = __builtin_nontemporal_load(gr + i);
        xv[k] = __builtin_nontemporal_load(xr + i);
      }
    }
    const double r = (double)rstd[row];
    double dot = 0.0;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = k * 64 + lane;
      if (i < nvec) {
        const u32x4 wv = wr[i];
#pragma unroll
        for (int d = 0; d < 4; ++d)
          dot = fma((double)as_f(xv[k][d]) * r, (double)as_f(wv[d]) * (double)as_f(g[k][d]), dot);
      }
    }
    const double c = wave_sum(dot) / (double)H;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      fence_regs(g[k]);
      fence_regs(xv[k]);
    }
    u32x4* outr = (u32x4*)(dx + row * lddx * 4);
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int i = k * 64 + lane;
      if (i < nvec) {
        const u32x4 wv = wr[i];
        u32x4 o;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const double xh = (double)as_f(xv[k][d]) * r, gd = (double)as_f(g[k][d]);
          o[d] = __builtin_bit_cast(uint32_t, (float)(r * ((double)as_f(wv[d]) * gd - xh * c)));
          acc[k][d] = __builtin_fmaf((float)gd, (float)xh, acc[k][d]);
        }
        __builtin_nontemporal_store(o, outr + i);
      }
    }
  }
  for (int wv = 0; wv < kWaves; ++wv) {
    if (wid == wv) {
#pragma unroll
      for (int k = 0; k < VPL; ++k) {
        const int i = k * 64 + lane;
        if (i < nvec)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = i * 4 + e;
            lds_acc[j] = (wv == 0 ? 0.0f : lds_acc[j]) + acc[k][e];
          }
      }
    }
    __syncthreads();
  }
  for (int j = threadIdx.x; j < H; j += 64 * kWaves) partial[(int64_t)blockIdx.x * H + j] = lds_acc[j];
}

// dw[j] = sum over the G partial rows, in order, in fp64; rounded once.
template <typename TO>
__global__ __launch_bounds__(256) void rms_dw_reduce(const float* partial, int G, int H, TO* dw) {
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= H) return;
  double s = 0.0;
  for (int g = 0; g < G; ++g) s += (double)partial[(int64_t)g * H + j];
  dw[j] = (TO)s;
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
  const int64_t g = (N + kWaves - 1) / kWaves;
  return (int)(g < 1 ? 1 : (g > kMaxBwdGroups ? kMaxBwdGroups : g));
}

typedef void (*FwdFn)(const char*, int64_t, const char*, int64_t, int, float, char*, int64_t, float*);
typedef void (*BwdFn)(const char*, int64_t, const char*, int64_t, const char*, const float*, int64_t, int, char*,
                      int64_t, float*);

#define RMS_VPL_CASES(MAKE) MAKE(1) MAKE(2) MAKE(4) MAKE(8) MAKE(16) MAKE(32)
#define RMS_BWD_VPL_CASES(MAKE) MAKE(1) MAKE(2) MAKE(4) MAKE(8)

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
#define MAKE(V)                                          \
  if (vpl == V) {                                        \
    if (dtype == CE_DTYPE_BF16) return rms_bwd16<BF16, V>; \
    if (dtype == CE_DTYPE_F16) return rms_bwd16<F16, V>;   \
    return rms_bwd32<V>;                                 \
  }
  RMS_BWD_VPL_CASES(MAKE)
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
  if (vpl == 0 || vpl > kMaxBwdVPL) return CE_ERR_UNSUPPORTED;
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
    hipLaunchKernelGGL(bwd_fn(dtype, vpl), dim3((unsigned)G), dim3(64 * kWaves), (size_t)H * 4, st, (const char*)dy,
                       ld_dy, (const char*)x, ld_x, (const char*)weight, rstd, N, (int)H, (char*)dx, ld_dx, partial);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  const int gsum = N > 0 ? G : 0;
  const unsigned rb = (unsigned)((H + 255) / 256);
  if (dtype == CE_DTYPE_BF16)
    hipLaunchKernelGGL(rms_dw_reduce<__bf16>, dim3(rb), dim3(256), 0, st, partial, gsum, (int)H, (__bf16*)dweight);
  else if (dtype == CE_DTYPE_F16)
    hipLaunchKernelGGL(rms_dw_reduce<_Float16>, dim3(rb), dim3(256), 0, st, partial, gsum, (int)H,
                       (_Float16*)dweight);
  else
    hipLaunchKernelGGL(rms_dw_reduce<float>, dim3(rb), dim3(256), 0, st, partial, gsum, (int)H, (float*)dweight);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

}  // extern "C"
