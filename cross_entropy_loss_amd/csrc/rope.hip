// rope.hip -- rotary position embedding with per-token position ids, for
// gfx950 (the C ABI in include/ce_mi355x.h: ce_rope).
//
// The pages list "Fast RoPE" among the package's kernels (PyPI page
// "fms-acceleration-foak 0.7.4", kernel list) and note that it takes no
// position ids (same page, known issues; fms-hf-tuning PR #280, "Notes on
// FastKernels"), which padding-free packed batches need.  Per token t with
// position p and head_dim D (P = D/2 pairs, pair i = elements i and i + P of
// every head):
//   theta_i = p base^(-2i/D),
//   y_i = x_i cos - x_{i+P} sin,   y_{i+P} = x_{i+P} cos + x_i sin,
// and the gradient is the same rotation by -theta (inverse = 1).
//
// Shape of the work.  Elementwise and HBM-bound; the angles depend on the
// token and the pair only.  One wave per token: it computes the token's P
// (cos, sin) pairs once, in fp64 (exp2 for the frequency, sincos of the full
// angle, so positions in the hundreds of thousands keep their digits), keeps
// them in LDS, then streams every head of q and k through buffer resources
// with 16-byte vectors: a lane holds one vector of a head's first half and the
// matching vector of its second half, P/EPV lanes per head, 64/(P/EPV) heads
// per pass, all of a batch of passes' loads in flight before any arithmetic.
// Heads past the end and idle lanes use an out-of-range offset (loads return
// 0, stores are dropped), so the row path has no branches.  16-bit formats
// rotate in fp32 (cos and sin rounded to fp32) and round once; fp32 data
// rotates in fp64.
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

constexpr int kMaxPairs = 128;  // head_dim up to 256
constexpr int kPasses = 4;      // head passes whose loads are issued together
constexpr int kNT = 2;          // buffer aux bits: nontemporal

struct RopeArgs {
  const char* x[2];
  char* y[2];
  int64_t ld_tok[2];   // elements between tokens
  int64_t ld_head[2];  // elements between heads
  int heads[2];        // 0: tensor absent
  uint32_t bytes[2];   // extent of one token's heads from its base, in bytes
  const int64_t* pos;
  int D;
  double log2_base;
  int inverse;
};

__device__ __forceinline__ u32x4 ld_vec(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, kNT));
}

// (cos, sin) of the token's P angles, in fp64 (sin negated for the inverse).
__device__ __forceinline__ void token_angles(const RopeArgs& a, double p, int lane, double* c, double* s, int P) {
  for (int i = lane; i < P; i += 64) {
    const double f = exp2(-(double)(2 * i) / (double)a.D * a.log2_base);
    double sn, cs;
    sincos(p * f, &sn, &cs);
    c[i] = cs;
    s[i] = a.inverse ? -sn : sn;
  }
}

// 16-bit formats: EPV = 8 elements per 16-byte vector.
template <typename T>
__global__ __launch_bounds__(64) void rope16(RopeArgs a) {
  __shared__ float lc[kMaxPairs], ls[kMaxPairs];
  __shared__ double tc[kMaxPairs], ts[kMaxPairs];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int P = a.D >> 1;
  token_angles(a, (double)a.pos[t], lane, tc, ts, P);
  for (int i = lane; i < P; i += 64) {
    lc[i] = (float)tc[i];
    ls[i] = (float)ts[i];
  }
  __syncthreads();
  const int lph = P / 8, hpw = 64 / lph;
  const int v = lane % lph, hg = lane / lph;
  float c[8], s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    c[e] = lc[v * 8 + e];
    s[e] = ls[v * 8 + e];
  }
  const int half = P * 2;  // bytes from a head's first half to its second
#pragma unroll
  for (int z = 0; z < 2; ++z) {
    const int H = a.heads[z];
    if (H == 0) continue;
    const __amdgpu_buffer_rsrc_t in = row_rsrc(a.x[z] + t * a.ld_tok[z] * 2, a.bytes[z]);
    const __amdgpu_buffer_rsrc_t out = row_rsrc(a.y[z] + t * a.ld_tok[z] * 2, a.bytes[z]);
    for (int h0 = 0; h0 < H; h0 += hpw * kPasses) {
      uint32_t off[kPasses];
      u32x4 lo[kPasses], hi[kPasses];
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        const int h = h0 + u * hpw + hg;
        off[u] = (hg < hpw && h < H) ? (uint32_t)((int64_t)h * a.ld_head[z] * 2 + v * 16) : a.bytes[z];
        lo[u] = ld_vec(in, off[u], 0);
        hi[u] = ld_vec(in, off[u], half);
      }
      __builtin_amdgcn_sched_barrier(0);  // every load in flight before the first use
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        u32x4 ol, oh;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const float a0 = T::lo(lo[u][d]), a1 = T::hi(lo[u][d]);
          const float b0 = T::lo(hi[u][d]), b1 = T::hi(hi[u][d]);
          const int e0 = 2 * d, e1 = 2 * d + 1;
          ol[d] = T::pack(__builtin_fmaf(a0, c[e0], -(b0 * s[e0])), __builtin_fmaf(a1, c[e1], -(b1 * s[e1])));
          oh[d] = T::pack(__builtin_fmaf(b0, c[e0], a0 * s[e0]), __builtin_fmaf(b1, c[e1], a1 * s[e1]));
        }
        buf_store<kNT>(ol, out, off[u], 0);
        buf_store<kNT>(oh, out, off[u], half);
      }
    }
  }
}

// fp32 data: EPV = 4, rotation in fp64, one rounding.
__global__ __launch_bounds__(64) void rope32(RopeArgs a) {
  __shared__ double tc[kMaxPairs], ts[kMaxPairs];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const int P = a.D >> 1;
  token_angles(a, (double)a.pos[t], lane, tc, ts, P);
  __syncthreads();
  const int lph = P / 4, hpw = 64 / lph;
  const int v = lane % lph, hg = lane / lph;
  double c[4], s[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    c[e] = tc[v * 4 + e];
    s[e] = ts[v * 4 + e];
  }
  const int half = P * 4;
#pragma unroll
  for (int z = 0; z < 2; ++z) {
    const int H = a.heads[z];
    if (H == 0) continue;
    const __amdgpu_buffer_rsrc_t in = row_rsrc(a.x[z] + t * a.ld_tok[z] * 4, a.bytes[z]);
    const __amdgpu_buffer_rsrc_t out = row_rsrc(a.y[z] + t * a.ld_tok[z] * 4, a.bytes[z]);
    for (int h0 = 0; h0 < H; h0 += hpw * kPasses) {
      uint32_t off[kPasses];
      u32x4 lo[kPasses], hi[kPasses];
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        const int h = h0 + u * hpw + hg;
        off[u] = (hg < hpw && h < H) ? (uint32_t)((int64_t)h * a.ld_head[z] * 4 + v * 16) : a.bytes[z];
        lo[u] = ld_vec(in, off[u], 0);
        hi[u] = ld_vec(in, off[u], half);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < kPasses; ++u) {
        u32x4 ol, oh;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double x1 = (double)as_f(lo[u][e]), x2 = (double)as_f(hi[u][e]);
          ol[e] = __builtin_bit_cast(uint32_t, (float)fma(x1, c[e], -(x2 * s[e])));
          oh[e] = __builtin_bit_cast(uint32_t, (float)fma(x2, c[e], x1 * s[e]));
        }
        buf_store<kNT>(ol, out, off[u], 0);
        buf_store<kNT>(oh, out, off[u], half);
      }
    }
  }
}

bool valid_dtype(int d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16 || d == CE_DTYPE_F16; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

// The (token, head) segments of D elements must not overlap: the smaller
// stride spans at least D, the larger at least the count along the smaller.
bool disjoint(int64_t T, int64_t H, int64_t ld_t, int64_t ld_h, int64_t D) {
  if (T <= 1 && H <= 1) return true;
  if (T <= 1) return ld_h >= D;
  if (H <= 1) return ld_t >= D;
  if (ld_h <= ld_t) return ld_h >= D && ld_t >= H * ld_h;
  return ld_t >= D && ld_h >= T * ld_t;
}

}  // namespace

extern "C" {

int ce_rope(const void* q, void* q_out, int64_t q_ld_token, int64_t q_ld_head, int64_t q_heads, const void* k,
            void* k_out, int64_t k_ld_token, int64_t k_ld_head, int64_t k_heads, const int64_t* positions,
            int64_t n_tokens, int64_t head_dim, double base, int inverse, int dtype, void* stream) {
  if (!valid_dtype(dtype)) return CE_ERR_DTYPE;
  const int64_t T = n_tokens, D = head_dim;
  if (T < 0 || q_heads < 0 || k_heads < 0 || D < 2 || (D & 1) || !(base > 0.0) || !isfinite(base) ||
      (inverse != 0 && inverse != 1))
    return CE_ERR_INVALID_ARG;
  const int es = dtype == CE_DTYPE_F32 ? 4 : 2, epv = 16 / es;
  if ((D / 2) % epv || D / 2 > kMaxPairs) return CE_ERR_UNSUPPORTED;
  if (T > 0x7fffffff || q_heads > 0x7fffffff || k_heads > 0x7fffffff) return CE_ERR_UNSUPPORTED;
  if (T == 0 || q_heads + k_heads == 0) return CE_OK;  // nothing is read or written (pointers may be NULL)
  if (positions == nullptr) return CE_ERR_INVALID_ARG;
  RopeArgs a;
  const void* xs[2] = {q, k};
  void* ys[2] = {q_out, k_out};
  const int64_t lts[2] = {q_ld_token, k_ld_token}, lhs[2] = {q_ld_head, k_ld_head}, hs[2] = {q_heads, k_heads};
  for (int z = 0; z < 2; ++z) {
    a.x[z] = (const char*)xs[z];
    a.y[z] = (char*)ys[z];
    a.ld_tok[z] = lts[z];
    a.ld_head[z] = lhs[z];
    a.heads[z] = (int)hs[z];
    a.bytes[z] = 0;
    if (hs[z] == 0) continue;
    if (xs[z] == nullptr || ys[z] == nullptr) return CE_ERR_INVALID_ARG;
    if (lts[z] < 0 || lhs[z] < 0 || !disjoint(T, hs[z], lts[z], lhs[z], D)) return CE_ERR_INVALID_ARG;
    if (!aligned16(xs[z]) || !aligned16(ys[z]) || (lts[z] * es) % 16 || (lhs[z] * es) % 16)
      return CE_ERR_UNSUPPORTED;
    const int64_t extent = ((hs[z] - 1) * lhs[z] + D) * es;  // one token's heads, from its base
    if (extent >= ((int64_t)1 << 31)) return CE_ERR_UNSUPPORTED;
    a.bytes[z] = (uint32_t)extent;
  }
  a.pos = positions;
  a.D = (int)D;
  a.log2_base = log2(base);
  a.inverse = inverse;
  hipStream_t st = (hipStream_t)stream;
  if (dtype == CE_DTYPE_BF16)
    hipLaunchKernelGGL(rope16<BF16>, dim3((unsigned)T), dim3(64), 0, st, a);
  else if (dtype == CE_DTYPE_F16)
    hipLaunchKernelGGL(rope16<F16>, dim3((unsigned)T), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL(rope32, dim3((unsigned)T), dim3(64), 0, st, a);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

}  // extern "C"
