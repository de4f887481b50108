// ce_linear.hip -- LM-head projection followed by the token-mean softmax
// cross-entropy, forward and backward (the C ABI in include/ce_mi355x.h:
// ce_linear_workspace_bytes, ce_linear_fwd_bwd).
//
// The pages compare the plain cross-entropy kernel with a fused linear
// cross-entropy (PyPI page "fms-acceleration-foak 0.7.4", "Running Liger
// Kernel Benchmarks"), list fused cross-entropy among the kernels to come
// (fms-hf-tuning PR #280, "Notes on FastKernels") and leave a chunked loss as
// a to-do (fms-acceleration PR #79, "TODO").  With hidden states h [N, H] and
// the weight W [V, H] of a bias-free linear layer, logits = h W^T, and
//   dL/dh = g W,   dL/dW = g^T h,   g = dloss * dL/dlogits.
//
// bf16 / fp16 (all three products on the matrix cores, lin_gemm.h):
//   1. prep: n_valid, the gradient scale s = dloss 2^k / n_valid (fp16 keeps
//      g in its normal range through 2^k, k = 14 - ilogb(dloss / n); bf16
//      k = 0), and a new epoch tag for the call.
//   2. logits + cross-entropy, cooperative, in chunks of rows: each
//      workgroup holds one 256 x 256 logits tile in its fp32 accumulators, so
//      no logits ever reach memory.  From the registers it takes per row the
//      tile's (max, sum of exp without the label column), publishes them as
//      epoch-tagged words, merges the rows it owns (every tile of a row is
//      resident at once: the chunk's grid is sized to be co-resident and
//      launched cooperatively), publishes lse and 1 - p_y, and then writes
//      the gradient tile g = s (softmax - onehot) in the input format straight
//      from its accumulators -- the per-chunk log-sum-exp merge of a chunked
//      loss, done across workgroups.
//   3. dh = g W        MFMA, g K-contiguous, W read K-outer (transposed on its
//                      way into LDS); scaled by 2^-k on output
//   4. dW = g^T h      MFMA, both read K-outer; scaled by 2^-k on output
//   5. the token mean over the batch, summed in row order in fp64.
// The workspace holds g (N x V in the input format) and the small tagged
// exchange arrays; no fp32 logits and no transposed copies.
//
// fp32 inputs: the same steps with a plain tiled fp32 GEMM (no MFMA) and the
// chunk's fp32 logits in the workspace, reduced by the cross-entropy kernels
// of ce_api.hip in place; dW accumulates in the output.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "ce_mi355x.h"
#include "lin_gemm.h"

namespace {

using lg::f32x16;
using lg::Tile;

constexpr int kNT = 1024;               // prep / finish kernels
constexpr int64_t kMaxChunks = 4096;    // per-chunk counts live in LDS (fp32 path)
constexpr int64_t kF32ChunkRows = 1024;  // fp32 path default
constexpr int kSpinLimit = 1 << 20;      // polls before an exchange wait gives up
constexpr uint32_t kStatusLabelRange = 0x1u, kStatusSyncTimeout = 0x2u;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int esize(int dtype) { return dtype == CE_DTYPE_F32 ? 4 : 2; }
bool valid_dtype(int d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16 || d == CE_DTYPE_F16; }
bool fits32(int64_t x) { return x >= 0 && x < ((int64_t)1 << 31); }

// ---------------------------------------------------------------------------
// Workspace of the 16-bit path.
// ---------------------------------------------------------------------------
struct LinHeader {
  uint32_t epoch;   // bumped by prep: this call's tag
  uint32_t status;  // status bits of this call (cleared by prep)
  float gscale;     // s = dloss 2^k / n_valid
  float unscale;    // 2^-k
  int32_t n_valid;
  uint32_t pad[59];
};
static_assert(sizeof(LinHeader) == 256, "header size");

struct FastLayout {
  size_t g, stats, xy, lse, pc, total;
  int64_t ldg;    // g's row stride: vocab rounded up to 8 elements
  int nvt;        // vocabulary tiles of 256
  int rt_chunk;   // row tiles per chunk
  int nchunks;
};

// Row tiles per cooperative chunk: every tile of the chunk resident at once.
FastLayout fast_layout(int64_t N, int64_t V, int64_t resident) {
  FastLayout L;
  memset(&L, 0, sizeof(L));
  L.ldg = (V + 7) / 8 * 8;
  L.nvt = (int)((V + 255) / 256);
  const int64_t rt_total = (N + 255) / 256;
  int64_t rc = resident / L.nvt;
  if (rc < 1) rc = 1;
  if (rc > rt_total) rc = rt_total > 0 ? rt_total : 1;
  L.rt_chunk = (int)rc;
  L.nchunks = (int)((rt_total + rc - 1) / rc);
  size_t off = sizeof(LinHeader);
  L.g = align256(off);
  off = L.g + align256((size_t)N * L.ldg * 2);
  L.stats = off;  // [chunk][row in chunk][vocab tile] x 2 tagged words
  off += align256((size_t)(L.nchunks > 0 ? L.nchunks : 1) * rc * 256 * L.nvt * 16);
  L.xy = off;
  off += align256((size_t)N * 8);
  L.lse = off;
  off += align256((size_t)N * 8);
  L.pc = off;
  off += align256((size_t)N * 8);
  L.total = off;
  return L;
}

// Co-resident workgroups of the 16-bit logits kernel: one per CU (its LDS
// and accumulator registers fill a CU).  Taken as the device's CU count.
int64_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

// ---------------------------------------------------------------------------
// Tagged exchange words: tag << 32 | float bits, one relaxed agent-scope
// 64-bit store / load each (the reader polls until the tag is this call's).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void put_tagged(uint64_t* p, uint32_t tag, float v) {
  __hip_atomic_store(p, ((uint64_t)tag << 32) | __builtin_bit_cast(uint32_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}
// Polls *p until it carries `tag`; on timeout returns NaN and sets *to.
__device__ __forceinline__ float get_tagged(const uint64_t* p, uint32_t tag, uint32_t& to) {
  for (int it = 0;; ++it) {
    const uint64_t w = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((uint32_t)(w >> 32) == tag) return __builtin_bit_cast(float, (uint32_t)w);
    if (to || it >= kSpinLimit) {
      to = 1;
      return __builtin_nanf("");
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// A tagged word's load, and its value once loaded (polled for when the word
// is not yet this call's): a thread issues all its loads before it checks
// any, so the exchange costs one round trip rather than one per word.
__device__ __forceinline__ uint64_t ld_tagged(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float tagged_value(uint64_t w, const uint64_t* p, uint32_t tag, uint32_t& to) {
  if ((uint32_t)(w >> 32) == tag) return __builtin_bit_cast(float, (uint32_t)w);
  return get_tagged(p, tag, to);
}

// Whole-wave max / sum (every lane gets the result; fixed order).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

template <typename T>
__device__ __forceinline__ uint16_t to_bits(float x);
template <>
__device__ __forceinline__ uint16_t to_bits<__bf16>(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <>
__device__ __forceinline__ uint16_t to_bits<_Float16>(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// 1. prep (one workgroup): n_valid, the scale, the epoch; for the fp32 path
// also each chunk's dloss share.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kNT) void lin_prep_kernel(const int64_t* labels, int64_t N, int64_t ignore, int64_t T,
                                                       int nc, const float* dloss, int fp16_range, LinHeader* hdr,
                                                       float* dl_chunk, int32_t* n_valid_out) {
  __shared__ int32_t cnt[kMaxChunks];
  __shared__ int64_t wsum[kNT / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int c = tid; c < nc; c += kNT) cnt[c] = 0;
  __syncthreads();
  for (int64_t base = 0; base < N; base += kNT) {
    const int64_t i = base + tid;
    const bool v = i < N && labels[i] != ignore;
    const uint64_t ballot = __ballot(v);
    // T is a multiple of 64: a wave's labels fall in one chunk
    if (lane == 0 && ballot && dl_chunk) atomicAdd(&cnt[(int)(i / T)], (int32_t)__popcll(ballot));
    if (lane == 0 && ballot && !dl_chunk) atomicAdd(&cnt[0], (int32_t)__popcll(ballot));
  }
  __syncthreads();
  int64_t s = 0;
  for (int c = tid; c < (dl_chunk ? nc : 1); c += kNT) s += cnt[c];
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  if (lane == 0) wsum[tid >> 6] = s;
  __syncthreads();
  int64_t n = 0;
  for (int w = 0; w < kNT / 64; ++w) n += wsum[w];
  const double dl = dloss ? (double)dloss[0] : 1.0;
  int k = 0;
  if (fp16_range && n > 0) {
    const double sc = fabs(dl / (double)n);
    if (sc > 0.0 && sc < 1e300) {
      k = 14 - ilogb(sc);
      k = k < -100 ? -100 : (k > 100 ? 100 : k);
    }
  }
  const double up = ldexp(1.0, k);
  if (dl_chunk)
    for (int c = tid; c < nc; c += kNT) dl_chunk[c] = n > 0 ? (float)(dl * up * (double)cnt[c] / (double)n) : 0.0f;
  if (tid == 0) {
    n_valid_out[0] = (int32_t)n;
    if (hdr) {
      hdr->epoch = hdr->epoch + 1u;
      hdr->status = 0u;
      hdr->gscale = n > 0 ? (float)(dl * up / (double)n) : 0.0f;
      hdr->unscale = (float)ldexp(1.0, -k);
      hdr->n_valid = (int32_t)n;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. logits tile + cross-entropy epilogue (16-bit; cooperative launches over
// chunks of row tiles).  Grid: rt x nvt workgroups in the XCD order, so the
// row tiles that share a weight slab run on one XCD.
// ---------------------------------------------------------------------------
struct LogitsArgs {
  const char* h;
  int64_t ldh;
  const char* w;
  int64_t ldw;
  const int64_t* labels;
  int64_t ignore;
  int64_t N, H, V;
  int64_t row0;  // first row of this chunk
  int rtc;       // row tiles in this chunk
  int nvt;
  int rt_chunk, nchunks, rt_total;  // row tiles per chunk, chunks, row tiles in all
  LinHeader* hdr;
  uint16_t* g;
  int64_t ldg;
  uint64_t* stats;  // this chunk's [rtc * 256][nvt][2] (every chunk's in the one-launch form)
  uint64_t* xy;     // [N]
  uint64_t* lse;    // [N]
  uint64_t* pc;     // [N]
  float* loss_rows;
};

// LDS: the K loop's stages (128 KB or 64 KB), then the epilogue's statistics
// (16 KB + a 72 KB transpose area) and four staged 128 x 136 gradient
// quarters (136 KB) at offset 16 KB: all of a CU's 160 KB.
constexpr int kLogitsLds = 160 * 1024;
static_assert(16384 + 4 * 128 * 136 * 2 <= kLogitsLds, "staged gradient quarters");
static_assert(16384 + 256 * 65 * 4 <= kLogitsLds, "statistics transpose");

// Row of accumulator element v of 32-row block i within a lane's rows (the
// lane's first row is wm * 128 + 4 * (lane / 32); see lg::acc_row).
__device__ constexpr int kRowOff(int i, int v) { return i * 32 + 8 * (v >> 2) + (v & 3); }
// Tiles per lane and round of the row merge (128 tiles a round).
constexpr int kMergeQ = 2;

template <typename T, bool DMA, int AK, int BKD>
// One tile of one chunk: workgroup blockIdx.x of a grid of rtg x nvt takes
// tile (rt, vt) of the chunk (none when rt is past the chunk's rtc row tiles).
// tid is the thread index (opaque to the compiler in the one-launch loop).
__device__ __forceinline__ void logits_ce_tile(const LogitsArgs& a, char* lds, int tid, int rtg) {
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), wm = wave >> 1, wn = wave & 1;
  // the row tiles that share a weight slab are neighbours in the XCD order,
  // so they run on one XCD and the slab is fetched into its L2 once
  const int lin = lg::xcd_order((int)blockIdx.x, rtg * a.nvt);
  const int rt = lin % rtg, vt = lin / rtg;
  if (rt >= a.rtc) return;  // the last chunk may have fewer row tiles
  const int64_t mrow0 = a.row0 + (int64_t)rt * 256;  // the tile's first row (global)
  const int n0 = vt * 256;
  const int M = (int)a.N, Nv = (int)a.V, K = (int)a.H;
  Tile t;
  if constexpr (DMA) lg::tile_nt<T>(t, lds, a.h, a.ldh, a.w, a.ldw, M, Nv, K, (int)mrow0, n0, tid);
  else lg::tile_rs<T, AK, BKD>(t, lds, a.h, a.ldh, a.w, a.ldw, M, Nv, K, (int)mrow0, n0);
  const uint32_t tag = a.hdr->epoch;
  const float gs = a.hdr->gscale;
  __syncthreads();  // every wave is done with the K loop's LDS

  // LDS after the K loop: per-row label data and statistics, and a
  // [256][kPS] transpose area for the per-lane partials (kPS = 65 floats per
  // row: the row reductions, one thread per row, read without bank
  // conflicts; the half-waves' writes, four rows apart, overlap on 28 banks).  The
  // epilogue walks the accumulators one 32-row block (index i) at a time so
  // that only that block's row constants are held in registers.
  constexpr int kPS = 65;
  int64_t* ys = (int64_t*)lds;              // [256] labels of the tile's rows
  int32_t* yrel = (int32_t*)(lds + 2048);   // [256] label column - n0 when in this tile, else -1
  float* mrow = (float*)(lds + 3072);       // [256] the tile's row max
  float* xyl = (float*)(lds + 4096);        // [256 + 64] label logits found here (+ junk slots)
  float* mrowc = (float*)(lds + 6144);      // [256] the row max times log2 e (0 for -inf): the exponentials' shift
  float* crow = (float*)(lds + 7168);       // [256] s 2^(mrowc - lse log2 e): g = e crow on a row's off-label elements
  float* lrow = (float*)(lds + 10240);      // [256] lse of the tile's rows
  float* prow = (float*)(lds + 11264);      // [256] 1 - p_y
  uint32_t* sflag = (uint32_t*)(lds + 12288);
  float* part = (float*)(lds + 16384);      // [256][kPS]
  if (tid == 0) sflag[0] = 0u;
  {
    const int64_t R = mrow0 + tid;
    const int64_t y = (R < a.N) ? a.labels[R] : a.ignore;
    ys[tid] = y;
    yrel[tid] = (y != a.ignore && y >= n0 && y < n0 + 256 && y < a.V) ? (int)(y - n0) : -1;
  }
  __syncthreads();
  const int lc = wn * 128 + (lane & 31);  // this lane's column in block j: lc + 32 j
  bool cvalid[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) cvalid[j] = n0 + lc + 32 * j < Nv;
  // every column of the tile inside the vocabulary (all tiles but the last):
  // the passes below then take no per-element column test
  const bool full = n0 + 256 <= Nv;
  // this lane's slot of row acc_row(wm, i, v, lane) in the transpose area:
  // part_l[kRowOff(i, v) * kPS], a compile-time offset per (i, v)
  float* part_l = part + (wm * 128 + 4 * (lane >> 5)) * kPS + wn * 32 + (lane & 31);
  // pass A: per lane and row the max over its four columns, through LDS to
  // one thread per row
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m[16];
    if (full) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        m[v] = fmaxf(fmaxf(t.acc[i][0][v], t.acc[i][1][v]), fmaxf(t.acc[i][2][v], t.acc[i][3][v]));
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) m[v] = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16 blk = t.acc[i][j];
#pragma unroll
        for (int v = 0; v < 16; ++v) m[v] = fmaxf(m[v], cvalid[j] ? blk[v] : -INFINITY);
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) part_l[kRowOff(i, v) * kPS] = m[v];
  }
  __syncthreads();
  {
    const float* pr = part + tid * kPS;
    float m = pr[0];
#pragma unroll 8
    for (int q = 1; q < 64; ++q) m = fmaxf(m, pr[q]);
    mrow[tid] = m;
    mrowc[tid] = (m == -INFINITY) ? 0.0f : m * kLog2e;
  }
  __syncthreads();
  // pass B: e = 2^(x log2 e - mc) for every element, written over its
  // logit in the accumulators (the gradient pass multiplies it by the row's
  // constant instead of taking a second exponential), and per lane and row
  // the label-excluded sum of its four.  For a row whose label lies in some
  // lane's columns (a ballot per row, rarely true) the lane that holds it
  // takes out the label's logit (into xyl) and sets its e to 0; no other
  // row pays a per-element label test.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = lg::acc_row(wm, i, v, lane);
      const float mc = mrowc[r];
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(t.acc[i][j][v], kLog2e, -mc));
        if (!full) e[j] = cvalid[j] ? e[j] : 0.0f;
      }
      const int d = yrel[r] - lc;         // the label's column is this lane's in block d / 32
      const bool own = (d & ~0x60) == 0;  // d in {0, 32, 64, 96}
      if (__ballot(own) != 0) {
        float xv = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bool hit = own && (d >> 5) == j;
          xv = hit ? t.acc[i][j][v] : xv;
          e[j] = hit ? 0.0f : e[j];
        }
        if (own) xyl[r] = xv;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) t.acc[i][j][v] = e[j];
      sv[v] = (e[0] + e[1]) + (e[2] + e[3]);
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) part_l[kRowOff(i, v) * kPS] = sv[v];
  }
  __syncthreads();
  {
    const int r = tid;
    const float* pr = part + r * kPS;
    float S = 0.0f;
#pragma unroll 8
    for (int q = 0; q < 64; ++q) S += pr[q];
    if (mrow0 + r < a.N) {
      uint64_t* sp = a.stats + ((size_t)(rt * 256 + r) * a.nvt + vt) * 2;
      put_tagged(sp, tag, mrow[r]);
      put_tagged(sp + 1, tag, S);
      if (yrel[r] >= 0) put_tagged(a.xy + mrow0 + r, tag, xyl[r]);
    }
  }

  // rows r = vt, vt + nvt, ... of this row tile are merged here, one wave per
  // row: its lanes fetch the nvt tiles' (max, sum) words (all loads issued
  // before any is waited on), merge their own, and the wave merges the lanes
  uint32_t to = 0;
  for (int k = wave;; k += 4) {
    const int r = vt + k * a.nvt;
    if (r >= 256 || mrow0 + r >= a.N) break;
    const int64_t R = mrow0 + r, y = ys[r];
    float loss = 0.0f;
    if (y != a.ignore) {
      if (y < 0 || y >= a.V) {
        loss = __builtin_nanf("");
      } else {
        const uint64_t* sp = a.stats + (size_t)(rt * 256 + r) * a.nvt * 2;
        const uint64_t wxy = ld_tagged(a.xy + R);
        float ml = -INFINITY, sl = 0.0f;  // this lane's running (max, sum)
        for (int v0 = 0; v0 < a.nvt; v0 += 64 * kMergeQ) {
          uint64_t wm_[kMergeQ], ws_[kMergeQ];
#pragma unroll
          for (int q = 0; q < kMergeQ; ++q) {
            const int v2 = v0 + lane + 64 * q;
            if (v2 < a.nvt) {
              wm_[q] = ld_tagged(sp + v2 * 2);
              ws_[q] = ld_tagged(sp + v2 * 2 + 1);
            }
          }
#pragma unroll
          for (int q = 0; q < kMergeQ; ++q) {
            const int v2 = v0 + lane + 64 * q;
            if (v2 < a.nvt) {
              const float mv = tagged_value(wm_[q], sp + v2 * 2, tag, to);
              const float sv = tagged_value(ws_[q], sp + v2 * 2 + 1, tag, to);
              if (mv != -INFINITY) {
                const float mn = fmaxf(ml, mv);
                sl = ((ml == -INFINITY) ? 0.0f : sl * __builtin_amdgcn_exp2f((ml - mn) * kLog2e)) +
                     sv * __builtin_amdgcn_exp2f((mv - mn) * kLog2e);
                ml = mn;
              }
            }
          }
        }
        const float Mx = wave_max(ml);
        const float S = wave_sum((ml == -INFINITY) ? 0.0f : sl * __builtin_amdgcn_exp2f((ml - Mx) * kLog2e));
        const float xy = tagged_value(wxy, a.xy + R, tag, to);
        const float ey = __builtin_amdgcn_exp2f((xy - Mx) * kLog2e);
        const float St = S + ey;
        const float l = Mx + logf(St), pcomp = S / St;
        loss = (pcomp >= 0.5f) ? (l - xy) : log1pf(S / ey);
        if (lane == 0) {
          put_tagged(a.lse + R, tag, l);
          put_tagged(a.pc + R, tag, pcomp);
        }
      }
    }
    if (lane == 0) a.loss_rows[R] = loss;
  }
  // every row of the tile: its lse and 1 - p_y
  {
    const int r = tid;
    const int64_t R = mrow0 + r, y = ys[r];
    float l = 0.0f, pcv = 0.0f;
    if (R < a.N && y != a.ignore && y >= 0 && y < a.V) {
      const uint64_t wl = ld_tagged(a.lse + R), wp = ld_tagged(a.pc + R);
      l = tagged_value(wl, a.lse + R, tag, to);
      pcv = tagged_value(wp, a.pc + R, tag, to);
    }
    lrow[r] = l;
    prow[r] = pcv;
    crow[r] = gs * __builtin_amdgcn_exp2f(mrowc[r] - l * kLog2e);
  }
  if (to) atomicOr(sflag, 1u);
  __syncthreads();
  if (tid == 0 && sflag[0]) atomicOr(&a.hdr->status, kStatusSyncTimeout);
  const bool bad_scale = sflag[0] != 0u;

  // g from the accumulators (which now hold e = 2^(x log2 e - mc)):
  // s 2^((x - lse) log2 e) = e crow off the label, -s (1 - p_y) on it, +0 on
  // ignored rows and past the vocabulary, NaN on rows with a label outside
  // [0, V).  Each wave stages its 128 x 128 quarter in LDS (rows of 272
  // bytes) and writes it out as 16-byte vectors.
  constexpr int kGS = 136;  // staged row stride in elements
  __syncthreads();  // the statistics area is free
  uint16_t* stg = (uint16_t*)(lds + 16384 + wave * (128 * kGS * 2));
  // The common case (a full tile, every exchange in time) writes e crow
  // everywhere, then fixes up the few special elements: the label's,
  // ignored rows (+0) and rows with a bad label (NaN).
  const bool fast = full && !bad_scale;
  const int64_t cbase = (int64_t)n0 + wn * 128;
  if (fast) {
    uint16_t* stg_l = stg + 4 * (lane >> 5) * kGS + (lane & 31);  // + kRowOff(i, v) * kGS + 32 j
    const uint32_t nanb = to_bits<T>(__builtin_nanf("")), nan2 = (nanb << 16) | nanb;
    // 32 rows of the quarter at a time: computed, fixed up and stored, so the
    // stores of one block overlap the arithmetic of the next
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cr[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) cr[v] = crow[lg::acc_row(wm, i, v, lane)];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16 blk = t.acc[i][j];
#pragma unroll
        for (int v = 0; v < 16; ++v) stg_l[kRowOff(i, v) * kGS + 32 * j] = to_bits<T>(blk[v] * cr[v]);
      }
      // fix-ups of rows 32 i .. 32 i + 31, after this wave's own staged
      // writes (LDS keeps a wave's order): the label's element, ignored rows
      // (+0), rows with a bad label (NaN)
      {
        const int rq = i * 32 + (lane & 31), r = wm * 128 + rq;
        const int64_t y = ys[r];
        const bool ign = (y == a.ignore), bad = !ign && (y < 0 || y >= a.V);
        const uint64_t zb = __ballot(lane < 32 && ign), nb = __ballot(lane < 32 && bad);
        const int d = yrel[r] - wn * 128;  // the label's column in this quarter
        if (lane < 32 && !ign && !bad && d >= 0 && d < 128) stg[rq * kGS + d] = to_bits<T>(-gs * prow[r]);
        for (uint64_t b = zb; b; b &= b - 1) ((uint32_t*)(stg + (i * 32 + __builtin_ctzll(b)) * kGS))[lane] = 0u;
        for (uint64_t b = nb; b; b &= b - 1) ((uint32_t*)(stg + (i * 32 + __builtin_ctzll(b)) * kGS))[lane] = nan2;
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (it reads only its own quarter)
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rr = i * 32 + q * 4 + (lane >> 4), cv = (lane & 15) * 8;
        const int64_t R = mrow0 + wm * 128 + rr;
        const int64_t c = cbase + cv;
        if (R < a.N && c < a.ldg) {
          const lg::u32x4 val = *(const lg::u32x4*)(stg + rr * kGS + cv);
          *(lg::u32x4*)(a.g + R * a.ldg + c) = val;
        }
      }
    }
    return;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float cr[16], gyv[16];
      int lj[16], kind[16];  // kind: 0 normal, 1 zero (ignored row), 2 NaN (bad label or failed exchange)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = lg::acc_row(wm, i, v, lane);
        const int64_t y = ys[r];
        const bool ign = (y == a.ignore), bad = !ign && (y < 0 || y >= a.V);
        kind[v] = ign ? 1 : ((bad || bad_scale) ? 2 : 0);
        cr[v] = crow[r];
        gyv[v] = -gs * prow[r];
        const int d = yrel[r] - lc;
        lj[v] = (d >= 0 && d < 128 && (d & 31) == 0) ? (d >> 5) : -1;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16 blk = t.acc[i][j];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float gv = blk[v] * cr[v];
          gv = (lj[v] == j) ? gyv[v] : gv;
          gv = (kind[v] == 2) ? __builtin_nanf("") : gv;
          gv = (kind[v] == 1 || !cvalid[j]) ? 0.0f : gv;
          const int r = lg::acc_row(wm, i, v, lane);
          stg[(r - wm * 128) * kGS + (lc - wn * 128) + 32 * j] = to_bits<T>(gv);
        }
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (it reads only its own quarter)
  // 128 rows x 16 vectors of the quarter: four rows per pass of the wave
#pragma unroll 4
  for (int q = 0; q < 32; ++q) {
    const int rr = q * 4 + (lane >> 4), cv = (lane & 15) * 8;
    const int64_t R = mrow0 + wm * 128 + rr;
    const int64_t c = cbase + cv;
    if (R < a.N && c < a.ldg) {
      const lg::u32x4 val = *(const lg::u32x4*)(stg + rr * kGS + cv);
      *(lg::u32x4*)(a.g + R * a.ldg + c) = val;
    }
  }
}

// The direct-to-LDS form walks every chunk in one cooperative launch: each
// workgroup takes tile (rt, vt) of chunk 0, 1, ... in turn.  The row tiles of
// a chunk exchange their statistics through slots of their own and every
// workgroup walks the chunks in the same order, so the waits of chunk c only
// involve workgroups that reach chunk c.  (One cooperative launch per chunk
// leaves the GPU idle ~19 us between chunks.)  The element-wise form, which
// the compiler cannot keep free of spills in the loop, launches per chunk.
template <typename T, bool DMA, int AK, int BKD>
__global__ __launch_bounds__(256, 1) void lin_logits_ce_kernel(LogitsArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  if constexpr (DMA) {
    uint64_t* stats0 = a.stats;
    for (int c = 0; c < a.nchunks; ++c) {
      LogitsArgs ac = a;
      ac.row0 = (int64_t)c * a.rt_chunk * 256;
      ac.rtc = min(a.rt_chunk, a.rt_total - c * a.rt_chunk);
      ac.stats = stats0 + (size_t)c * a.rt_chunk * 256 * a.nvt * 2;
      // a thread index the compiler cannot see through, so nothing
      // lane-dependent is hoisted out of this loop and held across a tile
      int tid = (int)threadIdx.x;
      asm volatile("" : "+v"(tid));
      logits_ce_tile<T, DMA, AK, BKD>(ac, lds, tid, a.rt_chunk);
      __syncthreads();  // the LDS is free for the next chunk's K loop
    }
  } else {
    logits_ce_tile<T, DMA, AK, BKD>(a, lds, (int)threadIdx.x, a.rtc);
  }
}

// ---------------------------------------------------------------------------
// 3-4. dh = g W and dW = g^T h (16-bit): MFMA tiles, 2^-k on output.
// ---------------------------------------------------------------------------
// LDS of the direct-to-LDS backward kernels: the K loop's stages, then the
// epilogue's four 128 x 136 staged quarters
constexpr int kBwdLds = (lg::kLdsBytes > 4 * 128 * 136 * 2) ? lg::kLdsBytes : 4 * 128 * 136 * 2;

struct BwdArgs {
  const char* A;
  int64_t lda;
  const char* B;
  int64_t ldb;
  int M, N, K;
  int Mx, Nx;  // loadable extents along M / N (at least M / N)
  uint16_t* C;
  int64_t ldc;
  int vec_out;  // C 16-byte aligned, ldc and N multiples of 8
  const LinHeader* hdr;
};

// DMA: both operands through direct-to-LDS loads (16-byte aligned rows;
// a.Mx / a.Nx bound the 16-byte chunks a KO operand may load), kLdsBytes of
// LDS; otherwise the register-staged loop, 2 kStageBytes.
template <typename T, int AK, int BKD, bool DMA>
__global__ __launch_bounds__(256, 1) void lin_bwd_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int mt = (a.M + 255) / 256, nt = (a.N + 255) / 256;
  int mti, nti;
  // g (the A operand of both products) is the larger operand: its tiles are
  // shared within an XCD
  lg::tile_of_rows(blockIdx.x, mt, nt, mti, nti);
  const int m0 = mti * 256, n0 = nti * 256;
  Tile t;
  if constexpr (DMA) lg::tile_dma<T, AK, BKD>(t, lds, a.A, a.lda, a.B, a.ldb, a.Mx, a.Nx, a.K, m0, n0);
  else lg::tile_rs<T, AK, BKD>(t, lds, a.A, a.lda, a.B, a.ldb, a.M, a.N, a.K, m0, n0);
  const float us = a.hdr->unscale;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  if constexpr (DMA) {
    // Each wave stages its 128 x 128 quarter in LDS (rows of 272 bytes) and
    // writes it out as 16-byte vectors (8 elements; a.vec_out: C 16-byte
    // aligned with whole vectors per row), else element by element.
    constexpr int kGS = 136;
    __syncthreads();  // every wave is done with the K loop's LDS
    uint16_t* stg = (uint16_t*)(lds + wave * (128 * kGS * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          stg[lg::acc_row(0, i, v, lane) * kGS + lg::acc_col(0, j, lane)] = to_bits<T>(t.acc[i][j][v] * us);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (it reads only its own quarter)
    const int cb = n0 + wn * 128;
#pragma unroll 4
    for (int q = 0; q < 32; ++q) {
      const int rr = q * 4 + (lane >> 4), cv = (lane & 15) * 8;
      const int R = m0 + wm * 128 + rr, c = cb + cv;
      if (R >= a.M || c >= a.N) continue;
      uint16_t* dst = a.C + (int64_t)R * a.ldc + c;
      const uint16_t* src = stg + rr * kGS + cv;
      if (a.vec_out) {
        *(lg::u32x4*)dst = *(const lg::u32x4*)src;
      } else {
        for (int e = 0; e < 8 && c + e < a.N; ++e) dst[e] = src[e];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = m0 + lg::acc_row(wm, i, v, lane);
      if (r >= a.M) continue;
      uint16_t* crow = a.C + (int64_t)r * a.ldc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int c = n0 + lg::acc_col(wn, j, lane);
        if (c < a.N) crow[c] = to_bits<T>(t.acc[i][j][v] * us);
      }
    }
}

// ---------------------------------------------------------------------------
// fp32 path: a plain tiled GEMM (64 x 64 tiles, 4 x 4 outputs per lane,
// fp32 FMA), element-wise loads of either operand layout:
//   C[m][n] = alpha sum_k A(m, k) B(n, k) + beta C[m][n]
//   A(m, k) = A[m lda + k] (AKO = 0) or A[k lda + m] (AKO = 1); B likewise.
// ---------------------------------------------------------------------------
template <bool AKO, bool BKO>
__global__ __launch_bounds__(256) void lin_gemm_f32_kernel(const float* A, int64_t lda, const float* B, int64_t ldb,
                                                           int M, int N, int K, float alpha, float beta, float* C,
                                                           int64_t ldc) {
  __shared__ float As[16][65], Bs[16][65];
  const int tid = threadIdx.x, tm = tid / 16, tn = tid % 16;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int e = tid; e < 16 * 64; e += 256) {
      const int kk = AKO ? e / 64 : e % 16, mm = AKO ? e % 64 : e / 16;
      const int m = m0 + mm, k = k0 + kk;
      As[kk][mm] = (m < M && k < K) ? (AKO ? A[(int64_t)k * lda + m] : A[(int64_t)m * lda + k]) : 0.0f;
      const int kb = BKO ? e / 64 : e % 16, nn = BKO ? e % 64 : e / 16;
      const int n = n0 + nn, kq = k0 + kb;
      Bs[kb][nn] = (n < N && kq < K) ? (BKO ? B[(int64_t)kq * ldb + n] : B[(int64_t)n * ldb + kq]) : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = __builtin_fmaf(As[kk][tm * 4 + x], Bs[kk][tn * 4 + y], acc[x][y]);
    __syncthreads();
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) {
      const int m = m0 + tm * 4 + x, n = n0 + tn * 4 + y;
      if (m < M && n < N) {
        float* c = C + (int64_t)m * ldc + n;
        *c = alpha * acc[x][y] + (beta != 0.0f ? beta * *c : 0.0f);
      }
    }
}

// ---------------------------------------------------------------------------
// Shared small kernels.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void lin_zero_kernel(uint16_t* dst, int64_t ld, int64_t cols, int esz) {
  if (esz == 4) {
    float* d = (float*)dst + (int64_t)blockIdx.x * ld;
    for (int64_t j = threadIdx.x; j < cols; j += 256) d[j] = 0.0f;
  } else {
    uint16_t* d = dst + (int64_t)blockIdx.x * ld;
    for (int64_t j = threadIdx.x; j < cols; j += 256) d[j] = 0;
  }
}

// One workgroup: L = sum of the valid rows' losses / n, in row order (each
// lane a contiguous slice, then a fixed tree), fp64; status from the labels
// (a label outside [0, V)), the exchange's status word and the fp32 path's
// per-chunk words.
__global__ __launch_bounds__(kNT) void lin_finish_kernel(const float* loss_rows, const int64_t* labels, int64_t N,
                                                         int64_t V, int64_t ignore, const int32_t* n_valid,
                                                         const uint32_t* chunk_status, int nc,
                                                         const LinHeader* hdr, float* loss_mean, uint32_t* status) {
  __shared__ double acc[kNT];
  __shared__ uint32_t st[kNT];
  const int tid = threadIdx.x;
  const int64_t i0 = N * tid / kNT, i1 = N * (tid + 1) / kNT;
  double a = 0.0;
  uint32_t s = 0;
  for (int64_t i = i0; i < i1; ++i) {
    const int64_t y = labels[i];
    if (y != ignore) {
      a += (double)loss_rows[i];
      if (y < 0 || y >= V) s |= kStatusLabelRange;
    }
  }
  if (chunk_status)
    for (int c = tid; c < nc; c += kNT) s |= chunk_status[c];
  acc[tid] = a;
  st[tid] = s;
  __syncthreads();
  for (int w = kNT / 2; w >= 1; w >>= 1) {
    if (tid < w) {
      acc[tid] += acc[tid + w];
      st[tid] |= st[tid + w];
    }
    __syncthreads();
  }
  if (tid == 0) {
    const uint32_t sw = st[0] | (hdr ? hdr->status : 0u);
    loss_mean[0] = (sw & kStatusSyncTimeout) ? __builtin_nanf("") : (float)(acc[0] / (double)n_valid[0]);
    if (status) status[0] = sw;
  }
}

__global__ __launch_bounds__(256) void lin_fill_kernel(uint32_t* p, size_t n_words) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n_words; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

__global__ void lin_empty_kernel(float* loss_mean, int32_t* n_valid, uint32_t* status) {
  if (threadIdx.x == 0) {
    loss_mean[0] = __builtin_nanf("");
    n_valid[0] = 0;
    if (status) status[0] = 0u;
  }
}

// ---------------------------------------------------------------------------
// fp32 path layout: the chunk's fp32 logits (the gradient is written over
// them), the cross-entropy workspace, per-chunk words.
// ---------------------------------------------------------------------------
struct F32Layout {
  size_t ce_ws, logits, dl_chunk, chunk_status, chunk_loss, chunk_n, total;
  size_t ce_ws_bytes;
  int64_t T;
  int nc;
};
F32Layout f32_layout(int64_t N, int64_t V, int64_t chunk_rows) {
  F32Layout L;
  memset(&L, 0, sizeof(L));
  int64_t t = chunk_rows > 0 ? chunk_rows : kF32ChunkRows;
  const int64_t min_t = (N + kMaxChunks - 1) / kMaxChunks;
  if (t < min_t) t = min_t;
  L.T = (t + 63) / 64 * 64;
  L.nc = (int)((N + L.T - 1) / L.T);
  const int64_t Tc = (N < L.T) ? (N > 0 ? N : 1) : L.T;
  L.ce_ws_bytes = ce_workspace_bytes(Tc, V, 0, CE_DTYPE_F32);
  size_t off = sizeof(LinHeader);
  L.ce_ws = align256(off);
  off = L.ce_ws + align256(L.ce_ws_bytes);
  L.logits = off;
  off += align256((size_t)Tc * V * 4);
  const size_t nc = (size_t)(L.nc > 0 ? L.nc : 1);
  L.dl_chunk = off;
  off += align256(nc * 4);
  L.chunk_status = off;
  off += align256(nc * 4);
  L.chunk_loss = off;
  off += align256(nc * 4);
  L.chunk_n = off;
  off += align256(nc * 4);
  L.total = off;
  return L;
}

bool aligned16(const void* p, int64_t ld, int es) { return ((uintptr_t)p % 16 == 0) && ((ld * es) % 16 == 0); }

template <typename K>
int set_lds(K* fn, int bytes) {
  return hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess
             ? CE_OK
             : CE_ERR_HIP;
}

// The 16-bit path (T = __bf16 or _Float16).
template <typename T>
int run_fast(const void* hidden, int64_t ldh, const void* weight, int64_t ldw, const int64_t* labels, int64_t N,
             int64_t H, int64_t V, int64_t ignore, const float* dloss, float* loss_mean, float* loss_rows,
             int32_t* n_valid, uint32_t* status, void* gh, int64_t ldgh, void* gw, int64_t ldgw, char* ws,
             const FastLayout& L, bool fp16, hipStream_t st) {
  LinHeader* hdr = (LinHeader*)ws;
  uint16_t* g = (uint16_t*)(ws + L.g);
  hipLaunchKernelGGL(lin_prep_kernel, dim3(1), dim3(kNT), 0, st, labels, N, ignore, (int64_t)64, 1, dloss,
                     fp16 ? 1 : 0, hdr, (float*)nullptr, n_valid);
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  // fast operand loads need 16-byte rows and a hidden size of whole 16-byte chunks
  const bool fast = aligned16(hidden, ldh, 2) && aligned16(weight, ldw, 2) && H % 8 == 0;
  LogitsArgs la;
  la.h = (const char*)hidden;
  la.ldh = ldh;
  la.w = (const char*)weight;
  la.ldw = ldw;
  la.labels = labels;
  la.ignore = ignore;
  la.N = N;
  la.H = H;
  la.V = V;
  la.nvt = L.nvt;
  la.hdr = hdr;
  la.g = g;
  la.ldg = L.ldg;
  la.xy = (uint64_t*)(ws + L.xy);
  la.lse = (uint64_t*)(ws + L.lse);
  la.pc = (uint64_t*)(ws + L.pc);
  la.loss_rows = loss_rows;
  const int64_t rt_total = (N + 255) / 256;
  auto kfn = fast ? lin_logits_ce_kernel<T, true, lg::kKC, lg::kKC> : lin_logits_ce_kernel<T, false, lg::kKCg, lg::kKCg>;
  const int lds_bytes = kLogitsLds;
  if (set_lds(kfn, lds_bytes) != CE_OK) return CE_ERR_HIP;
  la.rt_chunk = L.rt_chunk;
  la.nchunks = L.nchunks;
  la.rt_total = (int)rt_total;
  if (fast) {
    la.row0 = 0;
    la.rtc = L.rt_chunk;
    la.stats = (uint64_t*)(ws + L.stats);
    void* params[] = {&la};
    if (hipLaunchCooperativeKernel((const void*)kfn, dim3((unsigned)(L.rt_chunk * L.nvt)), dim3(256), params, lds_bytes,
                                   st) != hipSuccess)
      return CE_ERR_HIP;
  } else {
    for (int c = 0; c < L.nchunks; ++c) {
      const int64_t rt0 = (int64_t)c * L.rt_chunk;
      const int rtc = (int)((rt_total - rt0 < L.rt_chunk) ? rt_total - rt0 : L.rt_chunk);
      la.row0 = rt0 * 256;
      la.rtc = rtc;
      la.stats = (uint64_t*)(ws + L.stats) + (size_t)c * L.rt_chunk * 256 * L.nvt * 2;
      void* params[] = {&la};
      if (hipLaunchCooperativeKernel((const void*)kfn, dim3((unsigned)(rtc * L.nvt)), dim3(256), params, lds_bytes,
                                     st) != hipSuccess)
        return CE_ERR_HIP;
    }
  }
  if (gh) {  // dh [N, H] = g [N, V] W [V, H]
    BwdArgs b;
    b.A = (const char*)g;
    b.lda = L.ldg;
    b.B = (const char*)weight;
    b.ldb = ldw;
    b.M = (int)N;
    b.N = (int)H;
    b.K = (int)V;
    b.Mx = (int)N;
    b.Nx = (int)H;
    b.C = (uint16_t*)gh;
    b.ldc = ldgh;
    b.vec_out = aligned16(gh, ldgh, 2) && H % 8 == 0;
    b.hdr = hdr;
    auto fn = fast ? lin_bwd_kernel<T, lg::kKC, lg::kKO, true> : lin_bwd_kernel<T, lg::kKC, lg::kKOg, false>;
    const int lb = fast ? kBwdLds : 2 * lg::kStageBytes;
    if (set_lds(fn, lb) != CE_OK) return CE_ERR_HIP;
    const int64_t grid = ((N + 255) / 256) * ((H + 255) / 256);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), lb, st, b);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  if (gw) {  // dW [V, H] = g^T h: A(v, tok) = g[tok][v], B(h, tok) = h[tok][h]
    BwdArgs b;
    b.A = (const char*)g;
    b.lda = L.ldg;
    b.B = (const char*)hidden;
    b.ldb = ldh;
    b.M = (int)V;
    b.N = (int)H;
    b.K = (int)N;
    b.Mx = (int)L.ldg;  // g's pad columns (zeros) up to its row stride may load
    b.Nx = (int)H;
    b.C = (uint16_t*)gw;
    b.ldc = ldgw;
    b.vec_out = aligned16(gw, ldgw, 2) && H % 8 == 0;
    b.hdr = hdr;
    auto fn = fast ? lin_bwd_kernel<T, lg::kKO, lg::kKO, true> : lin_bwd_kernel<T, lg::kKO, lg::kKOg, false>;
    const int lb = fast ? kBwdLds : 2 * lg::kStageBytes;
    if (set_lds(fn, lb) != CE_OK) return CE_ERR_HIP;
    const int64_t grid = ((V + 255) / 256) * ((H + 255) / 256);
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), lb, st, b);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  }
  hipLaunchKernelGGL(lin_finish_kernel, dim3(1), dim3(kNT), 0, st, loss_rows, labels, N, V, ignore, n_valid,
                     (const uint32_t*)nullptr, 0, (const LinHeader*)hdr, loss_mean, status);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

int launch_f32_gemm(bool ako, bool bko, const float* A, int64_t lda, const float* B, int64_t ldb, int M, int N, int K,
                    float alpha, float beta, float* C, int64_t ldc, hipStream_t st) {
  const dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
  if (!ako && !bko) hipLaunchKernelGGL((lin_gemm_f32_kernel<false, false>), grid, dim3(256), 0, st, A, lda, B, ldb, M, N, K, alpha, beta, C, ldc);
  else if (!ako && bko) hipLaunchKernelGGL((lin_gemm_f32_kernel<false, true>), grid, dim3(256), 0, st, A, lda, B, ldb, M, N, K, alpha, beta, C, ldc);
  else if (ako && !bko) hipLaunchKernelGGL((lin_gemm_f32_kernel<true, false>), grid, dim3(256), 0, st, A, lda, B, ldb, M, N, K, alpha, beta, C, ldc);
  else hipLaunchKernelGGL((lin_gemm_f32_kernel<true, true>), grid, dim3(256), 0, st, A, lda, B, ldb, M, N, K, alpha, beta, C, ldc);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

// The fp32 path, chunk by chunk.
int run_f32(const float* h, int64_t ldh, const float* w, int64_t ldw, const int64_t* labels, int64_t N, int64_t H,
            int64_t V, int64_t ignore, const float* dloss, float* loss_mean, float* loss_rows, int32_t* n_valid,
            uint32_t* status, float* gh, int64_t ldgh, float* gw, int64_t ldgw, char* ws, const F32Layout& L,
            hipStream_t st) {
  float* logits = (float*)(ws + L.logits);
  float* dl_chunk = (float*)(ws + L.dl_chunk);
  uint32_t* chunk_status = (uint32_t*)(ws + L.chunk_status);
  float* chunk_loss = (float*)(ws + L.chunk_loss);
  int32_t* chunk_n = (int32_t*)(ws + L.chunk_n);
  // the chunks' cross-entropy workspace starts from zero in every call (the
  // same workspace may have served the 16-bit layout in between)
  const size_t words = L.ce_ws_bytes / 4;
  hipLaunchKernelGGL(lin_fill_kernel, dim3((unsigned)((words + 255) / 256 < 1024 ? (words + 255) / 256 : 1024)),
                     dim3(256), 0, st, (uint32_t*)(ws + L.ce_ws), words);
  hipLaunchKernelGGL(lin_prep_kernel, dim3(1), dim3(kNT), 0, st, labels, N, ignore, L.T, L.nc, dloss, 0,
                     (LinHeader*)nullptr, dl_chunk, n_valid);
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  for (int c = 0; c < L.nc; ++c) {
    const int64_t r0 = (int64_t)c * L.T;
    const int64_t Tc = (N - r0 < L.T) ? N - r0 : L.T;
    const float* hc = h + r0 * ldh;
    int rc = launch_f32_gemm(false, false, hc, ldh, w, ldw, (int)Tc, (int)V, (int)H, 1.0f, 0.0f, logits, V, st);
    if (rc != CE_OK) return rc;
    // the chunk's dloss share dloss n_c / n: its scale dloss' / n_c is the batch's
    rc = ce_fwd_bwd_inplace(logits, V, labels + r0, Tc, V, CE_DTYPE_F32, ignore, 0, dl_chunk + c, chunk_loss + c,
                            loss_rows + r0, nullptr, nullptr, chunk_n + c, chunk_status + c, ws + L.ce_ws,
                            L.ce_ws_bytes, st);
    if (rc != CE_OK) return rc;
    if (gh) {  // dh_c = g_c W: B(n = h, k = v) = W[v][h]
      rc = launch_f32_gemm(false, true, logits, V, w, ldw, (int)Tc, (int)H, (int)V, 1.0f, 0.0f, gh + r0 * ldgh, ldgh,
                           st);
      if (rc != CE_OK) return rc;
    }
    if (gw) {  // dW += g_c^T h_c: A(m = v, k = tok) = g[tok][v], B(n = h, k = tok) = h[tok][h]
      rc = launch_f32_gemm(true, true, logits, V, hc, ldh, (int)V, (int)H, (int)Tc, 1.0f, c == 0 ? 0.0f : 1.0f, gw,
                           ldgw, st);
      if (rc != CE_OK) return rc;
    }
  }
  hipLaunchKernelGGL(lin_finish_kernel, dim3(1), dim3(kNT), 0, st, loss_rows, labels, N, V, ignore, n_valid,
                     (const uint32_t*)chunk_status, L.nc, (const LinHeader*)nullptr, loss_mean, status);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

size_t workspace_for(int64_t N, int64_t H, int64_t V, int64_t chunk_rows, int dtype) {
  (void)H;
  if (dtype == CE_DTYPE_F32) {
    const F32Layout L = f32_layout(N, V, chunk_rows);
    return L.ce_ws_bytes ? L.total : 0;
  }
  const int64_t cus = device_cus();
  return fast_layout(N, V, cus > 0 ? cus : 256).total;
}

}  // namespace

extern "C" {

size_t ce_linear_workspace_bytes(int64_t n_rows, int64_t hidden_size, int64_t vocab, int64_t chunk_rows,
                                 int dtype) {
  if (!valid_dtype(dtype) || n_rows < 0 || hidden_size < 1 || vocab < 1 || chunk_rows < 0) return 0;
  if (!fits32(n_rows) || !fits32(hidden_size) || !fits32(vocab)) return 0;
  return workspace_for(n_rows, hidden_size, vocab, chunk_rows, dtype);
}

int ce_linear_fwd_bwd(const void* hidden, int64_t ld_hidden, const void* weight, int64_t ld_weight,
                      const int64_t* labels, int64_t n_rows, int64_t hidden_size, int64_t vocab, int dtype,
                      int64_t ignore_index, int64_t chunk_rows, const float* dloss, float* loss_mean,
                      float* loss_rows, int32_t* n_valid, uint32_t* status, void* grad_hidden,
                      int64_t ld_grad_hidden, void* grad_weight, int64_t ld_grad_weight, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return CE_ERR_DTYPE;
  const int64_t N = n_rows, H = hidden_size, V = vocab;
  if (N < 0 || H < 1 || V < 1 || chunk_rows < 0) return CE_ERR_INVALID_ARG;
  if (ld_hidden < H || ld_weight < H) return CE_ERR_INVALID_ARG;
  if (grad_hidden && ld_grad_hidden < H) return CE_ERR_INVALID_ARG;
  if (grad_weight && ld_grad_weight < H) return CE_ERR_INVALID_ARG;
  if (loss_mean == nullptr || n_valid == nullptr) return CE_ERR_INVALID_ARG;
  if (N > 0 && (hidden == nullptr || weight == nullptr || labels == nullptr || loss_rows == nullptr))
    return CE_ERR_INVALID_ARG;
  const int es = esize(dtype);
  const uintptr_t al = (uintptr_t)es;
  if ((uintptr_t)hidden % al || (uintptr_t)weight % al || (uintptr_t)grad_hidden % al ||
      (uintptr_t)grad_weight % al || (uintptr_t)labels % 8)
    return CE_ERR_INVALID_ARG;
  if (!fits32(N) || !fits32(H) || !fits32(V) || !fits32(ld_hidden) || !fits32(ld_weight) ||
      !fits32(ld_grad_hidden) || !fits32(ld_grad_weight))
    return CE_ERR_UNSUPPORTED;
  // buffer resources address each operand with 32-bit offsets below 2^31
  const int64_t lim = (int64_t)1 << 31;
  if ((N + 256) * ld_hidden * es >= lim || (V + 256) * ld_weight * es >= lim ||
      (N + 256) * ((V + 7) / 8 * 8) * es >= lim)
    return CE_ERR_UNSUPPORTED;
  const size_t need = workspace_for(N, H, V, chunk_rows, dtype);
  if (need == 0) return CE_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < need || (uintptr_t)workspace % 256) return CE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;
  if (N == 0) {
    hipLaunchKernelGGL(lin_empty_kernel, dim3(1), dim3(64), 0, st, loss_mean, n_valid, status);
    if (grad_weight)
      hipLaunchKernelGGL(lin_zero_kernel, dim3((unsigned)V), dim3(256), 0, st, (uint16_t*)grad_weight,
                         ld_grad_weight, H, es);
    return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
  }
  if (dtype == CE_DTYPE_F32)
    return run_f32((const float*)hidden, ld_hidden, (const float*)weight, ld_weight, labels, N, H, V, ignore_index,
                   dloss, loss_mean, loss_rows, n_valid, status, (float*)grad_hidden, ld_grad_hidden,
                   (float*)grad_weight, ld_grad_weight, ws, f32_layout(N, V, chunk_rows), st);
  const int64_t cus = device_cus();
  const FastLayout L = fast_layout(N, V, cus > 0 ? cus : 256);
  if (L.nvt > (cus > 0 ? cus : 256)) return CE_ERR_UNSUPPORTED;  // a row tile's vocabulary tiles must be co-resident
  if (dtype == CE_DTYPE_BF16)
    return run_fast<__bf16>(hidden, ld_hidden, weight, ld_weight, labels, N, H, V, ignore_index, dloss, loss_mean,
                            loss_rows, n_valid, status, grad_hidden, ld_grad_hidden, grad_weight, ld_grad_weight, ws,
                            L, false, st);
  return run_fast<_Float16>(hidden, ld_hidden, weight, ld_weight, labels, N, H, V, ignore_index, dloss, loss_mean,
                            loss_rows, n_valid, status, grad_hidden, ld_grad_hidden, grad_weight, ld_grad_weight, ws,
                            L, true, st);
}

}  // extern "C"
