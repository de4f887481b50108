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
//   1. prep: n_valid and the gradient scale s = dloss 2^k / n_valid (fp16
//      keeps g in its normal range through 2^k, k = 14 - ilogb(dloss / n);
//      bf16 k = 0).
//   2. logits: one workgroup per 256 x 256 tile of h W^T in fp32
//      accumulators; no logits reach memory.  Its epilogue takes per row the
//      tile's max and stores the tile's exponentials relative to it, in the
//      input format, where g will be, with the row's (shift, label-excluded
//      sum) for the tile and the label's logit -- the per-chunk statistics of
//      a chunked loss, with 256-column chunks.
//   3. per row: the tiles' statistics merged into the log-sum-exp, the loss,
//      and g = s (softmax - onehot) written over the exponentials (each
//      scaled by its tile's factor, rounded to the input format).
//   4. dh = g W        MFMA, g K-contiguous, W read K-outer (transposed on its
//                      way into LDS); scaled by 2^-k on output
//   5. dW = g^T h      MFMA, both read K-outer; scaled by 2^-k on output
//   6. the token mean over the batch, summed in row order in fp64.
// The workspace holds g (N x V in the input format) and per row and tile two
// floats; no fp32 logits and no transposed copies.
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
constexpr uint32_t kStatusLabelRange = 0x1u, kStatusSyncTimeout = 0x2u;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int esize(int dtype) { return dtype == CE_DTYPE_F32 ? 4 : 2; }
bool valid_dtype(int d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16 || d == CE_DTYPE_F16; }
bool fits32(int64_t x) { return x >= 0 && x < ((int64_t)1 << 31); }

// ---------------------------------------------------------------------------
// Workspace of the 16-bit path.
// ---------------------------------------------------------------------------
struct LinHeader {
  uint32_t status;  // status bits of this call (cleared by prep)
  float gscale;     // s = dloss 2^k / n_valid
  float unscale;    // 2^-k
  int32_t n_valid;
  uint32_t pad[60];
};
static_assert(sizeof(LinHeader) == 256, "header size");

struct FastLayout {
  size_t g, tstats, xy, part, total;
  int64_t ldg;  // g's row stride: vocab rounded up to 8 elements
  int nvt;      // vocabulary tiles of 256
  int dh_split; // K ranges of dh = g W (1: no split)
  int dh_kc;    // vocabulary columns per range (a multiple of 32)
};

// dh has ceil(N / 256) x ceil(H / 256) tiles, each over all V columns of g:
// with few rows that leaves most of the chip idle, so the vocabulary is cut
// into ranges (each at least 1024 columns), doubling their number while the
// tiles times the ranges still fit in one round of 256 workgroups (a second
// round would take as long as the ranges saved); every range writes an fp32
// partial tile, summed in range order by a small kernel.
void dh_split_of(int64_t N, int64_t H, int64_t V, int& split, int& kc) {
  const int64_t tiles = ((N + 255) / 256) * ((H + 255) / 256);
  int s = 1;
  while (s < 16 && tiles * 2 * s <= 256 && V / (2 * s) >= 1024) s *= 2;
  kc = (int)((V + 32 * s - 1) / (32 * s) * 32);
  split = (int)((V + kc - 1) / kc);
}

FastLayout fast_layout(int64_t N, int64_t H, int64_t V) {
  FastLayout L;
  memset(&L, 0, sizeof(L));
  L.ldg = (V + 7) / 8 * 8;
  L.nvt = (int)((V + 255) / 256);
  dh_split_of(N, H, V, L.dh_split, L.dh_kc);
  size_t off = sizeof(LinHeader);
  L.g = align256(off);
  off = L.g + align256((size_t)N * L.ldg * 2);
  L.tstats = off;  // [row][vocabulary tile]: (c, sum) float pairs
  off += align256((size_t)N * L.nvt * 8);
  L.xy = off;  // [row] the label's logit
  off += align256((size_t)N * 4);
  L.part = off;  // dh's fp32 partial tiles, [range][N][H], when split
  if (L.dh_split > 1) off += align256((size_t)L.dh_split * N * H * 4);
  L.total = off;
  return L;
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
// 1. prep (one workgroup): n_valid and the scale; for the fp32 path
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
      hdr->status = 0u;
      hdr->gscale = n > 0 ? (float)(dl * up / (double)n) : 0.0f;
      hdr->unscale = (float)ldexp(1.0, -k);
      hdr->n_valid = (int32_t)n;
    }
  }
}

// ---------------------------------------------------------------------------
// 2. logits tile + the tile's share of the cross-entropy (16-bit).  One
// workgroup per 256 x 256 tile of logits = h W^T, over a plain grid of every
// tile (no co-residency, no exchange between workgroups).  From its fp32
// accumulators the epilogue takes per row the tile's max m over the columns
// inside the vocabulary and writes, into g's place, in the input format,
//   e = 2^(x log2 e - c),  c = m log2 e - E   (E = 14 for fp16, else 0:
//                                              fp16 keeps e in its normal range)
// with 0 at the label's column (the label's logit goes to xy), and per row
// the pair (c, sum of the tile's e).  The row's log-sum-exp needs every tile
// of the row, so the scale that turns e into g comes in the next kernel.
// ---------------------------------------------------------------------------
struct LogitsArgs {
  const char* h;
  int64_t ldh;
  const char* w;
  int64_t ldw;
  const int64_t* labels;
  int64_t ignore;
  int64_t N, H, V;
  int mt, nvt;     // row tiles, vocabulary tiles
  float eshift;    // E
  uint16_t* g;
  int64_t ldg;
  float2* tstats;  // [N][nvt]: (c, sum of e); c = -inf for a row with no finite max in the tile
  float* xy;       // [N]: the label's logit (written by the tile that holds it)
};

// LDS: the K loop's stages (128 KB, or 64 KB for the element-wise loop),
// then over them the epilogue's row data (4 KB) and its statistics transpose
// (65 KB at offset 16 KB), and once the statistics are out, four staged
// 128 x 136 quarters of e (136 KB, also at offset 16 KB).
constexpr int kLogitsLds = 160 * 1024;
static_assert(16384 + 4 * 128 * 136 * 2 <= kLogitsLds, "staged quarters");
static_assert(16384 + 256 * 65 * 4 <= kLogitsLds, "statistics transpose");

// Row of accumulator element v of 32-row block i within a lane's rows (the
// lane's first row is wm * 128 + 4 * (lane / 32); see lg::acc_row).
__device__ constexpr int kRowOff(int i, int v) { return i * 32 + 8 * (v >> 2) + (v & 3); }

// Row tiles per group of the tile order (8 and 4 measured alike at 4096 x
// 4096 x 32000, 16 about 2% slower per call).
constexpr int kRowGroup = 8;

// Tile order: groups of kRowGroup row tiles; inside a group the tiles walk
// the vocabulary slab by slab with the group's row tiles of a slab adjacent.
// In the XCD order each XCD takes one contiguous stretch of that walk, so the
// row tiles that share a weight slab run on one XCD at about the same time
// and the slab comes into that XCD's L2 once.
__device__ __forceinline__ void logits_tile_of(int bid, int mt, int nvt, int& rt, int& vt) {
  const int lin = lg::xcd_order(bid, mt * nvt);
  const int grp = lin / (kRowGroup * nvt), idx = lin - grp * (kRowGroup * nvt);
  const int rows = min(kRowGroup, mt - grp * kRowGroup);
  rt = grp * kRowGroup + idx % rows;
  vt = idx / rows;
}

template <typename T, bool DMA>
__global__ __launch_bounds__(256, 1) void lin_logits_kernel(LogitsArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int rt, vt;
  logits_tile_of((int)blockIdx.x, a.mt, a.nvt, rt, vt);
  const int64_t mrow0 = (int64_t)rt * 256;  // the tile's first row
  const int n0 = vt * 256;
  const int M = (int)a.N, Nv = (int)a.V, K = (int)a.H;
  Tile t;
  if constexpr (DMA) lg::tile_nt<T>(t, lds, a.h, a.ldh, a.w, a.ldw, M, Nv, K, (int)mrow0, n0);
  else lg::tile_rs<T, lg::kKCg, lg::kKCg>(t, lds, a.h, a.ldh, a.w, a.ldw, M, Nv, K, (int)mrow0, n0);
  __syncthreads();  // every wave is done with the K loop's LDS

  // LDS after the K loop: per-row label data and statistics, and a
  // [256][kPS] transpose area for the per-lane partials (kPS = 65 floats per
  // row: the row reductions, one thread per row, read without bank
  // conflicts).  The passes walk the accumulators one 32-row block (index i)
  // at a time so that only that block's row constants are held in registers.
  constexpr int kPS = 65;
  int32_t* yrel = (int32_t*)lds;        // [256] label column - n0 when in this tile, else -1
  float* mrow = (float*)(lds + 1024);   // [256] the tile's row max
  float* mrowc = (float*)(lds + 2048);  // [256] c (0 for a row whose max is -inf): the exponentials' shift
  float* xyl = (float*)(lds + 3072);    // [256] label logits found here
  float* part = (float*)(lds + 16384);  // [256][kPS]
  {
    const int64_t R = mrow0 + tid;
    const int64_t y = (R < a.N) ? a.labels[R] : a.ignore;
    yrel[tid] = (y != a.ignore && y >= n0 && y < n0 + 256 && y < a.V) ? (int)(y - n0) : -1;
  }
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
    if (__builtin_expect(full, 1)) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        m[v] = fmaxf(fmaxf(t.acc[i][0][v], t.acc[i][1][v]), fmaxf(t.acc[i][2][v], t.acc[i][3][v]));
    } else {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = cvalid[j] ? t.acc[i][j][v] : -INFINITY;
        m[v] = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
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
    mrowc[tid] = (m == -INFINITY) ? 0.0f : m * kLog2e - a.eshift;
  }
  __syncthreads();
  // pass B: e = 2^(x log2 e - c) for every element, written over its logit
  // in the accumulators, and per lane and row the label-excluded sum of its
  // four.  For a row whose label lies in some lane's columns (a ballot per
  // row, rarely true) the lane that holds it takes out the label's logit
  // (into xyl) and sets its e to 0; no other row pays a per-element label
  // test.
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // the block's row shifts and label columns for this lane's 16 rows
    // (rows rb + 8 k + u, v = 4 k + u), as four 16-byte reads each
    const int rb = wm * 128 + i * 32 + 4 * (lane >> 5);
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    float mcv[16];
    int ycv[16];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x4 qm = *(const f32x4*)(mrowc + rb + 8 * k);
      const i32x4 qy = *(const i32x4*)(yrel + rb + 8 * k);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        mcv[4 * k + u] = qm[u];
        ycv[4 * k + u] = qy[u];
      }
    }
    float sv[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = lg::acc_row(wm, i, v, lane);
      const float mc = mcv[v];
      float e[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(t.acc[i][j][v], kLog2e, -mc));
        e[j] = cvalid[j] ? e[j] : 0.0f;  // all true in every tile but the last
      }
      const int d = ycv[v] - lc;          // the label's column is this lane's in block d / 32
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
    const int64_t R = mrow0 + r;
    if (R < a.N) {
      a.tstats[R * a.nvt + vt] = make_float2(mrow[r] == -INFINITY ? -INFINITY : mrowc[r], S);
      if (yrel[r] >= 0) a.xy[R] = xyl[r];
    }
  }
  __syncthreads();  // the statistics area is free

  // e in the input format: each wave stages its 128 x 128 quarter in LDS
  // (rows of 272 bytes), 32 rows at a time, and writes them out as 16-byte
  // vectors, so the stores of one block overlap the conversions of the next.
  constexpr int kGS = 136;  // staged row stride in elements
  uint16_t* stg = (uint16_t*)(lds + 16384 + wave * (128 * kGS * 2));
  uint16_t* stg_l = stg + 4 * (lane >> 5) * kGS + (lane & 31);  // + kRowOff(i, v) * kGS + 32 j
  const int64_t cbase = (int64_t)n0 + wn * 128;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x16 blk = t.acc[i][j];
#pragma unroll
      for (int v = 0; v < 16; ++v) stg_l[kRowOff(i, v) * kGS + 32 * j] = to_bits<T>(blk[v]);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (it reads only its own quarter)
    asm volatile("" ::: "memory");       // and the compiler keeps the 16-bit writes before the 16-byte reads
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rr = i * 32 + q * 4 + (lane >> 4), cv = (lane & 15) * 8;
      const int64_t R = mrow0 + wm * 128 + rr;
      const int64_t c = cbase + cv;
      if (R < a.N && c < a.ldg) *(lg::u32x4*)(a.g + R * a.ldg + c) = *(const lg::u32x4*)(stg + rr * kGS + cv);
    }
  }
}

// ---------------------------------------------------------------------------
// 3. per row (a workgroup walks rows R = blockIdx.x, + gridDim.x, ...): the
// row's log-sum-exp from its tiles' (c, sum) pairs, merged in a fixed order,
// the row's loss (lse - x_y, or log1p(S / e^{x_y}) when p_y > 1/2, S the
// label-excluded sum), and g = s (softmax - onehot) written over the stored
// e, rounded once more to the input format: e s 2^(c - lse log2 e) off the
// label, -s (1 - p_y) on it; +0 on ignored rows, NaN on rows with a label
// outside [0, V) (+0 past the vocabulary).
// ---------------------------------------------------------------------------
struct RescaleArgs {
  const int64_t* labels;
  int64_t ignore;
  int64_t N, V;
  int nvt;
  uint16_t* g;
  int64_t ldg;
  const float2* tstats;
  const float* xy;
  const LinHeader* hdr;
  float* loss_rows;
};

constexpr int kMaxRescaleTiles = 8192;  // dynamic LDS: two floats per tile
constexpr float kLn2 = 0.6931471805599453f;

template <typename T>
__device__ __forceinline__ float from_bits(uint32_t b);
template <>
__device__ __forceinline__ float from_bits<__bf16>(uint32_t b) {
  return __builtin_bit_cast(float, b << 16);
}
template <>
__device__ __forceinline__ float from_bits<_Float16>(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

template <typename T>
__global__ __launch_bounds__(256) void lin_rescale_kernel(RescaleArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  float* tc = (float*)lds;   // [nvt] the tiles' c, then their factors s 2^(c - L)
  float* tsum = tc + a.nvt;  // [nvt] the tiles' sums
  __shared__ float red[8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nvec = (int)(a.ldg >> 3);
  const float gs = a.hdr->gscale;
  const uint32_t nanb = to_bits<T>(__builtin_nanf(""));
  for (int64_t R = blockIdx.x; R < a.N; R += gridDim.x) {
    const int64_t y = a.labels[R];
    uint16_t* grow = a.g + R * a.ldg;
    if (y == a.ignore || y < 0 || y >= a.V) {  // the same for the whole workgroup
      const bool ign = (y == a.ignore);
      for (int q = tid; q < nvec; q += 256) {
        uint32_t wv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t c = (int64_t)q * 8 + 2 * k;
          const uint32_t lo = (!ign && c < a.V) ? nanb : 0u, hi = (!ign && c + 1 < a.V) ? nanb : 0u;
          wv[k] = lo | (hi << 16);
        }
        __builtin_nontemporal_store(lg::u32x4{wv[0], wv[1], wv[2], wv[3]}, (lg::u32x4*)(grow + (int64_t)q * 8));
      }
      if (tid == 0) a.loss_rows[R] = ign ? 0.0f : __builtin_nanf("");
      continue;
    }
    const float2* ts = a.tstats + R * a.nvt;
    const float xyv = a.xy[R];
    float mx = -INFINITY;
    for (int v = tid; v < a.nvt; v += 256) {
      const float2 p = ts[v];
      tc[v] = p.x;
      tsum[v] = p.y;
      mx = fmaxf(mx, p.x);
    }
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    const float Mc = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    float sl = 0.0f;
    for (int v = tid; v < a.nvt; v += 256) {
      const float c = tc[v];
      if (c != -INFINITY) sl += tsum[v] * __builtin_amdgcn_exp2f(c - Mc);
    }
    sl = wave_sum(sl);
    if (lane == 0) red[4 + wave] = sl;
    __syncthreads();
    // S: the label-excluded sum, ey the label's term, both relative to 2^Mc
    const float S = (red[4] + red[5]) + (red[6] + red[7]);
    const float ey = __builtin_amdgcn_exp2f(xyv * kLog2e - Mc);
    const float St = S + ey;
    const float L = Mc + log2f(St);  // lse log2 e
    const float pcomp = S / St;      // 1 - p_y
    if (tid == 0) a.loss_rows[R] = (pcomp >= 0.5f) ? (L * kLn2 - xyv) : log1pf(S / ey);
    for (int v = tid; v < a.nvt; v += 256) {
      const float c = tc[v];
      tc[v] = (c == -INFINITY) ? 0.0f : gs * __builtin_amdgcn_exp2f(c - L);
    }
    __syncthreads();
    const uint32_t gyb = to_bits<T>(-gs * pcomp);
    const int yq = (int)(y >> 3), ys = (int)(y & 7) * 16;
    // four 16-byte vectors per lane in flight, then their products
    for (int q0 = tid; q0 < nvec; q0 += 1024) {
      lg::u32x4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + 256 * u;
        if (q < nvec) v[u] = *(const lg::u32x4*)(grow + (int64_t)q * 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int q = q0 + 256 * u;
        if (q < nvec) {
          const float f = tc[q >> 5];  // 32 vectors per 256-column tile
          uint32_t o[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const uint32_t wd = v[u][k];
            o[k] = to_bits<T>(from_bits<T>(wd & 0xFFFFu) * f) | ((uint32_t)to_bits<T>(from_bits<T>(wd >> 16) * f) << 16);
          }
          if (q == yq) {
            const int k = ys >> 5, sh = ys & 16;
            o[k] = (o[k] & ~(0xFFFFu << sh)) | (gyb << sh);
          }
          __builtin_nontemporal_store(lg::u32x4{o[0], o[1], o[2], o[3]}, (lg::u32x4*)(grow + (int64_t)q * 8));
        }
      }
    }
    __syncthreads();  // tc / red are rewritten for the next row
  }
}

// ---------------------------------------------------------------------------
// 4-5. dh = g W and dW = g^T h (16-bit): MFMA tiles, 2^-k on output.
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
  int ksplit, kc;  // K ranges of kc columns (ksplit 1: the whole K, C written directly)
  float* part;     // ksplit > 1: fp32 partial tiles [range][M][N] instead of C
};

// DMA: both operands through direct-to-LDS loads (16-byte aligned rows;
// a.Mx / a.Nx bound the 16-byte chunks a KO operand may load), kLdsBytes of
// LDS; otherwise the register-staged loop, 2 kStageBytes.
template <typename T, int AK, int BKD, bool DMA>
__global__ __launch_bounds__(256, 1) void lin_bwd_kernel(BwdArgs a) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int mt = (a.M + 255) / 256, nt = (a.N + 255) / 256, tiles = mt * nt;
  // g (the A operand of both products) is the larger operand: the tiles of
  // a K range that share its rows are neighbours in the XCD order
  int lin = lg::xcd_order((int)blockIdx.x, tiles * a.ksplit);
  const int ks = lin / tiles;
  lin -= ks * tiles;
  const int mti = lin / nt, nti = lin % nt;
  const int m0 = mti * 256, n0 = nti * 256;
  // this workgroup's K range: columns k0 .. k0 + kr of A and B
  const int64_t k0 = (int64_t)ks * a.kc;
  const int kr = (int)(a.K - k0 < a.kc ? a.K - k0 : a.kc);
  const char* A = a.A + (AK == lg::kKC ? k0 * 2 : k0 * a.lda * 2);
  const char* B = a.B + (BKD == lg::kKC ? k0 * 2 : k0 * a.ldb * 2);
  Tile t;
  if constexpr (DMA) lg::tile_dma<T, AK, BKD>(t, lds, A, a.lda, B, a.ldb, a.Mx, a.Nx, kr, m0, n0);
  else lg::tile_rs<T, AK, BKD>(t, lds, A, a.lda, B, a.ldb, a.M, a.N, kr, m0, n0);
  const float us = a.hdr->unscale;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, wm = wave >> 1, wn = wave & 1;
  if (a.ksplit > 1) {  // the range's fp32 partial tile; the sum, the scale and the rounding come later
    float* P = a.part + (size_t)ks * a.M * a.N;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int R = m0 + lg::acc_row(wm, i, v, lane), c = n0 + lg::acc_col(wn, j, lane);
          if (R < a.M && c < a.N) P[(int64_t)R * a.N + c] = t.acc[i][j][v];
        }
    return;
  }
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
    asm volatile("" ::: "memory");       // and the compiler keeps the 16-bit writes before the 16-byte reads
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

// The split dh: C = us (sum over the K ranges of the partial tiles, in range
// order), rounded once; four columns per thread (N a multiple of 4).
template <typename T>
__global__ __launch_bounds__(256) void lin_split_sum_kernel(const float* part, int ksplit, int M, int N,
                                                            const LinHeader* hdr, uint16_t* C, int64_t ldc,
                                                            int vec_out) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const float us = hdr->unscale;
  const int64_t n4 = N / 4, total = (int64_t)M * n4, plane = (int64_t)M * N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / n4, c = (i - r * n4) * 4;
    const float* p = part + r * N + c;
    f32x4 acc = *(const f32x4*)p;
    for (int k = 1; k < ksplit; ++k) acc += *(const f32x4*)(p + k * plane);
    uint16_t* d = C + r * ldc + c;
    const uint32_t w0 = (uint32_t)to_bits<T>(acc[0] * us) | ((uint32_t)to_bits<T>(acc[1] * us) << 16);
    const uint32_t w1 = (uint32_t)to_bits<T>(acc[2] * us) | ((uint32_t)to_bits<T>(acc[3] * us) << 16);
    if (vec_out) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      *(u32x2*)d = u32x2{w0, w1};
    } else {
      d[0] = (uint16_t)w0;
      d[1] = (uint16_t)(w0 >> 16);
      d[2] = (uint16_t)w1;
      d[3] = (uint16_t)(w1 >> 16);
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
  la.mt = (int)((N + 255) / 256);
  la.nvt = L.nvt;
  la.eshift = fp16 ? 14.0f : 0.0f;
  la.g = g;
  la.ldg = L.ldg;
  la.tstats = (float2*)(ws + L.tstats);
  la.xy = (float*)(ws + L.xy);
  auto kfn = fast ? lin_logits_kernel<T, true> : lin_logits_kernel<T, false>;
  if (set_lds(kfn, kLogitsLds) != CE_OK) return CE_ERR_HIP;
  hipLaunchKernelGGL(kfn, dim3((unsigned)((int64_t)la.mt * L.nvt)), dim3(256), kLogitsLds, st, la);
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
  RescaleArgs ra;
  ra.labels = labels;
  ra.ignore = ignore;
  ra.N = N;
  ra.V = V;
  ra.nvt = L.nvt;
  ra.g = g;
  ra.ldg = L.ldg;
  ra.tstats = la.tstats;
  ra.xy = la.xy;
  ra.hdr = hdr;
  ra.loss_rows = loss_rows;
  const int rs_lds = 2 * L.nvt * 4;
  if (set_lds(lin_rescale_kernel<T>, rs_lds) != CE_OK) return CE_ERR_HIP;
  hipLaunchKernelGGL(lin_rescale_kernel<T>, dim3((unsigned)(N < (1 << 20) ? N : (1 << 20))), dim3(256), rs_lds, st,
                     ra);
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
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
    const int split = fast ? L.dh_split : 1;  // K ranges (direct-to-LDS path only)
    b.ksplit = split;
    b.kc = split > 1 ? L.dh_kc : (int)V;
    b.part = split > 1 ? (float*)(ws + L.part) : nullptr;
    auto fn = fast ? lin_bwd_kernel<T, lg::kKC, lg::kKO, true> : lin_bwd_kernel<T, lg::kKC, lg::kKOg, false>;
    const int lb = fast ? kBwdLds : 2 * lg::kStageBytes;
    if (set_lds(fn, lb) != CE_OK) return CE_ERR_HIP;
    const int64_t grid = ((N + 255) / 256) * ((H + 255) / 256) * split;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(256), lb, st, b);
    if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
    if (split > 1) {
      const int64_t quads = N * H / 4, blocks = (quads + 255) / 256;
      hipLaunchKernelGGL(lin_split_sum_kernel<T>, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0, st,
                         (const float*)b.part, split, (int)N, (int)H, (const LinHeader*)hdr, (uint16_t*)gh, ldgh,
                         b.vec_out);
      if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;
    }
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
    b.ksplit = 1;  // ceil(V / 256) x ceil(H / 256) tiles fill the chip
    b.kc = (int)N;
    b.part = nullptr;
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
  if ((V + 255) / 256 > kMaxRescaleTiles) return 0;
  return fast_layout(N, H, V).total;
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
  // buffer resources address h and W with 32-bit offsets below 2^31; g too
  // in the element-wise loads (one resource over all of g's rows) and the fp32
  // path, not in the direct-to-LDS ones (resources per tile or per K step)
  const int64_t lim = (int64_t)1 << 31;
  const bool fast16 = dtype != CE_DTYPE_F32 && aligned16(hidden, ld_hidden, 2) && aligned16(weight, ld_weight, 2) &&
                      H % 8 == 0;
  if ((N + 256) * ld_hidden * es >= lim || (V + 256) * ld_weight * es >= lim ||
      (!fast16 && (N + 256) * ((V + 7) / 8 * 8) * es >= lim))
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
  const FastLayout L = fast_layout(N, H, V);
  if (dtype == CE_DTYPE_BF16)
    return run_fast<__bf16>(hidden, ld_hidden, weight, ld_weight, labels, N, H, V, ignore_index, dloss, loss_mean,
                            loss_rows, n_valid, status, grad_hidden, ld_grad_hidden, grad_weight, ld_grad_weight, ws,
                            L, false, st);
  return run_fast<_Float16>(hidden, ld_hidden, weight, ld_weight, labels, N, H, V, ignore_index, dloss, loss_mean,
                            loss_rows, n_valid, status, grad_hidden, ld_grad_hidden, grad_weight, ld_grad_weight, ws,
                            L, true, st);
}

}  // extern "C"
