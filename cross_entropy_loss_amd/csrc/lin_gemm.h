// lin_gemm.h -- gfx950 MFMA matrix products for the LM-head path.
//
// The LM head of the pages' fused linear cross-entropy (PyPI page
// "fms-acceleration-foak 0.7.4", "Running Liger Kernel Benchmarks") is three
// dense contractions over bf16 / fp16 operands with fp32 accumulation:
// logits = h W^T, dh = g W and dW = g^T h.  These are the real matrix work of
// the path, so they run on the matrix cores: v_mfma_f32_32x32x16_{bf16,f16}.
//
// One kernel shape, "NT": C[M, N] = A[M, K] B[N, K]^T with both operands
// K-contiguous (row i of A at A + i * lda elements).  A workgroup of 256 lanes
// (four waves as 2 x 2) owns a 256 x 256 tile of C; each wave a 128 x 128
// quarter as 4 x 4 blocks of 32 x 32 fp32 accumulators (256 accumulator
// registers per lane, one wave per SIMD).  K advances in steps of 32: each
// step's A and B slabs (256 rows x 64 bytes each) stream straight into LDS
// with direct-to-LDS buffer loads, four steps in flight (4 x 32 KB of LDS),
// so the loads need no staging registers.  Inside a slab row the four
// 16-byte chunks are XOR-swizzled by the row index (the loading lane picks
// the global chunk for its fixed LDS slot), which spreads the MFMA operand
// reads of 32 consecutive rows over distinct LDS banks.
//
// Bounds: loads go through buffer resources whose extent is the operand's
// rows; rows past M / N and 16-byte chunks past K load zeros (K must be a
// multiple of 8 elements).  The epilogue masks its own stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4, NTH = 256;
constexpr int kSlabBytes = 256 * BK * 2;        // one operand's rows of a K step: 16 KB
constexpr int kStageBytes = 2 * kSlabBytes;     // A and B: 32 KB
constexpr int kLdsBytes = STAGES * kStageBytes;  // 128 KB
constexpr uint32_t kOob = 0x80000000u;           // a buffer offset past every extent served

constexpr int kBufFlags = 0x00020000;  // raw 32-bit dword buffer, gfx9 layout

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kBufFlags);
}

// Buffer resource words (base, 16 bits of base | stride 0, extent, format)
// for the inline direct-to-LDS load below.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return u32x4{(uint32_t)b, (uint32_t)(b >> 32) & 0xFFFFu, bytes, (uint32_t)kBufFlags};
}
// One 16-byte-per-lane direct-to-LDS load: lane l's 16 bytes at resource
// offset voff + soff (zeros past the extent) go to LDS byte lds_addr + 16 l.
// Written as inline assembly so that the compiler does not track it as a
// pending LDS write: it would otherwise wait for every such load in flight
// (vmcnt 0) before each transposing LDS read.  The caller orders the loads
// against the LDS reads with explicit vmcnt waits and workgroup barriers;
// every operand comes from scalar arithmetic (the "s" constraints fail to
// assemble otherwise), so no vector-written SGPR feeds the load, and M0 is
// set one wait state before its use.  No result registers are involved.
__device__ __forceinline__ void dma16(u32x4 rs, uint32_t lds_addr, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
               : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_addr_of(const char* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Chunk swizzle of slab row r (2 bits): rows r and r + 8 of a 16-row group,
// and every pair of the 8-row groups, land on different chunk slots.
__device__ __forceinline__ uint32_t swz(uint32_t r) { return ((r >> 1) & 3u) ^ ((r >> 3) & 1u); }

template <typename T>
struct Mfma;
template <>
struct Mfma<__bf16> {
  __device__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  }
};
template <>
struct Mfma<_Float16> {
  __device__ static f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
};

__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
// s_waitcnt with only vmcnt = N (gfx9 encoding: vmcnt bits [3:0] and [15:14])
template <int N>
__device__ __forceinline__ void wait_vm() {
  sched_fence();
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  sched_fence();
}
__device__ __forceinline__ void wait_lgkm0() {
  sched_fence();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  sched_fence();
}
// A workgroup barrier for LDS traffic only (no global-memory fence, so the
// K steps' loads stay in flight across it).
__device__ __forceinline__ void lds_barrier() {
  wait_lgkm0();
  __builtin_amdgcn_s_barrier();
  sched_fence();
}

// Direct-to-LDS loads of one operand's K step: 256 rows x 32 elements into a
// 16 KB LDS slab.  Each of the wave's four instructions fills 16 rows (1 KB):
// lane l writes LDS row r = 16 (4 wave + i) + l / 4, slot l % 4, and so loads
// global chunk c = (l % 4) ^ swz(r) of that row.  The per-lane byte offsets
// (r ld + 16 c, or an out-of-range offset for rows past the operand) are
// computed once per tile; the K step advances through the scalar offset.
struct SlabOffsets {
  uint32_t off[4];
  int chunk[4];
};
__device__ __forceinline__ SlabOffsets slab_offsets(int64_t ld_bytes, int rows, int wave, int lane) {
  SlabOffsets o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ (int)swz((uint32_t)r);
    o.chunk[i] = c;
    o.off[i] = (r < rows) ? (uint32_t)((int64_t)r * ld_bytes + c * 16) : kOob;
  }
  return o;
}
// Step kt: elements [32 kt, 32 kt + 32) of each row; chunks at or past K load
// zeros (only the last step can have such chunks).
__device__ __forceinline__ void load_step(__amdgpu_buffer_rsrc_t rs, char* slab, const SlabOffsets& o, int kt, int K,
                                          int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
  const uint32_t so = (uint32_t)kt * (BK * 2);
  const bool tail = (kt + 1) * BK > K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t off = o.off[i];
    if (tail && kt * BK + o.chunk[i] * 8 >= K) off = kOob;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(slab + (wave * 4 + i) * 1024),
                                             16, off, so, 0, 0);
  }
#endif
}

// The MFMA operand of slab row r, K half h (elements h*8 .. h*8+7 of the
// 16-element step kk): 16 bytes at its swizzled chunk.
__device__ __forceinline__ u32x4 frag(const char* slab, int r, int kk, int h) {
  const int c = kk * 2 + h;
  return *(const u32x4*)(slab + r * 64 + ((c ^ (int)swz((uint32_t)r)) << 4));
}

struct Tile {
  f32x16 acc[4][4];
};

// Operand layouts.  KC: K-contiguous, row i of the operand at p + i ld
// (h and W in the logits product, g in dh).  KO: K-outer, element (i, k) at
// p + k ld + i, the operand's rows contiguous (W in dh, g and h in dW).
enum { kKC = 0, kKO = 1 };

// KO slabs hold a K step as 32 K rows of the tile's 256 operand rows
// (512 bytes each, 16 KB), the 16-byte chunks of row k XOR-swizzled by
// ko_swz(k % 4).  The MFMA operand of lane l (operand row l % 32 of a block,
// K run 8 (l / 32) .. +7) is then gathered with two transposing reads
// (ds_read_b64_tr_b16): in each 16-lane group, result lane j takes element
// j % 4 of the 8-byte chunks addressed by lanes j / 4, j / 4 + 4, + 8, + 12
// of its group, so source lane q of group g points at operand rows
// 16 (g % 2) + 4 (q % 4) .. +3 of K row 8 (g / 2) + 4 h + q / 4 (read h
// gives K elements 4 h .. 4 h + 3 of the run).  The swizzle values keep the
// four K rows of a 16-lane group, and of a 32-lane half, on distinct banks.
__device__ __forceinline__ uint32_t ko_swz(uint32_t k4) { return (0xCA60u >> (4 * k4)) & 15u; }  // 0, 6, 10, 12

// One operand's direct-to-LDS loads and MFMA operand reads.
template <int KIND>
struct DmaOp;

template <>
struct DmaOp<kKC> {
  u32x4 rw;
  SlabOffsets o;
  int K;
  // rows: the operand's extent along M / N from the tile origin
  __device__ __forceinline__ void init(const char* p, int64_t ld, int origin, int extent, int K_, int wave, int lane) {
    const int64_t lb = ld * 2;
    const int rows = extent - origin;
    rw = rsrc_words(p + (int64_t)origin * lb, (uint32_t)((int64_t)(rows < 256 ? rows : 256) * lb));
    o = slab_offsets(lb, rows, wave, lane);
    K = K_;
  }
  // instruction i of step kt: slab rows 16 (4 wave + i) .. +15; chunks at or
  // past K (only in the last step, or in steps past it) load zeros
  __device__ __forceinline__ void load1(char* slab, int kt, int wave, int i) const {
    uint32_t off = o.off[i];
    if ((kt + 1) * BK > K && kt * BK + o.chunk[i] * 8 >= K) off = kOob;
    dma16(rw, lds_addr_of(slab + (wave * 4 + i) * 1024), off, (uint32_t)kt * (BK * 2));
  }
  __device__ __forceinline__ void load(char* slab, int kt, int wave) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) load1(slab, kt, wave, i);
  }
  // per-step context of the loads (none) and load i of a step
  __device__ __forceinline__ int ctx(int) const { return 0; }
  __device__ __forceinline__ void issue(int, char* slab, int kt, int wave, int i) const { load1(slab, kt, wave, i); }
  // operand of block rows mb .. mb + 31 (relative to the tile), K half kk
  __device__ __forceinline__ u32x4 frag_of(const char* slab, int mb, int kk, int lane) const {
    return frag(slab, mb + (lane & 31), kk, lane >> 5);
  }
  static constexpr int kReads = 1;  // LDS instructions per operand
};

template <>
struct DmaOp<kKO> {
  const char* base;   // element (origin, 0)
  int64_t lb;         // bytes between K rows
  int K;
  uint32_t full, part;  // extent of a whole step / of the last partial one
  uint32_t off[4];    // per instruction: byte offset in the step's 32 K rows, or past every extent
  uint32_t rd;        // per lane: K row and 8-byte half of its first transposing read (kk 0, h 0)
  uint32_t cx;        // per lane: low chunk bits and swizzle, XORed with a block's chunk base
  // extent: the operand's rows (columns of the stored matrix) that may be
  // loaded; whole 16-byte chunks from origin on below it are loaded
  __device__ __forceinline__ void init(const char* p, int64_t ld, int origin, int extent, int K_, int wave, int lane) {
    lb = ld * 2;
    base = p + (int64_t)origin * 2;
    K = K_;
    full = (uint32_t)(BK * lb);
    part = (uint32_t)((K % BK) * lb);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = 2 * (wave * 4 + i) + (lane >> 5);  // K row of the step
      const int c = (lane & 31) ^ (int)ko_swz((uint32_t)rr & 3u);
      off[i] = (origin + 8 * c < extent) ? (uint32_t)((int64_t)rr * lb + c * 16) : kOob;
    }
    const int g = lane >> 4, q = lane & 15;
    const int k = 8 * (g >> 1) + (q >> 2);      // K row of read h = 0 (its row mod 4 is (q / 4) mod 4)
    const int cl = 2 * (g & 1) + ((q & 3) >> 1);  // chunk within the block's four
    rd = (uint32_t)(k * 512 + (q & 1) * 8);
    cx = (uint32_t)cl ^ ko_swz((uint32_t)(q >> 2) & 3u);
  }
  // step kt: K rows 32 kt .. 32 kt + 31 through a resource that ends at K,
  // so rows past K (and every row of a step past the last) load zeros.  The
  // extent is chosen with scalar selects (a clamp would be a vector op).
  __device__ __forceinline__ u32x4 step_words(int kt) const {
    const int kf = K / BK;
    const uint32_t nrec = kt < kf ? full : (kt == kf ? part : 0u);
    return rsrc_words(base + (int64_t)kt * BK * lb, nrec);
  }
  __device__ __forceinline__ void load1(const u32x4& rw, char* slab, int wave, int i) const {
    dma16(rw, lds_addr_of(slab + (wave * 4 + i) * 1024), off[i], 0u);
  }
  __device__ __forceinline__ void load(char* slab, int kt, int wave) const {
    const u32x4 rw = step_words(kt);
#pragma unroll
    for (int i = 0; i < 4; ++i) load1(rw, slab, wave, i);
  }
  __device__ __forceinline__ u32x4 ctx(int kt) const { return step_words(kt); }
  __device__ __forceinline__ void issue(const u32x4& rw, char* slab, int, int wave, int i) const {
    load1(rw, slab, wave, i);
  }
  // block rows mb .. mb + 31 (mb a multiple of 32): the lane's chunk is
  // mb / 8 + cl, whose slot is (mb / 8 + cl) ^ swz = (mb / 8) ^ cx (mb / 8 is a
  // multiple of 4 and cl < 4, so the sum is an XOR)
  __device__ __forceinline__ u32x4 frag_of(const char* slab, int mb, int kk, int /* lane: in rd, cx */) const {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const uint32_t a = rd + ((((uint32_t)mb >> 3) ^ cx) << 4) + (uint32_t)kk * (16 * 512);
    const __attribute__((address_space(3))) char* sl = (const __attribute__((address_space(3))) char*)slab;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sl + a));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sl + a + 4 * 512));
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    const u32x2_t l2 = __builtin_bit_cast(u32x2_t, lo), h2 = __builtin_bit_cast(u32x2_t, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
  static constexpr int kReads = 2;
};

// The wave's eight MFMA operands of half kk of a K step: A rows
// wm * 128 + i * 32 + lane % 32 and B rows wn * 128 + j * 32 + lane % 32.
template <int AK, int BKD>
__device__ __forceinline__ void read_frags(const char* st, const DmaOp<AK>& oa, const DmaOp<BKD>& ob, int wm, int wn,
                                           int lane, int kk, u32x4 (&a)[4], u32x4 (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = oa.frag_of(st, wm * 128 + i * 32, kk, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = ob.frag_of(st + kSlabBytes, wn * 128 + j * 32, kk, lane);
}

// The same for two KC slabs (the register-staged loop below).
__device__ __forceinline__ void read_frags(const char* st, int wm, int wn, int lane, int kk, u32x4 (&a)[4],
                                           u32x4 (&b)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = frag(st, wm * 128 + i * 32 + (lane & 31), kk, lane >> 5);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = frag(st + kSlabBytes, wn * 128 + j * 32 + (lane & 31), kk, lane >> 5);
}

// The K loop of one 256 x 256 tile: acc = A[m0:, :] B[n0:, :]^T, A and B
// of layouts AK / BKD (16-byte aligned rows; a KO operand's extent along
// its tile dimension a whole number of 16-byte chunks or padded to one).
// Needs kLdsBytes of LDS.  tid_: the thread index, when the caller runs tiles
// in a loop and passes one the compiler cannot see through (so no
// lane-dependent address is hoisted out of that loop and held across it);
// threadIdx.x otherwise.
template <typename T, int AK, int BKD, int S = STAGES>
__device__ __forceinline__ void tile_dma(Tile& t, char* lds, const char* A, int64_t lda, const char* B, int64_t ldb,
                                         int M, int N, int K, int m0, int n0, int tid_ = -1) {
  static_assert(S >= 4, "the loads of a step go out two and three steps ahead");
  const int tid = tid_ < 0 ? (int)threadIdx.x : tid_, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  DmaOp<AK> oa;
  DmaOp<BKD> ob;
  oa.init(A, lda, m0, M, K, wave, lane);
  ob.init(B, ldb, n0, N, K, wave, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) t.acc[i][j] = f32x16{};
  const int KT = (K + BK - 1) / BK;
  // Steps at or past KT load nothing (zero fills of a stage that is never
  // read for a product).  That keeps the loop body one basic block and the
  // wait counts fixed.
#pragma unroll
  for (int s = 0; s < S - 1; ++s) {
    char* st = lds + s * kStageBytes;
    oa.load(st, s, wave);
    if (s < S - 2) ob.load(st + kSlabBytes, s, wave);  // step S - 2's B loads go out in step 0
  }
  wait_vm<(S - 3) * 8 + 4>();  // step 0 (this lane's part)
  lds_barrier();
  u32x4 a0[4], b0[4], a1[4], b1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a0[i] = oa.frag_of(lds, wm * 128 + i * 32, 0, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) b0[j] = ob.frag_of(lds + kSlabBytes, wn * 128 + j * 32, 0, lane);
  // Rotated pipeline over S stages, one wave per SIMD, its instruction
  // order fixed by scheduling fences.  Step kt, first half: the 16 products
  // on (a0, b0), the first eight each preceded by one read of the
  // second-half operands (a1, b1), the next four by the B loads of step
  // kt + S - 2 (into the stage of step kt - 2, free since the last
  // barrier).  Then the barrier for step kt + 1 (every lane's loads of it
  // have landed, and every lane has consumed step kt - 1, whose stage is
  // free).  Second half: the 16 products on (a1, b1), preceded by the eight
  // reads of step kt + 1's first operands and then by the A loads of step
  // kt + S - 1 into step kt - 1's stage (reads before loads: both touch
  // LDS).  The two halves' loads keep the four waves from flooding the
  // address unit at once.  Each half starts by waiting for the reads of the
  // half before (long landed by then), so no product waits on a read just
  // issued.
  for (int kt = 0; kt < KT; ++kt) {
    const char* st = lds + (kt % S) * kStageBytes;
    char* n2 = lds + ((kt + S - 2) % S) * kStageBytes + kSlabBytes;
    const auto cb = ob.ctx(kt + S - 2);
    wait_lgkm0();
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < 4) a1[s] = oa.frag_of(st, wm * 128 + s * 32, 1, lane);
      else if (s < 8) b1[s - 4] = ob.frag_of(st + kSlabBytes, wn * 128 + (s - 4) * 32, 1, lane);
      else if (s < 12) ob.issue(cb, n2, kt + S - 2, wave, s - 8);
      t.acc[s >> 2][s & 3] = Mfma<T>::run(a0[s >> 2], b0[s & 3], t.acc[s >> 2][s & 3]);
      sched_fence();
    }
    wait_vm<(S - 3) * 8>();  // step kt + 1 (the newer loads: steps kt + 2 .. kt + S - 2)
    __builtin_amdgcn_s_barrier();
    wait_lgkm0();
    const char* s1 = lds + ((kt + 1) % S) * kStageBytes;
    char* nx = lds + ((kt + S - 1) % S) * kStageBytes;
    const auto ca = oa.ctx(kt + S - 1);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      if (s < 4) a0[s] = oa.frag_of(s1, wm * 128 + s * 32, 0, lane);
      else if (s < 8) b0[s - 4] = ob.frag_of(s1 + kSlabBytes, wn * 128 + (s - 4) * 32, 0, lane);
      else if (s < 12) oa.issue(ca, nx, kt + S - 1, wave, s - 8);
      t.acc[s >> 2][s & 3] = Mfma<T>::run(a1[s >> 2], b1[s & 3], t.acc[s >> 2][s & 3]);
      sched_fence();
    }
  }
  // the zero-fill loads of the steps past KT and the last reads are drained
  // before the caller reuses the LDS
  wait_vm<0>();
  wait_lgkm0();
}

template <typename T>
__device__ __forceinline__ void tile_nt(Tile& t, char* lds, const char* A, int64_t lda, const char* B, int64_t ldb,
                                        int M, int N, int K, int m0, int n0, int tid = -1) {
  tile_dma<T, kKC, kKC>(t, lds, A, lda, B, ldb, M, N, K, m0, n0, tid);
}

// ---------------------------------------------------------------------------
// Register-staged K loop for operands of either layout.  KC: K-contiguous
// (row i of the operand at p + i ld: 256 rows x 32 elements per step, four
// 16-byte loads per lane); KO: K-outer (element (i, k) at p + k ld + i, the
// operand's rows contiguous: a lane loads an 8 (k) x 4 (i) block as eight
// 8-byte loads and turns it with byte permutes into four 16-byte K runs).
// Either way each lane writes its part of the step into the same swizzled
// LDS slab that tile_nt's direct-to-LDS loads fill, and the MFMA loop is
// the same.  One register set: in step kt the set (step kt + 1, loaded one
// step earlier) goes to LDS and the loads of step kt + 2 refill it; LDS holds
// two steps.
// ---------------------------------------------------------------------------
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Stage {
  u32x4 q[4];  // KC: four 16-byte chunks; KO: eight 8-byte loads in q[0..3] as pairs
};

// KC lane map: 16 (4 wave + i) + lane / 4 = slab row, (lane % 4) ^ swz = chunk
// (the same slots as the direct-to-LDS loads).
__device__ __forceinline__ void kc_load(Stage& st, __amdgpu_buffer_rsrc_t rs, const SlabOffsets& o, int kt, int K) {
  const uint32_t so = (uint32_t)kt * (BK * 2);
  const bool tail = (kt + 1) * BK > K;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t off = o.off[i];
    if (tail && kt * BK + o.chunk[i] * 8 >= K) off = kOob;
    st.q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, so, 0));
  }
}
__device__ __forceinline__ void kc_store(const Stage& st, char* slab, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4*)(slab + (wave * 4 + i) * 1024 + lane * 16) = st.q[i];
}

// KO lane map: thread t owns slab rows i = 4 (t % 64) .. +3 and K elements
// 8 (t / 64) .. +7 of the step (one 16-byte chunk of each of its four rows).
struct KoOffsets {
  uint32_t off;  // byte offset of (k = 8 (t / 64), i = 4 (t % 64)), or past the extent
};
__device__ __forceinline__ KoOffsets ko_offsets(int64_t ld_bytes, int cols, int tid) {
  KoOffsets o;
  const int i = 4 * (tid & 63), kg = tid >> 6;
  o.off = (i < cols) ? (uint32_t)((int64_t)kg * 8 * ld_bytes + i * 2) : kOob;
  return o;
}
__device__ __forceinline__ void ko_load(Stage& st, __amdgpu_buffer_rsrc_t rs, const KoOffsets& o, int64_t ld_bytes,
                                        int kt, int K, int tid) {
  const int kg = tid >> 6;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int k = kt * BK + kg * 8 + r;
    const uint32_t so = (uint32_t)((int64_t)kt * BK * ld_bytes + (int64_t)r * ld_bytes);
    const uint32_t off = (k < K) ? o.off : kOob;
    const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, so, 0));
    st.q[r >> 1][(r & 1) * 2 + 0] = v[0];
    st.q[r >> 1][(r & 1) * 2 + 1] = v[1];
  }
}
// q[r / 2][(r % 2) * 2 + d] holds elements (k = r, i = 2 d, 2 d + 1) of the
// block; slab row 4 (t % 64) + ii gets the K run k = 0..7 of column ii.
__device__ __forceinline__ void ko_store(const Stage& st, char* slab, int tid) {
  const int i0 = 4 * (tid & 63), kg = tid >> 6;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int d = ii >> 1;
    const uint32_t sel = (ii & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = st.q[e][d], hi = st.q[e][2 + d];  // rows k = 2e and 2e + 1
      o[e] = __builtin_amdgcn_perm(hi, lo, sel);
    }
    const int r = i0 + ii;
    *(u32x4*)(slab + r * 64 + ((kg ^ (int)swz((uint32_t)r)) << 4)) = o;
  }
}

// Element-wise variants for operands whose rows are not 16-byte aligned (or
// whose K is not a multiple of 8): the same lane maps and LDS slots, one
// 2-byte load per element, every element bounds-checked (rows, K, columns).
enum { kKCg = 2, kKOg = 3 };
__device__ __forceinline__ uint32_t ld16(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return (uint32_t)(uint16_t)__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
}
__device__ __forceinline__ void kcg_load(Stage& st, __amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int rows, int kt,
                                         int K, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (wave * 4 + i) * 16 + (lane >> 2);
    const int c = (lane & 3) ^ (int)swz((uint32_t)r);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const int k0 = kt * BK + c * 8 + 2 * d;
      const int64_t base = (int64_t)r * ld_bytes + (int64_t)k0 * 2;
      const uint32_t lo = (r < rows && k0 < K) ? ld16(rs, (uint32_t)base) : 0u;
      const uint32_t hi = (r < rows && k0 + 1 < K) ? ld16(rs, (uint32_t)(base + 2)) : 0u;
      st.q[i][d] = lo | (hi << 16);
    }
  }
}
__device__ __forceinline__ void kog_load(Stage& st, __amdgpu_buffer_rsrc_t rs, int64_t ld_bytes, int cols, int kt,
                                         int K, int tid) {
  const int i0 = 4 * (tid & 63), kg = tid >> 6;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int k = kt * BK + kg * 8 + r;
    const int64_t base = (int64_t)k * ld_bytes + (int64_t)i0 * 2;
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const uint32_t lo = (k < K && i0 + 2 * d < cols) ? ld16(rs, (uint32_t)(base + 4 * d)) : 0u;
      const uint32_t hi = (k < K && i0 + 2 * d + 1 < cols) ? ld16(rs, (uint32_t)(base + 4 * d + 2)) : 0u;
      st.q[r >> 1][(r & 1) * 2 + d] = lo | (hi << 16);
    }
  }
}

template <int KIND>
struct OpLoader {
  __amdgpu_buffer_rsrc_t rs;
  int64_t ld_bytes;
  int rows;  // extent from the tile origin (clipped to 256)
  SlabOffsets kc;
  KoOffsets ko;
};

// rows: the operand's extent along the tile (M or N) from the tile origin;
// for KO, the operand's rows are along K, so the buffer spans all K rows.
template <int KIND>
__device__ __forceinline__ OpLoader<KIND> make_loader(const char* p, int64_t ld, int origin, int extent, int K,
                                                      int wave, int lane, int tid) {
  OpLoader<KIND> L;
  L.ld_bytes = ld * 2;
  const int rows = extent - origin;
  L.rows = rows < 256 ? rows : 256;
  if constexpr (KIND == kKC || KIND == kKCg) {
    L.rs = make_rsrc(p + (int64_t)origin * L.ld_bytes, (uint32_t)((int64_t)L.rows * L.ld_bytes));
    if constexpr (KIND == kKC) L.kc = slab_offsets(L.ld_bytes, rows, wave, lane);
  } else {
    L.rs = make_rsrc(p + (int64_t)origin * 2, (uint32_t)((int64_t)K * L.ld_bytes));
    if constexpr (KIND == kKO) L.ko = ko_offsets(L.ld_bytes, L.rows, tid);
  }
  return L;
}
template <int KIND>
__device__ __forceinline__ void op_load(Stage& st, const OpLoader<KIND>& L, int kt, int K, int tid) {
  if constexpr (KIND == kKC) kc_load(st, L.rs, L.kc, kt, K);
  else if constexpr (KIND == kKO) ko_load(st, L.rs, L.ko, L.ld_bytes, kt, K, tid);
  else if constexpr (KIND == kKCg) kcg_load(st, L.rs, L.ld_bytes, L.rows, kt, K, tid >> 6, tid & 63);
  else kog_load(st, L.rs, L.ld_bytes, L.rows, kt, K, tid);
}
template <int KIND>
__device__ __forceinline__ void op_store(const Stage& st, char* slab, int wave, int lane, int tid) {
  if constexpr (KIND == kKC || KIND == kKCg) kc_store(st, slab, wave, lane);
  else ko_store(st, slab, tid);
}

// One step's MFMA work in the rotated form of tile_nt: first half with the
// second-half reads between the products, then (hook) the step's
// register-to-LDS stores and the barrier, then the second half with the next
// step's first reads.
template <typename T, int AK, int BKD>
__device__ __forceinline__ void rs_step(Tile& t, char* lds, int kt, int KT, int K, int wm, int wn, int wave, int lane,
                                        int tid, const OpLoader<AK>& la, const OpLoader<BKD>& lb, Stage& sa, Stage& sb,
                                        u32x4 (&a0)[4], u32x4 (&b0)[4], u32x4 (&a1)[4], u32x4 (&b1)[4]) {
  const char* st = lds + (kt & 1) * kStageBytes;
  read_frags(st, wm, wn, lane, 1, a1, b1);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) t.acc[i][j] = Mfma<T>::run(a0[i], b0[j], t.acc[i][j]);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
  sched_fence();
  if (kt + 1 < KT) {
    // step kt + 1 (loaded two steps ago) into the other buffer, whose step
    // kt - 1 every lane finished reading before the last barrier
    char* nx = lds + ((kt + 1) & 1) * kStageBytes;
    op_store<AK>(sa, nx, wave, lane, tid);
    op_store<BKD>(sb, nx + kSlabBytes, wave, lane, tid);
    if (kt + 2 < KT) {
      op_load<AK>(sa, la, kt + 2, K, tid);
      op_load<BKD>(sb, lb, kt + 2, K, tid);
    }
    lds_barrier();
  }
  sched_fence();
  if (kt + 1 < KT) read_frags(lds + ((kt + 1) & 1) * kStageBytes, wm, wn, lane, 0, a0, b0);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) t.acc[i][j] = Mfma<T>::run(a1[i], b1[j], t.acc[i][j]);
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
  sched_fence();
}

// acc = A B^T over K for the tile at (m0, n0), A and B of kinds AK / BKD.
// Needs 2 * kStageBytes of LDS.
template <typename T, int AK, int BKD>
__device__ __forceinline__ void tile_rs(Tile& t, char* lds, const char* A, int64_t lda, const char* B, int64_t ldb,
                                        int M, int N, int K, int m0, int n0) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const OpLoader<AK> la = make_loader<AK>(A, lda, m0, M, K, wave, lane, tid);
  const OpLoader<BKD> lb = make_loader<BKD>(B, ldb, n0, N, K, wave, lane, tid);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) t.acc[i][j] = f32x16{};
  const int KT = (K + BK - 1) / BK;
  // step 0 straight to LDS; step 1 into the register set
  Stage sa, sb;
  op_load<AK>(sa, la, 0, K, tid);
  op_load<BKD>(sb, lb, 0, K, tid);
  op_store<AK>(sa, lds, wave, lane, tid);
  op_store<BKD>(sb, lds + kSlabBytes, wave, lane, tid);
  if (KT > 1) {
    op_load<AK>(sa, la, 1, K, tid);
    op_load<BKD>(sb, lb, 1, K, tid);
  }
  lds_barrier();
  u32x4 a0[4], b0[4], a1[4], b1[4];
  read_frags(lds, wm, wn, lane, 0, a0, b0);
  for (int kt = 0; kt < KT; ++kt)
    rs_step<T, AK, BKD>(t, lds, kt, KT, K, wm, wn, wave, lane, tid, la, lb, sa, sb, a0, b0, a1, b1);
}

// Workgroups are placed on the 8 XCDs round-robin by id.  xcd_order(bid,
// total) renumbers a grid of `total` workgroups so that each XCD takes one
// contiguous range of the new order (XCD x: the ids b = x mod 8, in
// increasing order), whatever the grid size.
__device__ __forceinline__ int xcd_order(int bid, int total) {
  const int x = bid & 7, q = bid >> 3;
  const int per = total >> 3, extra = total & 7;  // XCDs below `extra` take one more
  return x * per + (x < extra ? x : extra) + q;
}

// Tile order for a grid of mt x nt tiles: each XCD walks whole rows of column
// tiles, so the nt column tiles that share one A tile run on one XCD (for
// products whose A operand is the larger one).
__device__ __forceinline__ void tile_of_rows(int bid, int mt, int nt, int& m_tile, int& n_tile) {
  const int lin = xcd_order(bid, mt * nt);
  m_tile = lin / nt;
  n_tile = lin % nt;
}

// Row and column of accumulator element v of block (i, j) in this lane,
// relative to the tile origin.
__device__ __forceinline__ int acc_row(int wm, int i, int v, int lane) {
  return wm * 128 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 128 + j * 32 + (lane & 31); }

}  // namespace lg
