// ce_linear.hip -- LM-head projection followed by the cross-entropy of
// ce_api.hip, forward and backward, token-chunked (the C ABI in
// include/ce_mi355x.h: ce_linear_workspace_bytes, ce_linear_fwd_bwd).
//
// The pages compare the plain cross-entropy kernel with a fused linear
// cross-entropy (PyPI page "fms-acceleration-foak 0.7.4", "Running Liger
// Kernel Benchmarks"), list fused cross-entropy among the kernels to come
// (fms-hf-tuning PR #280, "Notes on FastKernels") and leave a chunked loss as
// a to-do (fms-acceleration PR #79, "TODO").  With hidden states h [N, H] and
// the weight W [V, H] of a bias-free linear layer, logits = h W^T, and
//   dL/dh = g W,   dL/dW = g^T h,   g = dloss * dL/dlogits.
//
// Per chunk of T rows, on the caller's stream:
//   1. logits_c = h_c W^T            rocBLAS GEMM, fp32 accumulate, fp32 out
//   2. loss and g over logits_c      ce_fwd_bwd_inplace on the fp32 chunk, its
//                                    dloss set to dloss * n_c / n so that its
//                                    scale dloss' / n_c is the batch's dloss / n
//   3. g rounded to the input format (bf16 / fp16) for the two GEMMs below
//   4. dh_c = g W                    rocBLAS GEMM, fp32 accumulate, dtype out
//   5. dW32 += g^T h_c               GEMM, fp32 accumulate and out (16-bit, shapes
//                                    tiling by 64: TN on transposed copies of g, h_c)
// then dW32 is rounded once to the input format (with a single chunk the GEMM
// writes the input format itself, from its fp32 sums), and the token mean over the
// whole batch is summed in row order in fp64.  The batch's logits are never
// stored: one fp32 chunk (T x V) lives in the workspace.
//
// fp16 range.  |g| <= s = dloss / n (about 1e-6 at n = 4096 and V = 32000
// per element), deep in fp16's subnormal range, where rounding g for the
// GEMMs would cost percents.  For fp16 the chunk's dloss' carries a power of
// two 2^k, k = 14 - ilogb(s), so the rounded g lies below 2^15 and keeps its
// 11 bits down to s 2^-28; the dh GEMM takes alpha = 2^-k and the final dW
// cast multiplies by 2^-k, both exact.  bf16 and fp32 have fp32's range and
// keep k = 0.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <math.h>
#include <rocblas/rocblas.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "ce_internal.h"
#include "ce_mi355x.h"

namespace {

// 4096 rows: the chunk's fp32 logits and rounded gradient take 4096 V 6
// bytes (786 MB at V = 32000), and the GEMMs run at their larger-shape
// rate (4096 x 4096 x 32000 bf16: 3.7 ms per call against 5.5 ms with
// 1024-row chunks).
constexpr int64_t kDefaultChunkRows = 4096;
constexpr int64_t kMaxChunks = 4096;  // per-chunk counts live in LDS
constexpr int kNT = 1024;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
int esize(int dtype) { return dtype == CE_DTYPE_F32 ? 4 : 2; }
bool valid_dtype(int d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16 || d == CE_DTYPE_F16; }

// Rows per chunk: a multiple of 64 (a wave's labels fall in one chunk) and
// at most kMaxChunks chunks.
int64_t chunk_rows_for(int64_t N, int64_t chunk_rows) {
  int64_t t = chunk_rows > 0 ? chunk_rows : kDefaultChunkRows;
  const int64_t min_t = (N + kMaxChunks - 1) / kMaxChunks;
  if (t < min_t) t = min_t;
  t = (t + 63) / 64 * 64;
  return t;
}

struct LinLayout {
  size_t ce_ws, logits, g16, dw32, dl_chunk, chunk_status, chunk_loss, chunk_n, consts, gT, hT, total;
  bool tn;  // weight gradient from transposed operands
  size_t ce_ws_bytes;
  int64_t T;
  int nc;
};

LinLayout lin_layout(int64_t N, int64_t H, int64_t V, int64_t chunk_rows, int dtype) {
  LinLayout L;
  memset(&L, 0, sizeof(L));
  L.T = chunk_rows_for(N, chunk_rows);
  L.nc = (int)((N + L.T - 1) / L.T);
  const int64_t Tc = (N < L.T) ? (N > 0 ? N : 1) : L.T;
  L.ce_ws_bytes = ce_workspace_bytes(Tc, V, 0, CE_DTYPE_F32);
  size_t off = 0;
  L.ce_ws = off;
  off += align256(L.ce_ws_bytes);
  L.logits = off;
  off += align256((size_t)Tc * V * 4);
  if (dtype != CE_DTYPE_F32) {
    L.g16 = off;
    off += align256((size_t)Tc * V * 2);
    if (L.nc > 1) {  // one chunk: the weight-gradient GEMM writes the output format directly
      L.dw32 = off;
      off += align256((size_t)V * H * 4);
    }
  }
  const size_t nc = (size_t)(L.nc > 0 ? L.nc : 1);
  L.dl_chunk = off;
  off += align256(nc * 4);
  L.chunk_status = off;
  off += align256(nc * 4);
  L.chunk_loss = off;
  off += align256(nc * 4);
  L.chunk_n = off;
  off += align256(nc * 4);
  L.consts = off;  // 1, 0, 2^-k (GEMM scalars read in device pointer mode)
  off += 256;
  // 16-bit weight gradient as a TN GEMM on transposed copies of the chunk's
  // g and h (reduction dimension contiguous: 0.81 vs 1.03 ms for the NT form
  // on 4096 x 4096 x 32000 bf16), when every chunk tiles by 64
  // (T is a multiple of 64, so N % 64 == 0 makes every chunk's rows one)
  L.tn = dtype != CE_DTYPE_F32 && N > 0 && N % 64 == 0 && V % 64 == 0 && H % 64 == 0;
  if (L.tn) {
    L.gT = off;
    off += align256((size_t)V * Tc * 2);
    L.hT = off;
    off += align256((size_t)H * Tc * 2);
  }
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// Kernels.
// ---------------------------------------------------------------------------

// One workgroup: valid rows per chunk (T a multiple of 64, so a wave's 64
// consecutive labels fall in one chunk), the batch count n, each chunk's
// dloss' = dloss 2^k n_c / n, and the GEMM scalars {1, 0, 2^-k}.
__global__ __launch_bounds__(kNT) void lin_prep_kernel(const int64_t* labels, int64_t N, int64_t ignore, int64_t T,
                                                       int nc, const float* dloss, int fp16_range, float* dl_chunk,
                                                       int32_t* n_valid_out, float* consts) {
  __shared__ int32_t cnt[kMaxChunks];
  __shared__ int64_t wsum[kNT / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int c = tid; c < nc; c += kNT) cnt[c] = 0;
  __syncthreads();
  for (int64_t base = 0; base < N; base += kNT) {
    const int64_t i = base + tid;
    const bool v = i < N && labels[i] != ignore;
    const uint64_t ballot = __ballot(v);
    if (lane == 0 && ballot) atomicAdd(&cnt[(int)((i) / T)], (int32_t)__popcll(ballot));
  }
  __syncthreads();
  int64_t s = 0;
  for (int c = tid; c < nc; c += kNT) s += cnt[c];
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
  for (int c = tid; c < nc; c += kNT) dl_chunk[c] = n > 0 ? (float)(dl * up * (double)cnt[c] / (double)n) : 0.0f;
  if (tid == 0) {
    n_valid_out[0] = (int32_t)n;
    consts[0] = 1.0f;
    consts[1] = 0.0f;
    consts[2] = (float)ldexp(1.0, -k);
  }
}

// fp32 * scale (a power of two, or NULL = 1) -> storage format, nearest-even,
// one workgroup per row: 16-byte loads and 8-byte stores where the row's
// alignment allows (a per-row choice), single elements otherwise.
template <typename T>
__global__ __launch_bounds__(256) void lin_cast_kernel(const float* src, int64_t ld_src, int64_t cols, T* dst,
                                                       int64_t ld_dst, const float* scale) {
  const float* s = src + (int64_t)blockIdx.x * ld_src;
  T* d = dst + (int64_t)blockIdx.x * ld_dst;
  const float f = scale ? scale[0] : 1.0f;
  int64_t j0 = 0;
  if ((uintptr_t)s % 16 == 0 && (uintptr_t)d % 8 == 0) {
    const int64_t n4 = cols / 4;
    for (int64_t q = threadIdx.x; q < n4; q += 256) {
      const float4 x = ((const float4*)s)[q];
      const T o[4] = {(T)(x.x * f), (T)(x.y * f), (T)(x.z * f), (T)(x.w * f)};
      uint2 w;
      __builtin_memcpy(&w, o, sizeof(w));
      ((uint2*)d)[q] = w;
    }
    j0 = n4 * 4;
  }
  for (int64_t j = j0 + threadIdx.x; j < cols; j += 256) d[j] = (T)(s[j] * f);
}

__global__ __launch_bounds__(256) void lin_zero_kernel(uint16_t* dst, int64_t ld, int64_t cols, int esz) {
  if (esz == 4) {
    float* d = (float*)dst + (int64_t)blockIdx.x * ld;
    for (int64_t j = threadIdx.x; j < cols; j += 256) d[j] = 0.0f;
  } else {
    uint16_t* d = dst + (int64_t)blockIdx.x * ld;
    for (int64_t j = threadIdx.x; j < cols; j += 256) d[j] = 0;
  }
}

// dst[c][r] = src[r][c] for a rows x cols matrix of 16-bit elements (both
// row-major, rows and cols multiples of 64): one 64 x 64 tile per workgroup,
// read and written in 16-byte vectors, turned through LDS (rows padded to 66
// elements so a column read falls in distinct banks).  It gives the
// weight-gradient GEMM operands whose reduction dimension is contiguous.
__global__ __launch_bounds__(256) void lin_transpose16_kernel(const uint16_t* src, int64_t ld_src, uint16_t* dst,
                                                              int64_t ld_dst) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ uint16_t tile[64][66];
  const int64_t r0 = (int64_t)blockIdx.y * 64, c0 = (int64_t)blockIdx.x * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = tid + h * 256, r = u >> 3, cv = (u & 7) * 8;
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(src + (r0 + r) * ld_src + c0 + cv));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      tile[r][cv + 2 * d] = (uint16_t)(v[d] & 0xffffu);
      tile[r][cv + 2 * d + 1] = (uint16_t)(v[d] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = tid + h * 256, c = u >> 3, rv = (u & 7) * 8;
    u32x4 o;
#pragma unroll
    for (int d = 0; d < 4; ++d) o[d] = (uint32_t)tile[rv + 2 * d][c] | ((uint32_t)tile[rv + 2 * d + 1][c] << 16);
    __builtin_nontemporal_store(o, (u32x4*)(dst + (c0 + c) * ld_dst + r0 + rv));
  }
}

// One workgroup: L = sum of the valid rows' losses / n, in row order (each
// lane a contiguous slice, then a fixed tree), fp64; status = OR of the chunks'.
__global__ __launch_bounds__(kNT) void lin_finish_kernel(const float* loss_rows, const int64_t* labels, int64_t N,
                                                         int64_t ignore, const int32_t* n_valid,
                                                         const uint32_t* chunk_status, int nc, float* loss_mean,
                                                         uint32_t* status) {
  __shared__ double acc[kNT];
  __shared__ uint32_t st[kNT];
  const int tid = threadIdx.x;
  const int64_t i0 = N * tid / kNT, i1 = N * (tid + 1) / kNT;
  double a = 0.0;
  for (int64_t i = i0; i < i1; ++i)
    if (labels[i] != ignore) a += (double)loss_rows[i];
  uint32_t s = 0;
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
    loss_mean[0] = (float)(acc[0] / (double)n_valid[0]);
    if (status) status[0] = st[0];
  }
}

__global__ void lin_empty_kernel(float* loss_mean, int32_t* n_valid, uint32_t* status) {
  if (threadIdx.x == 0) {
    loss_mean[0] = __builtin_nanf("");
    n_valid[0] = 0;
    if (status) status[0] = 0u;
  }
}

// ---------------------------------------------------------------------------
// rocBLAS: one handle per device for the process lifetime; calls on a device
// are serialised around it (the handle's stream is set per call).
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::mutex g_blas_mu[kMaxDevices];
rocblas_handle g_blas[kMaxDevices];

// hipBLASLt for the 16-bit GEMMs (its first heuristic choice measured 14-19%
// faster than rocBLAS on the 4096 x 4096 x 32000 shapes); rocBLAS serves fp32
// and any shape hipBLASLt offers no algorithm for.  Per device: one handle and
// the descriptors and algorithm chosen for each GEMM shape, kept for the
// process (host memory); no GEMM workspace is asked for.  Its scalars are
// passed from the host: with device-resident scalars
// (HIPBLASLT_POINTER_MODE_DEVICE) the installed hipBLASLt returned wrong
// results (only element 0 of D right), so a GEMM whose alpha exists only on
// the device (fp16's 2^-k) stays on rocBLAS.
struct LtPlan {
  bool ta, tb;
  int64_t m, n, k, lda, ldb, ldc;
  hipDataType ab, c;
  bool ok;
  hipblasLtMatmulDesc_t md;
  hipblasLtMatrixLayout_t la, lb, lc;
  hipblasLtMatmulAlgo_t algo;
};
hipblasLtHandle_t g_lt[kMaxDevices];
bool g_lt_failed[kMaxDevices];
std::vector<LtPlan> g_plans[kMaxDevices];
// Plans kept per device; past this many (callers whose row counts keep
// changing) the oldest is destroyed, so the cache stays bounded.
constexpr size_t kMaxPlans = 128;

void destroy_plan(LtPlan& p) {
  if (p.md) hipblasLtMatmulDescDestroy(p.md);
  if (p.la) hipblasLtMatrixLayoutDestroy(p.la);
  if (p.lb) hipblasLtMatrixLayoutDestroy(p.lb);
  if (p.lc) hipblasLtMatrixLayoutDestroy(p.lc);
  p.md = nullptr;
  p.la = p.lb = p.lc = nullptr;
}

// The plan for a GEMM shape (nullptr: hipBLASLt offers none).  Called with the
// device's lock held; the pointer is valid until the next call.
const LtPlan* lt_plan(int dev, bool ta, bool tb, int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb,
                      int64_t ldc, hipDataType ab, hipDataType c) {
  if (g_lt_failed[dev]) return nullptr;
  if (g_lt[dev] == nullptr && hipblasLtCreate(&g_lt[dev]) != HIPBLAS_STATUS_SUCCESS) {
    g_lt[dev] = nullptr;
    g_lt_failed[dev] = true;
    return nullptr;
  }
  for (const LtPlan& p : g_plans[dev])
    if (p.ta == ta && p.tb == tb && p.m == m && p.n == n && p.k == k && p.lda == lda && p.ldb == ldb &&
        p.ldc == ldc && p.ab == ab && p.c == c)
      return p.ok ? &p : nullptr;
  LtPlan p;
  memset(&p, 0, sizeof(p));
  p.ta = ta, p.tb = tb, p.m = m, p.n = n, p.k = k, p.lda = lda, p.ldb = ldb, p.ldc = ldc, p.ab = ab, p.c = c;
  const hipblasOperation_t oa = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N, ob = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
  hipblasLtMatmulPreference_t pref = nullptr;
  uint64_t no_ws = 0;
  hipblasLtMatmulHeuristicResult_t res;
  int nres = 0;
  p.ok = hipblasLtMatmulDescCreate(&p.md, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSA, &oa, sizeof(oa)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(p.md, HIPBLASLT_MATMUL_DESC_TRANSB, &ob, sizeof(ob)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.la, ab, ta ? k : m, ta ? m : k, lda) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.lb, ab, tb ? n : k, tb ? k : n, ldb) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatrixLayoutCreate(&p.lc, c, m, n, ldc) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &no_ws,
                                               sizeof(no_ws)) == HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulAlgoGetHeuristic(g_lt[dev], p.md, p.la, p.lb, p.lc, p.lc, pref, 1, &res, &nres) ==
             HIPBLAS_STATUS_SUCCESS &&
         nres > 0 && res.workspaceSize == 0;
  if (pref) hipblasLtMatmulPreferenceDestroy(pref);
  if (p.ok) p.algo = res.algo;
  else destroy_plan(p);  // remembered as unavailable: rocBLAS serves the shape
  if (g_plans[dev].size() >= kMaxPlans) {
    destroy_plan(g_plans[dev].front());
    g_plans[dev].erase(g_plans[dev].begin());
  }
  g_plans[dev].push_back(p);
  return p.ok ? &g_plans[dev].back() : nullptr;
}

rocblas_datatype blas_type(int dtype) {
  if (dtype == CE_DTYPE_BF16) return rocblas_datatype_bf16_r;
  if (dtype == CE_DTYPE_F16) return rocblas_datatype_f16_r;
  return rocblas_datatype_f32_r;
}

hipDataType lt_type(rocblas_datatype t) {
  return t == rocblas_datatype_bf16_r ? HIP_R_16BF : (t == rocblas_datatype_f16_r ? HIP_R_16F : HIP_R_32F);
}

// A GEMM scalar: its device copy, and its value when the host knows it (NaN
// when only the device does).
struct Scalar {
  const float* dev;
  float host;
};

// D = alpha op(A) op(B) + beta C (column-major, as BLAS): hipBLASLt for
// 16-bit inputs when both scalars are known on the host and it has an
// algorithm for the shape, else rocBLAS with the device scalars.
int gemm(int dev, rocblas_handle h, hipStream_t st, rocblas_operation ta, rocblas_operation tb, int64_t m, int64_t n,
         int64_t k, Scalar alpha_s, const void* A, rocblas_datatype at, int64_t lda, const void* B,
         rocblas_datatype bt, int64_t ldb, Scalar beta_s, void* C, rocblas_datatype ct, int64_t ldc) {
  if (at != rocblas_datatype_f32_r && !isnan(alpha_s.host) && !isnan(beta_s.host)) {
    const LtPlan* p = lt_plan(dev, ta == rocblas_operation_transpose, tb == rocblas_operation_transpose, m, n, k, lda,
                              ldb, ldc, lt_type(at), lt_type(ct));
    if (p) {
      const hipblasStatus_t s = hipblasLtMatmul(g_lt[dev], p->md, &alpha_s.host, A, p->la, B, p->lb, &beta_s.host, C,
                                                p->lc, C, p->lc, &p->algo, nullptr, 0, st);
      return s == HIPBLAS_STATUS_SUCCESS ? CE_OK : CE_ERR_HIP;
    }
  }
  const float* alpha = alpha_s.dev;
  const float* beta = beta_s.dev;
  const rocblas_status s =
      rocblas_gemm_ex(h, ta, tb, (rocblas_int)m, (rocblas_int)n, (rocblas_int)k, alpha, A, at, (rocblas_int)lda, B, bt,
                      (rocblas_int)ldb, beta, C, ct, (rocblas_int)ldc, C, ct, (rocblas_int)ldc,
                      rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
  return s == rocblas_status_success ? CE_OK : CE_ERR_HIP;
}

bool fits32(int64_t x) { return x >= 0 && x < ((int64_t)1 << 31); }

}  // namespace

extern "C" {

size_t ce_linear_workspace_bytes(int64_t n_rows, int64_t hidden_size, int64_t vocab, int64_t chunk_rows,
                                 int dtype) {
  if (!valid_dtype(dtype) || n_rows < 0 || hidden_size < 1 || vocab < 1 || chunk_rows < 0) return 0;
  if (!fits32(n_rows) || !fits32(hidden_size) || !fits32(vocab)) return 0;
  const LinLayout L = lin_layout(n_rows, hidden_size, vocab, chunk_rows, dtype);
  if (L.ce_ws_bytes == 0) return 0;
  return L.total;
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
  const LinLayout L = lin_layout(N, H, V, chunk_rows, dtype);
  if (L.ce_ws_bytes == 0) return CE_ERR_UNSUPPORTED;
  if (workspace == nullptr || workspace_bytes < L.total || (uintptr_t)workspace % 256) return CE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  char* ws = (char*)workspace;

  if (N == 0) {
    hipLaunchKernelGGL(lin_empty_kernel, dim3(1), dim3(64), 0, st, loss_mean, n_valid, status);
    if (grad_weight)
      hipLaunchKernelGGL(lin_zero_kernel, dim3((unsigned)V), dim3(256), 0, st, (uint16_t*)grad_weight,
                         ld_grad_weight, H, es);
    return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
  }

  float* logits = (float*)(ws + L.logits);
  float* dl_chunk = (float*)(ws + L.dl_chunk);
  uint32_t* chunk_status = (uint32_t*)(ws + L.chunk_status);
  float* chunk_loss = (float*)(ws + L.chunk_loss);
  int32_t* chunk_n = (int32_t*)(ws + L.chunk_n);
  void* g_lo = (dtype == CE_DTYPE_F32) ? (void*)logits : (void*)(ws + L.g16);
  // the weight gradient: accumulated over chunks in fp32 (the output itself for
  // fp32, else a workspace copy rounded once at the end); a single chunk is
  // written by its GEMM in the output format (fp32 accumulation, one rounding)
  const bool dw_direct = dtype == CE_DTYPE_F32 || L.nc == 1;
  float* dw32 = dw_direct ? (float*)grad_weight : (float*)(ws + L.dw32);
  const int64_t ld_dw = dw_direct ? ld_grad_weight : H;
  const rocblas_datatype dt = blas_type(dtype);
  const float* cs = (const float*)(ws + L.consts);  // 1, 0, 2^-k on the device
  const Scalar one = {cs, 1.0f}, zero = {cs + 1, 0.0f};
  const Scalar down = {cs + 2, dtype == CE_DTYPE_F16 ? NAN : 1.0f};  // 2^-k: k = 0 unless fp16

  hipLaunchKernelGGL(lin_prep_kernel, dim3(1), dim3(kNT), 0, st, labels, N, ignore_index, L.T, L.nc, dloss,
                     dtype == CE_DTYPE_F16 ? 1 : 0, dl_chunk, n_valid, (float*)(ws + L.consts));
  if (hipGetLastError() != hipSuccess) return CE_ERR_HIP;

  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_blas_mu[dev]);
  if (g_blas[dev] == nullptr) {
    if (rocblas_create_handle(&g_blas[dev]) != rocblas_status_success) {
      g_blas[dev] = nullptr;
      return CE_ERR_HIP;
    }
    // GEMM kernels that accumulate with atomics would make results depend on
    // timing: the call is deterministic like the rest of the library
    rocblas_set_atomics_mode(g_blas[dev], rocblas_atomics_not_allowed);
  }
  rocblas_handle bh = g_blas[dev];
  if (rocblas_set_stream(bh, st) != rocblas_status_success ||
      rocblas_set_pointer_mode(bh, rocblas_pointer_mode_device) != rocblas_status_success)
    return CE_ERR_HIP;

  const char* hb = (const char*)hidden;
  int rc = CE_OK;
  for (int c = 0; c < L.nc && rc == CE_OK; ++c) {
    const int64_t r0 = (int64_t)c * L.T;
    const int64_t Tc = (N - r0 < L.T) ? N - r0 : L.T;
    const void* hc = hb + r0 * ld_hidden * es;
    // 1. logits_c [Tc x V] = h_c W^T  (column-major: V x Tc = (H x V)^T (H x Tc))
    rc = gemm(dev, bh, st, rocblas_operation_transpose, rocblas_operation_none, V, Tc, H, one, weight, dt, ld_weight,
              hc, dt, ld_hidden, zero, logits, rocblas_datatype_f32_r, V);
    if (rc != CE_OK) break;
    // 2-3. the chunk's losses and g: for bf16 / fp16 one kernel reads the fp32
    // logits and writes g in the input format for the GEMMs; otherwise (fp32,
    // or rows it does not serve) g is written over the fp32 logits and cast
    bool fused = false;
    if (dtype != CE_DTYPE_F32) {
      rc = ce_lin_chunk_f32_to16(logits, V, labels + r0, Tc, V, dtype, ignore_index, dl_chunk + c, chunk_loss + c,
                                 loss_rows + r0, chunk_n + c, chunk_status + c, g_lo, V, ws + L.ce_ws,
                                 L.ce_ws_bytes, st);
      if (rc == CE_OK) fused = true;
      else if (rc != CE_ERR_UNSUPPORTED) break;
    }
    if (!fused) {
      rc = ce_fwd_bwd_inplace(logits, V, labels + r0, Tc, V, CE_DTYPE_F32, ignore_index, 0, dl_chunk + c,
                              chunk_loss + c, loss_rows + r0, nullptr, nullptr, chunk_n + c, chunk_status + c,
                              ws + L.ce_ws, L.ce_ws_bytes, st);
      if (rc != CE_OK) break;
      if (dtype == CE_DTYPE_BF16)
        hipLaunchKernelGGL(lin_cast_kernel<__bf16>, dim3((unsigned)Tc), dim3(256), 0, st, logits, V, V,
                           (__bf16*)g_lo, V, (const float*)nullptr);
      else if (dtype == CE_DTYPE_F16)
        hipLaunchKernelGGL(lin_cast_kernel<_Float16>, dim3((unsigned)Tc), dim3(256), 0, st, logits, V, V,
                           (_Float16*)g_lo, V, (const float*)nullptr);
      if (hipGetLastError() != hipSuccess) {
        rc = CE_ERR_HIP;
        break;
      }
    }
    if (grad_hidden == nullptr && grad_weight == nullptr) continue;
    // 4. dh_c [Tc x H] = g W  (column-major: H x Tc = (H x V)(V x Tc))
    if (grad_hidden) {
      rc = gemm(dev, bh, st, rocblas_operation_none, rocblas_operation_none, H, Tc, V, down, weight, dt, ld_weight,
                g_lo, dt, V, zero, (char*)grad_hidden + r0 * ld_grad_hidden * es, dt, ld_grad_hidden);
      if (rc != CE_OK) break;
    }
    // 5. dW [V x H] += g^T h_c  (column-major: H x V = (H x Tc)(Tc x V)): NT on
    // the stored operands, or TN on transposed copies gT [V x Tc], hT [H x Tc]
    if (grad_weight) {
      rocblas_operation oa = rocblas_operation_none, ob = rocblas_operation_transpose;
      const void *A = hc, *B = g_lo;
      int64_t lda = ld_hidden, ldb = V;
      if (L.tn && (uintptr_t)hc % 16 == 0 && ld_hidden % 8 == 0) {
        uint16_t* gT = (uint16_t*)(ws + L.gT);
        uint16_t* hT = (uint16_t*)(ws + L.hT);
        hipLaunchKernelGGL(lin_transpose16_kernel, dim3((unsigned)(V / 64), (unsigned)(Tc / 64)), dim3(256), 0, st,
                           (const uint16_t*)g_lo, V, gT, Tc);
        hipLaunchKernelGGL(lin_transpose16_kernel, dim3((unsigned)(H / 64), (unsigned)(Tc / 64)), dim3(256), 0, st,
                           (const uint16_t*)hc, ld_hidden, hT, Tc);
        if (hipGetLastError() != hipSuccess) {
          rc = CE_ERR_HIP;
          break;
        }
        oa = rocblas_operation_transpose;
        ob = rocblas_operation_none;
        A = hT;
        B = gT;
        lda = ldb = Tc;
      }
      if (dw_direct)  // fp32: accumulate in the output; one 16-bit chunk: scale by 2^-k and round once
        rc = gemm(dev, bh, st, oa, ob, H, V, Tc, dtype == CE_DTYPE_F32 ? one : down, A, dt, lda, B, dt, ldb,
                  c == 0 ? zero : one, dw32, dtype == CE_DTYPE_F32 ? rocblas_datatype_f32_r : dt, ld_dw);
      else
        rc = gemm(dev, bh, st, oa, ob, H, V, Tc, one, A, dt, lda, B, dt, ldb, c == 0 ? zero : one, dw32,
                  rocblas_datatype_f32_r, ld_dw);
      if (rc != CE_OK) break;
    }
  }
  if (rc != CE_OK) return rc;
  if (grad_weight && !dw_direct) {
    if (dtype == CE_DTYPE_BF16)
      hipLaunchKernelGGL(lin_cast_kernel<__bf16>, dim3((unsigned)V), dim3(256), 0, st, dw32, H, H,
                         (__bf16*)grad_weight, ld_grad_weight, down.dev);
    else
      hipLaunchKernelGGL(lin_cast_kernel<_Float16>, dim3((unsigned)V), dim3(256), 0, st, dw32, H, H,
                         (_Float16*)grad_weight, ld_grad_weight, down.dev);
  }
  hipLaunchKernelGGL(lin_finish_kernel, dim3(1), dim3(kNT), 0, st, loss_rows, labels, N, ignore_index, n_valid,
                     chunk_status, L.nc, loss_mean, status);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

}  // extern "C"
