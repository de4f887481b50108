// ce_api.hip -- the C ABI declared in include/ce_mi355x.h: host-side argument
// checks, workspace layout, kernel choice and launches on the caller's stream.
// Every step of the computation runs in the kernels of ce_kernels.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "ce_kernels.h"
#include "ce_mi355x.h"

namespace {

using cek::Args;
typedef void (*KernelFn)(Args);

#ifndef CE_POL
#define CE_POL 3  // nontemporal loads and stores (measured fastest for the fused rows)
#endif
constexpr int kPol = CE_POL;
constexpr int64_t kMaxRows = 0x7fffffff;

int esize(int dtype) { return dtype == CE_DTYPE_F32 ? 4 : 2; }
int epv(int dtype) { return 16 / esize(dtype); }

// Largest row (or slab) the on-chip kernels hold: 1024 lanes x 16 vectors.
int64_t max_slab(int dtype) { return (int64_t)1024 * 16 * epv(dtype); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Vocabulary split: C slabs of width `width` (C == 1: whole rows on chip).
// A row that fits on chip is read once whatever `chunk` is: its workgroup
// already merges (max, sum) partials of many lanes and waves, a finer
// partition of the same log-sum-exp merge, and the result differs from a
// per-chunk merge only by rounding.  The fused 16-bit rows wider than 64K
// elements reduce two chunks separately and merge them when `chunk` is half
// the workgroup's capacity (65536); other on-chip widths reduce the row
// whole.  Rows wider than on-chip capacity are cut into slabs of width
// `chunk` (default 65536 16-bit / 32768 fp32 elements) whose partials are
// merged per row.
struct Split {
  int64_t width;
  int C;
};
bool make_split(int64_t V, int64_t chunk, int dtype, Split* s) {
  const int64_t cap = max_slab(dtype);
  int64_t w;
  if (V <= cap) w = V;
  else if (chunk == 0 || chunk >= V) w = (dtype == CE_DTYPE_F32) ? 32768 : 65536;
  else w = chunk;
  if (w > cap) return false;
  s->width = w;
  s->C = (int)((V + w - 1) / w);
  return true;
}

// Workspace: header, tagged per-row loss slots, then (chunked only) slab
// partials, label logits and fp64 scratch for the row statistics.
struct WsLayout {
  size_t slots, slab_ms, slab_xy, lse_scratch, pcomp_scratch, total;
};
WsLayout ws_layout(int64_t N, const Split& sp) {
  WsLayout L;
  size_t off = cek::kWsHeaderBytes;
  L.slab_ms = L.slab_xy = L.lse_scratch = L.pcomp_scratch = 0;
  L.slots = off;
  off += align256((size_t)N * sizeof(uint64_t));
  if (sp.C > 1) {
    L.slab_ms = off;
    off += align256((size_t)N * sp.C * sizeof(double2));
    L.slab_xy = off;
    off += align256((size_t)N * sizeof(float));
    L.lse_scratch = off;
    off += align256((size_t)N * sizeof(double));
    L.pcomp_scratch = off;
    off += align256((size_t)N * sizeof(double));
  }
  L.total = off;
  return L;
}

bool valid_dtype(int d) { return d == CE_DTYPE_F32 || d == CE_DTYPE_BF16 || d == CE_DTYPE_F16; }

// Checks shared by every entry point.
int check_shape(const void* logits, int64_t ld, const int64_t* labels, int64_t N, int64_t V, int dtype) {
  if (!valid_dtype(dtype)) return CE_ERR_DTYPE;
  if (N < 0 || N > kMaxRows || V < 1 || V > kMaxRows || ld < V) return CE_ERR_INVALID_ARG;
  if (ld > ((int64_t)1 << 40)) return CE_ERR_INVALID_ARG;
  if (N > 0 && (logits == nullptr || labels == nullptr)) return CE_ERR_INVALID_ARG;
  if (((uintptr_t)logits) % esize(dtype) != 0) return CE_ERR_INVALID_ARG;
  if (((uintptr_t)labels) % 8 != 0) return CE_ERR_INVALID_ARG;
  return CE_OK;
}

int counters_for(int64_t N, int64_t G) {
  int64_t k = (N + 1023) / 1024;
  if (k < 1) k = 1;
  if (k > cek::kMaxCounters) k = cek::kMaxCounters;
  if (k > G) k = G;
  return (int)k;
}

// Co-resident workgroups of a kernel on the current device (cached per device
// and kernel; the cache is shared by every host thread, hence the lock).
int64_t resident_blocks(KernelFn fn, int block) {
  struct Entry {
    int dev;
    KernelFn fn;
    int block;
    int64_t val;
  };
  static std::mutex mu;
  static Entry cache[64];
  static int n = 0;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < n; ++i)
      if (cache[i].dev == dev && cache[i].fn == fn && cache[i].block == block) return cache[i].val;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, block, 0) != hipSuccess) return 0;
  const int64_t r = (int64_t)cus * per_cu;
  std::lock_guard<std::mutex> lock(mu);
  if (n < 64) cache[n++] = Entry{dev, fn, block, r};
  return r;
}

// Persistent grid for N rows: no more workgroups than are co-resident, and
// the same number of rows for every workgroup where N allows it.
int64_t persistent_grid(KernelFn fn, int block, int64_t N) {
  int64_t cap = resident_blocks(fn, block);
  if (cap <= 0 || cap > N) return N;
  const int64_t per = (N + cap - 1) / cap;
  return (N + per - 1) / per;
}

int launch(KernelFn fn, int64_t grid, int block, Args a, hipStream_t st) {
  if (grid <= 0) return CE_OK;
  if (grid > 0x7fffffff) return CE_ERR_UNSUPPORTED;
  void* params[] = {&a};
  hipError_t e = hipLaunchKernel((const void*)fn, dim3((unsigned)grid), dim3(block), params, 0, st);
  return e == hipSuccess ? CE_OK : CE_ERR_HIP;
}

// ---- kernel tables ---------------------------------------------------------
struct Cfg {
  int nt, vpl;
};
// Whole-row / slab shapes (lanes x 16-byte vectors per lane), smallest
// capacity first; a row takes the first that holds it.  Measured on the
// 4096 x 32000 bf16 call: 512 x 8 (four rows per CU) 105.7 us, 256 x 16
// 110.3 us, 1024 x 4 142.7 us (its per-wave fixed work is paid 16 times per
// row); on 16384 x 49152 fp16: 512 x 12 554 us, 1024 x 6 676 us.
const Cfg kCfgs[] = {{256, 1}, {256, 2}, {256, 4}, {256, 8}, {512, 8}, {512, 12}, {512, 16}, {1024, 12}, {1024, 16}};

Cfg pick_cfg(int64_t nvec_max) {
  for (const Cfg& c : kCfgs)
    if ((int64_t)c.nt * c.vpl >= nvec_max) return c;
  return kCfgs[sizeof(kCfgs) / sizeof(kCfgs[0]) - 1];
}

#define CE_CFG_CASES(MAKE)                                                                               \
  MAKE(256, 1) MAKE(256, 2) MAKE(256, 4) MAKE(256, 8) MAKE(512, 8) MAKE(512, 12) MAKE(512, 16) MAKE(1024, 12) \
  MAKE(1024, 16)

template <typename T, bool FUSED>
KernelFn row16_fn(Cfg c) {
#define MAKE(NT, VPL) \
  if (c.nt == NT && c.vpl == VPL) return cek::row_kernel_16<T, NT, VPL, kPol, FUSED>;
  CE_CFG_CASES(MAKE)
#undef MAKE
  return nullptr;
}
template <typename T>
KernelFn aligned_fn(Cfg c) {
#define MAKE(NT, VPL) \
  if (c.nt == NT && c.vpl == VPL) return cek::row_fused_aligned<T, NT, VPL, kPol>;
  CE_CFG_CASES(MAKE)
#undef MAKE
  return nullptr;
}
// Two vocabulary chunks of half the vector slots each (1024 lanes x 8 slots
// x 8 elements = 65536 16-bit elements per chunk).
template <typename T>
KernelFn aligned2_fn(Cfg c) {
  if (c.nt == 1024 && c.vpl == 16) return cek::row_fused_aligned<T, 1024, 16, kPol, 8>;
  return nullptr;
}
template <bool FUSED>
KernelFn row32_fn(Cfg c) {
#define MAKE(NT, VPL) \
  if (c.nt == NT && c.vpl == VPL) return cek::row_kernel_32<NT, VPL, kPol, FUSED>;
  CE_CFG_CASES(MAKE)
#undef MAKE
  return nullptr;
}
template <typename T>
KernelFn stats_fn(Cfg c) {
#define MAKE(NT, VPL) \
  if (c.nt == NT && c.vpl == VPL) return cek::slab_stats_kernel<T, NT, VPL, kPol>;
  CE_CFG_CASES(MAKE)
#undef MAKE
  return nullptr;
}
template <typename T>
KernelFn slabgrad_fn(Cfg c) {
#define MAKE(NT, VPL) \
  if (c.nt == NT && c.vpl == VPL) return cek::slab_grad_kernel<T, NT, VPL, kPol>;
  CE_CFG_CASES(MAKE)
#undef MAKE
  return nullptr;
}

constexpr int kGradNT = 256, kGradVPL = 4;  // backward slab: 1024 vectors
KernelFn grad_fn(int dtype) {
  if (dtype == CE_DTYPE_BF16) return cek::grad_kernel<cek::BF16, kGradNT, kGradVPL, kPol>;
  if (dtype == CE_DTYPE_F16) return cek::grad_kernel<cek::F16, kGradNT, kGradVPL, kPol>;
  return cek::grad_kernel<cek::F32, kGradNT, kGradVPL, kPol>;
}

KernelFn row_fn(int dtype, bool fused, Cfg c) {
  if (dtype == CE_DTYPE_BF16) return fused ? row16_fn<cek::BF16, true>(c) : row16_fn<cek::BF16, false>(c);
  if (dtype == CE_DTYPE_F16) return fused ? row16_fn<cek::F16, true>(c) : row16_fn<cek::F16, false>(c);
  return fused ? row32_fn<true>(c) : row32_fn<false>(c);
}
KernelFn slab_stats_fn(int dtype, Cfg c) {
  if (dtype == CE_DTYPE_BF16) return stats_fn<cek::BF16>(c);
  if (dtype == CE_DTYPE_F16) return stats_fn<cek::F16>(c);
  return stats_fn<cek::F32>(c);
}
KernelFn slab_grad_fn(int dtype, Cfg c) {
  if (dtype == CE_DTYPE_BF16) return slabgrad_fn<cek::BF16>(c);
  if (dtype == CE_DTYPE_F16) return slabgrad_fn<cek::F16>(c);
  return nullptr;  // fp32 chunked rows take forward + backward
}

// Test hook state (ce_debug_sync_override): a spin limit other than the
// default and extra partial-count words that no workgroup publishes.
std::atomic<int> g_spin_limit{0};
std::atomic<int> g_extra_counters{0};

// K counter workgroups publish; pollers wait for K words (plus any extra
// ones the test hook asks for, which then never arrive).
void set_counters(Args& a, int K) {
  a.K = K;
  int kp = K + g_extra_counters.load(std::memory_order_relaxed);
  if (kp > cek::kMaxCounters) kp = cek::kMaxCounters;
  a.Kpoll = kp;
}

Args base_args(const void* logits, int64_t ld, const int64_t* labels, int64_t N, int64_t V, int64_t ignore,
               void* ws) {
  Args a;
  memset(&a, 0, sizeof(a));
  const int sl = g_spin_limit.load(std::memory_order_relaxed);
  a.spin_limit = sl > 0 ? sl : cek::kSpinLimit;
  a.logits = (char*)logits;
  a.ld = ld;
  a.grad = (char*)logits;
  a.grad_ld = ld;
  a.labels = labels;
  a.N = N;
  a.V = V;
  a.ignore = ignore;
  a.ws = (cek::WsHeader*)ws;
  a.C = 1;
  return a;
}

// Forward (and, when fused, the in-place gradient) of one call.
int run_forward(bool fused, void* logits, int64_t ld, const int64_t* labels, int64_t N, int64_t V, int dtype,
                int64_t ignore, int64_t chunk, const float* dloss, float* loss_mean, float* loss_rows,
                double* lse_rows, double* pcomp_rows, int32_t* n_valid, uint32_t* status, void* ws,
                size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(logits, ld, labels, N, V, dtype);
  if (rc != CE_OK) return rc;
  if (chunk < 0) return CE_ERR_INVALID_ARG;
  if (loss_mean == nullptr || n_valid == nullptr || (N > 0 && loss_rows == nullptr)) return CE_ERR_INVALID_ARG;
  Split sp;
  if (!make_split(V, chunk, dtype, &sp)) return CE_ERR_UNSUPPORTED;
  const WsLayout L = ws_layout(N, sp);
  if (ws == nullptr || ws_bytes < L.total || ((uintptr_t)ws) % 256 != 0) return CE_ERR_WORKSPACE;
  if (N == 0) {
    hipLaunchKernelGGL(cek::empty_call_kernel, dim3(1), dim3(64), 0, st, loss_mean, n_valid, status);
    return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
  }
  Args a = base_args(logits, ld, labels, N, V, ignore, ws);
  a.slots = (uint64_t*)((char*)ws + L.slots);
  a.dloss = dloss;
  a.loss_mean = loss_mean;
  a.loss_rows = loss_rows;
  a.lse_rows = lse_rows;
  a.pcomp_rows = pcomp_rows;
  a.n_valid_out = n_valid;
  a.status = status;
  const int e = epv(dtype);
  if (sp.C == 1) {
    const Cfg c = pick_cfg((V + e - 1) / e);
    KernelFn fn = row_fn(dtype, fused, c);
    int64_t G = N;  // one workgroup per row
    // rows wider than 64K 16-bit elements, 16-byte aligned: the persistent
    // buffer-addressed kernel (one 1024-lane workgroup per CU sweeps rows)
    const bool aligned = ((uintptr_t)logits % 16 == 0) && ((ld * esize(dtype)) % 16 == 0) && (V % e == 0);
    if (fused && aligned && dtype != CE_DTYPE_F32 && c.nt == 1024) {
      // a chunk of exactly half the workgroup's vector slots: the two chunks'
      // (max, sum) are reduced separately and merged on chip
      const bool two = chunk > 0 && chunk < V && chunk == (int64_t)c.nt * (c.vpl / 2) * e;
      KernelFn f2 = nullptr;
      if (two) f2 = (dtype == CE_DTYPE_BF16) ? aligned2_fn<cek::BF16>(c) : aligned2_fn<cek::F16>(c);
      fn = f2 ? f2 : ((dtype == CE_DTYPE_BF16) ? aligned_fn<cek::BF16>(c) : aligned_fn<cek::F16>(c));
      G = persistent_grid(fn, c.nt, N);
    }
    set_counters(a, counters_for(N, G));
    return launch(fn, G, c.nt, a, st);
  }
  // chunked: per-slab statistics, then merge (+ gradient)
  char* wsb = (char*)ws;
  a.slab_ms = (double2*)(wsb + L.slab_ms);
  a.slab_xy = (float*)(wsb + L.slab_xy);
  a.chunk = sp.width;
  a.C = sp.C;
  const Cfg c = pick_cfg((sp.width + e - 1) / e);
  const int64_t G = N * sp.C;
  set_counters(a, counters_for(N, G));
  rc = launch(slab_stats_fn(dtype, c), G, c.nt, a, st);
  if (rc != CE_OK) return rc;
  if (fused && dtype != CE_DTYPE_F32) return launch(slab_grad_fn(dtype, c), G, c.nt, a, st);
  if (fused) {  // fp32: row statistics first, then the elementwise backward
    if (!a.lse_rows) a.lse_rows = (double*)(wsb + L.lse_scratch);
    if (!a.pcomp_rows) a.pcomp_rows = (double*)(wsb + L.pcomp_scratch);
  }
  rc = launch(cek::slab_merge_kernel<64>, N, 64, a, st);
  if (rc != CE_OK || !fused) return rc;
  Args b = a;
  b.lse_in = a.lse_rows;
  b.pcomp_in = a.pcomp_rows;
  b.n_valid_in = n_valid;
  b.C = (int)(((V + e - 1) / e + kGradNT * kGradVPL - 1) / (kGradNT * kGradVPL));
  return launch(grad_fn(dtype), N * (int64_t)b.C, kGradNT, b, st);
}

// ---- the allocation-free entry point ---------------------------------------
// Its workspace is this file-scope device array, one copy per GPU, held until
// the process ends.  Host code never passes the array's name to a kernel (on
// the host it is a stand-in symbol, not a device address): the device
// address of each GPU's copy is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept below.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  int rc = CE_ERR_HIP;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address; on first use on a device, the lookup
// and a zero fill enqueued on `st` (the workspace protocol starts from zero).
int device_scratch(hipStream_t st, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CE_ERR_HIP;
  ScratchSlot& sl = g_scratch[dev];
  std::call_once(sl.once, [&] {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return;
    hipLaunchKernelGGL(cek::ws_fill_kernel, dim3(256), dim3(256), 0, st, (uint32_t*)p, kScratchBytes / 4);
    if (hipGetLastError() != hipSuccess) return;
    sl.ptr = p;
    sl.rc = CE_OK;
  });
  *out = sl.ptr;
  return sl.rc;
}

}  // namespace

extern "C" {

int ce_fwd_bwd_inplace_noalloc(void* logits, int64_t ld, const int64_t* labels, int64_t n_rows, int64_t vocab,
                               int dtype, int64_t ignore_index, int64_t chunk, const float* dloss, float* loss_mean,
                               float* loss_rows, double* lse_rows, double* pcomp_rows, int32_t* n_valid,
                               uint32_t* status, void* stream) {
  int rc = check_shape(logits, ld, labels, n_rows, vocab, dtype);
  if (rc != CE_OK) return rc;
  if (chunk < 0) return CE_ERR_INVALID_ARG;
  Split sp;
  if (!make_split(vocab, chunk, dtype, &sp)) return CE_ERR_UNSUPPORTED;
  if (ws_layout(n_rows, sp).total > kScratchBytes) return CE_ERR_SCRATCH;
  void* ws = nullptr;
  rc = device_scratch((hipStream_t)stream, &ws);
  if (rc != CE_OK) return rc;
  return run_forward(true, logits, ld, labels, n_rows, vocab, dtype, ignore_index, chunk, dloss, loss_mean,
                     loss_rows, lse_rows, pcomp_rows, n_valid, status, ws, kScratchBytes, (hipStream_t)stream);
}

int ce_abi_version(void) { return CE_ABI_VERSION; }

int ce_debug_sync_override(int spin_limit, int extra_counters) {
  if (spin_limit < 0 || extra_counters < 0 || extra_counters > cek::kMaxCounters) return CE_ERR_INVALID_ARG;
  g_spin_limit.store(spin_limit, std::memory_order_relaxed);
  g_extra_counters.store(extra_counters, std::memory_order_relaxed);
  return CE_OK;
}

const char* ce_error_string(int code) {
  switch (code) {
    case CE_OK: return "ok";
    case CE_ERR_INVALID_ARG: return "invalid argument (size, stride, pointer or alignment)";
    case CE_ERR_DTYPE: return "unknown dtype";
    case CE_ERR_WORKSPACE: return "workspace missing, misaligned or smaller than ce_workspace_bytes()";
    case CE_ERR_UNSUPPORTED: return "request not served by this library";
    case CE_ERR_HIP: return "HIP runtime error";
    case CE_ERR_SCRATCH: return "request needs more than the allocation-free entry point's 8 MiB static scratch";
    default: return "unknown error code";
  }
}

size_t ce_workspace_bytes(int64_t n_rows, int64_t vocab, int64_t chunk, int dtype) {
  if (!valid_dtype(dtype) || n_rows < 0 || n_rows > kMaxRows || vocab < 1 || vocab > kMaxRows || chunk < 0) return 0;
  Split sp;
  if (!make_split(vocab, chunk, dtype, &sp)) return 0;
  return ws_layout(n_rows, sp).total;
}

int ce_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (workspace == nullptr || workspace_bytes < cek::kWsHeaderBytes || ((uintptr_t)workspace) % 256 != 0)
    return CE_ERR_WORKSPACE;
  const size_t words = workspace_bytes / 4;
  int64_t blocks = (int64_t)((words + 255) / 256);
  if (blocks > 1024) blocks = 1024;
  hipLaunchKernelGGL(cek::ws_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t*)workspace, words);
  return hipGetLastError() == hipSuccess ? CE_OK : CE_ERR_HIP;
}

int ce_forward(const void* logits, int64_t ld, const int64_t* labels, int64_t n_rows, int64_t vocab, int dtype,
               int64_t ignore_index, int64_t chunk, float* loss_mean, float* loss_rows, double* lse_rows,
               double* pcomp_rows, int32_t* n_valid, uint32_t* status, void* workspace, size_t workspace_bytes,
               void* stream) {
  return run_forward(false, (void*)logits, ld, labels, n_rows, vocab, dtype, ignore_index, chunk, nullptr,
                     loss_mean, loss_rows, lse_rows, pcomp_rows, n_valid, status, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

int ce_fwd_bwd_inplace(void* logits, int64_t ld, const int64_t* labels, int64_t n_rows, int64_t vocab, int dtype,
                       int64_t ignore_index, int64_t chunk, const float* dloss, float* loss_mean, float* loss_rows,
                       double* lse_rows, double* pcomp_rows, int32_t* n_valid, uint32_t* status, void* workspace,
                       size_t workspace_bytes, void* stream) {
  return run_forward(true, logits, ld, labels, n_rows, vocab, dtype, ignore_index, chunk, dloss, loss_mean,
                     loss_rows, lse_rows, pcomp_rows, n_valid, status, workspace, workspace_bytes,
                     (hipStream_t)stream);
}

int ce_backward(const void* logits, int64_t ld, const int64_t* labels, const double* lse_rows,
                const double* pcomp_rows, const int32_t* n_valid, const float* dloss, int64_t n_rows, int64_t vocab,
                int dtype, int64_t ignore_index, void* grad, int64_t grad_ld, void* stream) {
  int rc = check_shape(logits, ld, labels, n_rows, vocab, dtype);
  if (rc != CE_OK) return rc;
  if (n_rows == 0) return CE_OK;
  if (lse_rows == nullptr || pcomp_rows == nullptr || n_valid == nullptr || grad == nullptr || grad_ld < vocab)
    return CE_ERR_INVALID_ARG;
  const int es = esize(dtype);
  if (((uintptr_t)grad) % es != 0) return CE_ERR_INVALID_ARG;
  const uintptr_t lo = (uintptr_t)logits, go = (uintptr_t)grad;
  if (go == lo) {
    if (grad_ld != ld) return CE_ERR_INVALID_ARG;
  } else {
    const uintptr_t lend = lo + (uintptr_t)((n_rows - 1) * ld + vocab) * es;
    const uintptr_t gend = go + (uintptr_t)((n_rows - 1) * grad_ld + vocab) * es;
    if (go < lend && lo < gend) return CE_ERR_INVALID_ARG;  // partial overlap
  }
  Args a = base_args(logits, ld, labels, n_rows, vocab, ignore_index, nullptr);
  a.grad = (char*)grad;
  a.grad_ld = grad_ld;
  a.lse_in = lse_rows;
  a.pcomp_in = pcomp_rows;
  a.n_valid_in = n_valid;
  a.dloss = dloss;
  const int e = epv(dtype);
  a.C = (int)(((vocab + e - 1) / e + kGradNT * kGradVPL - 1) / (kGradNT * kGradVPL));
  return launch(grad_fn(dtype), n_rows * (int64_t)a.C, kGradNT, a, (hipStream_t)stream);
}

}  // extern "C"
