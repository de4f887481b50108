// calib_copy.hip -- plain device copies and reads of known size.  The
// benchmark times several shapes of each and takes the fastest as the
// attainable rate for that size (the ceiling the kernels' rates are set
// against), and uses the counters of a copy to calibrate rocprofv3's
// FETCH_SIZE / WRITE_SIZE for its traffic figure.
//
// Copy shapes (16-byte vectors):
//   0  grid-stride, one vector per thread per pass, at most 16384 workgroups,
//      nontemporal loads and stores (the kernels' request mix)
//   1  one vector per thread, a workgroup per 256 vectors (no grid cap), nontemporal
//   2  four vectors per thread, all four loads before the stores, nontemporal
//   3  eight vectors per thread, nontemporal
//   4  four vectors per thread, ordinary (cached) loads and stores
//   5  persistent: 8 workgroups per CU, each thread four vectors per pass, nontemporal
// Read shapes: the same with the stores replaced by an xor into a register
// (written out only if it equals a value no input can give).
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int kShapes = 6;

// NT is resolved at compile time: a run-time select between the two forms
// would let the compiler merge the loads and drop the nontemporal hint.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const u32x4* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}
template <bool NT>
__device__ __forceinline__ void st(u32x4 v, u32x4* p) {
  if constexpr (NT) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// U vectors per thread per pass; a pass covers gridDim.x * 256 * U vectors.
template <int U, bool NT>
__global__ __launch_bounds__(256) void calib_copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  const int64_t pass = (int64_t)gridDim.x * 256 * U;
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += pass) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n ? ld<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      if (i < n) st<NT>(v[u], dst + i);
    }
  }
}
template <int U, bool NT>
__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4* src, int64_t n, uint32_t* sink) {
  const int64_t pass = (int64_t)gridDim.x * 256 * U;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t base = (int64_t)blockIdx.x * 256 * U + threadIdx.x; base < n; base += pass) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * 256;
      v[u] = i < n ? ld<NT>(src + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0xDEADBEEFu && acc.x == 0x12345678u) sink[0] = acc.x;
}

template <int U, bool NT, bool READ>
void run(int64_t g, const u32x4* s, u32x4* d, int64_t n, uint32_t* sink, hipStream_t st) {
  if constexpr (READ) hipLaunchKernelGGL((calib_read_kernel<U, NT>), dim3((unsigned)g), dim3(256), 0, st, s, n, sink);
  else hipLaunchKernelGGL((calib_copy_kernel<U, NT>), dim3((unsigned)g), dim3(256), 0, st, s, d, n);
}

template <bool READ>
int launch(int shape, const void* src, void* dst, int64_t n, uint32_t* sink, hipStream_t st) {
  const u32x4* s = (const u32x4*)src;
  u32x4* d = (u32x4*)dst;
  auto blocks = [&](int64_t per) { return (n + per - 1) / per; };
  int64_t g;
  switch (shape) {
    case 0:
      g = blocks(256);
      if (g > 16384) g = 16384;
      run<1, true, READ>(g, s, d, n, sink, st);
      break;
    case 1:
      g = blocks(256);
      run<1, true, READ>(g, s, d, n, sink, st);
      break;
    case 2:
      g = blocks(1024);
      run<4, true, READ>(g, s, d, n, sink, st);
      break;
    case 3:
      g = blocks(2048);
      run<8, true, READ>(g, s, d, n, sink, st);
      break;
    case 4:
      g = blocks(1024);
      run<4, false, READ>(g, s, d, n, sink, st);
      break;
    default: {
      int dev = 0, cus = 0;
      if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                  hipSuccess)
        return 2;
      g = (int64_t)cus * 8;
      const int64_t need = blocks(1024);
      if (g > need) g = need;
      run<4, true, READ>(g, s, d, n, sink, st);
    }
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // namespace

extern "C" {

// Number of shapes of ce_calib_copy_shape / ce_calib_read_shape.
int ce_calib_shapes(void) { return kShapes; }

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on
// `stream` with copy shape `shape` (0 .. ce_calib_shapes() - 1).  Returns 0,
// or 1 for bad arguments, 2 for a launch failure.
int ce_calib_copy_shape(const void* src, void* dst, size_t bytes, int shape, void* stream) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16 || shape < 0 || shape >= kShapes) return 1;
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return 0;
  if ((n + 255) / 256 > 0x7fffffff) return 1;
  return launch<false>(shape, src, dst, n, nullptr, (hipStream_t)stream);
}

// Reads `bytes` at src (16-byte aligned, a multiple of 16) with read shape
// `shape`; sink: one device word the kernel writes only for an input no
// buffer holds in practice (keeps the loads alive).
int ce_calib_read_shape(const void* src, size_t bytes, int shape, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes % 16 || (uintptr_t)src % 16 || shape < 0 || shape >= kShapes) return 1;
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return 0;
  if ((n + 255) / 256 > 0x7fffffff) return 1;
  return launch<true>(shape, src, nullptr, n, sink, (hipStream_t)stream);
}

// The first shape (the counters' calibration copy).
int ce_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  return ce_calib_copy_shape(src, dst, bytes, 0, stream);
}

}  // extern "C"
