// calib_copy.hip -- a plain device copy of known size, used only to calibrate
// the rocprofv3 FETCH_SIZE / WRITE_SIZE counters for the benchmark's traffic
// figure.  It issues the same 16-byte nontemporal loads and stores as the
// cross-entropy kernels, so the counters see the same request mix.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void calib_copy_kernel(const u32x4* src, u32x4* dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Copies `bytes` (a multiple of 16; both pointers 16-byte aligned) on `stream`.
// Returns 0, or 1 for bad arguments, 2 for a launch failure.
extern "C" int ce_calib_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst || bytes % 16 || ((uintptr_t)src | (uintptr_t)dst) % 16) return 1;
  const int64_t n = (int64_t)(bytes / 16);
  if (n == 0) return 0;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(calib_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
