// ce_buffer.h -- raw buffer-resource helpers for gfx950 row kernels (the
// cross-entropy kernels and the RMSNorm kernels).
//
// A buffer resource per row (SGPRs: base, byte size) lets every access use
// one per-lane VGPR offset plus a per-vector SGPR offset, and its size bounds
// every access: loads past the row return 0 and stores past it are dropped.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cek {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufFlags = 0x00020000;  // raw 32-bit dword buffer, gfx9 layout

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, kBufFlags);
}
// aux bits of buffer instructions on gfx94x/gfx950: sc0 = 1, nt = 2, sc1 = 16
template <int POL>
constexpr int aux_load() { return (POL & 1) ? 2 : 0; }
template <int POL>
constexpr int aux_store() { return (POL & 2) ? 2 : 0; }

// A 128-bit buffer store.  The hardware reads a store's data registers after
// the instruction issues, and a VALU write to them must wait two cycles; the
// compiler leaves no such gap when the store's soffset is a register (it
// assumes the hazard only exists without one), and a gradient vector built in
// the same registers right after a store then reached memory in part.  Two
// wait states follow every store here, kept in place by scheduling barriers.
template <int AUX>
__device__ __forceinline__ void buf_store(u32x4 v, __amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, v), rs, voff, soff,
                                         AUX);
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 1");
  __builtin_amdgcn_sched_barrier(0);
}

}  // namespace cek
