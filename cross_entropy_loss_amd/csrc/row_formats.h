// row_formats.h -- 16-bit element formats for the row kernels (RMSNorm,
// RoPE): the two halves of a 32-bit word as floats, and two floats rounded to
// nearest even into one word.  Words are taken by value (clang reads element 0
// when a bit cast is applied directly to an ext-vector element expression).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rowfmt {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf2 __attribute__((ext_vector_type(2)));

struct BF16 {
  __device__ static float lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
  __device__ static float hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xffff0000u); }
  __device__ static uint32_t pack(float a, float b) {
    f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
  }
};
struct F16 {
  __device__ static float lo(uint32_t u) { return (float)__builtin_bit_cast(h2, u).x; }
  __device__ static float hi(uint32_t u) { return (float)__builtin_bit_cast(h2, u).y; }
  __device__ static uint32_t pack(float a, float b) {
    f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  }
};

__device__ __forceinline__ float as_f(uint32_t u) { return __builtin_bit_cast(float, u); }

}  // namespace rowfmt
