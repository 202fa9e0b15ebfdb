// Device helpers shared by the gfx950 kernels of the GDN beam-decode library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

namespace onela {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// float32 -> bfloat16 bits, round to nearest with ties to even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits_rne(float x) {
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Loads of one element of q/k/v as float32, for either input dtype.
__device__ __forceinline__ float load_in(const float* p, size_t i) { return p[i]; }
__device__ __forceinline__ float load_in(const uint16_t* p, size_t i) { return bf16_bits_to_f32(p[i]); }

// Sum over the 16 lanes of each DPP row; every lane of the row receives the row's sum.
// Steps: swap neighbours (quad_perm 1,0,3,2), swap pairs (quad_perm 2,3,0,1), mirror within each half
// row, mirror within the row.  All 16 lanes of a row must be active.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, true));
  return x;
}

// Sum over each group of 8 lanes (the first three steps of row16_sum); every lane of the group receives it.
__device__ __forceinline__ float row8_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, true));
  return x;
}

// Sum over each group of N = 8, 16 or 32 lanes (32: two DPP rows joined by a lane exchange).
template <int N>
__device__ __forceinline__ float rows_sum(float x) {
  if constexpr (N == 32) {
    x = row16_sum(x);
    return x + __shfl_xor(x, 16, 64);
  } else if constexpr (N == 16) {
    return row16_sum(x);
  } else {
    return row8_sum(x);
  }
}

// Sum over a full 64-lane wave; every lane receives it.
__device__ __forceinline__ float wave_sum(float x) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// Dot product of two vectors of 8 bfloat16 each (packed in 4 dwords), accumulated in float32.
// Each dword is copied to a scalar before the bit cast: a bit cast applied directly to an element of an
// ext_vector_type value has been compiled as a read of element 0.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float dot8_bf16(u32x4_t a, u32x4_t b) {
  const uint32_t a0 = a.x, a1 = a.y, a2 = a.z, a3 = a.w;
  const uint32_t b0 = b.x, b1 = b.y, b2 = b.z, b3 = b.w;
  float s = dot2_bf16(a0, b0, 0.f);
  s = dot2_bf16(a1, b1, s);
  s = dot2_bf16(a2, b2, s);
  s = dot2_bf16(a3, b3, s);
  return s;
}

}  // namespace onela
