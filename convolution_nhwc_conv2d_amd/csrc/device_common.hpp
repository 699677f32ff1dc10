// Device helpers shared by the gfx950 kernels: vector types, the matrix-core
// builtins, and conversions between fp32 and the 16-bit storage types.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

namespace cnhwc {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// D += A * B on a 32x32 block with 16-deep K from 8 fp16/bf16 values per lane.
template <bool BF16>
__device__ __forceinline__ v16f mfma_32x32x16(uint4 a, uint4 b, v16f c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a),
                                                   __builtin_bit_cast(v8bf, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a),
                                                  __builtin_bit_cast(v8h, b), c, 0, 0, 0);
  }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));  // IEEE RNE
}

template <typename E, bool BF16>
__device__ __forceinline__ E from_f32(float v) {
  if constexpr (std::is_same<E, float>::value) {
    return v;
  } else {
    return BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
  }
}

template <typename E, bool BF16>
__device__ __forceinline__ float to_f32(E v) {
  if constexpr (std::is_same<E, float>::value) {
    return v;
  } else if constexpr (BF16) {
    return __builtin_bit_cast(float, uint32_t(v) << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, v));
  }
}

}  // namespace cnhwc
