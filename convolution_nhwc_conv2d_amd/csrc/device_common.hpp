// Device helpers shared by the gfx950 kernels: vector types, the matrix-core
// builtins, conversions between fp32 and the 16-bit storage types, the
// constant-matrix product of the Winograd transforms and the XCD-contiguous
// workgroup order.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>
#include <type_traits>

namespace cnhwc {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));
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

// out[i] = sum_k Mat[i][k] * in[k] (k ascending), zero coefficients skipped.
template <int R, int C>
__device__ __forceinline__ void cmatvec(const float (&mat)[R][C], const float (&in)[C], float (&out)[R]) {
#pragma unroll
  for (int i = 0; i < R; ++i) {
    float s = 0.0f;
    bool first = true;
#pragma unroll
    for (int k = 0; k < C; ++k) {
      const float m = mat[i][k];
      if (m != 0.0f) {
        const float t = (m == 1.0f) ? in[k] : (m == -1.0f) ? -in[k] : m * in[k];
        s = first ? t : s + t;
        first = false;
      }
    }
    out[i] = s;
  }
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Remap so that XCD x runs one contiguous range of logical workgroups:
// neighbouring Winograd tiles, whose input windows overlap by two pixels, then
// share an L2.  A bijection on [0, gridDim.x) for round-robin dispatch.
__device__ __forceinline__ int64_t xcd_block(int64_t bid, int64_t nwg) {
  constexpr int64_t kXcd = 8;
  const int64_t x = bid % kXcd, k = bid / kXcd;
  const int64_t q = nwg / kXcd, r = nwg % kXcd;
  const int64_t start = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return start + k;
}

}  // namespace cnhwc
