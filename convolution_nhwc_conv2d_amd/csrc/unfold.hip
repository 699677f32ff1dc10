// Explicit unfold (im2col) for gfx950: one chunk of output rows at a time.
//
// MLX PR "Use the explicit gemm for wide convs on neural accelerators", intro:
// unfolding costs an extra pass over the input (about 2*M*K elements moved)
// before a dense GEMM; Notes: the unfold is tiled against a buffer limit and
// the one buffer is reused chunk after chunk.  This kernel is a pure copy, so
// it is HBM-bound: consecutive threads move consecutive 16-byte vectors of a
// row, each vector a contiguous channel run of one filter tap of the NHWC
// input (or zeros outside the image and in the pad columns k >= K).
//   buf[r][k], r = 0..rows-1 for output row m0 + r, k = (kh*KW + kw)*C + c,
//   row stride kp (K rounded up to 16 bytes).
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "device_common.hpp"

namespace cnhwc {
namespace {

struct UnfoldGeo {
  int64_t h, w, c, oh, ow, kh, kw;
  int32_t sh, sw, ph, pw, dh, dw;
  int64_t m0, rows, kp;
};

// One 16-byte vector per thread (requires C % VE == 0).
template <typename E>
__global__ __launch_bounds__(256) void unfold_vec_kernel(const E* __restrict__ x, UnfoldGeo g,
                                                         E* __restrict__ buf, int64_t total) {
  constexpr int VE = 16 / sizeof(E);
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t nv = g.kp / VE;
  const int64_t r = t / nv, v = t - r * nv;
  const int64_t k = v * VE;
  const int64_t m = g.m0 + r;
  const int64_t hw = g.oh * g.ow;
  const int64_t n = m / hw, rem = m - n * hw;
  const int64_t oh = rem / g.ow, ow = rem - oh * g.ow;
  const int64_t tap = k / g.c, c = k - tap * g.c;
  uint4 val = make_uint4(0, 0, 0, 0);
  if (tap < g.kh * g.kw) {
    const int64_t a = tap / g.kw, b = tap - a * g.kw;
    const int64_t ih = oh * g.sh - g.ph + a * g.dh;
    const int64_t iw = ow * g.sw - g.pw + b * g.dw;
    if (ih >= 0 && ih < g.h && iw >= 0 && iw < g.w)
      val = *reinterpret_cast<const uint4*>(x + ((n * g.h + ih) * g.w + iw) * g.c + c);
  }
  *reinterpret_cast<uint4*>(buf + r * g.kp + k) = val;
}

// One 16-byte vector of a row per thread for any C (C % VE != 0, e.g. the
// 3-channel stem): the (tap, channel) of the vector's first element comes from
// one division chain, the rest are walked from it; the elements are gathered
// one by one and stored as one vector.
template <typename E>
__global__ __launch_bounds__(256) void unfold_gather_kernel(const E* __restrict__ x, UnfoldGeo g,
                                                            E* __restrict__ buf, int64_t total) {
  constexpr int VE = 16 / sizeof(E);
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t nv = g.kp / VE;
  const int64_t r = t / nv, v = t - r * nv;
  const int64_t k0 = v * VE;
  const int64_t m = g.m0 + r;
  const int64_t hw = g.oh * g.ow;
  const int64_t n = m / hw, rem = m - n * hw;
  const int64_t oh = rem / g.ow, ow = rem - oh * g.ow;
  const int64_t ih0 = oh * g.sh - g.ph, iw0 = ow * g.sw - g.pw;
  const E* __restrict__ xn = x + n * g.h * g.w * g.c;
  int64_t tap = k0 / g.c, c = k0 - tap * g.c;
  int64_t a = tap / g.kw, b = tap - a * g.kw;  // a >= kh: past K (pad columns)
  E e[VE];
#pragma unroll
  for (int i = 0; i < VE; ++i) {
    E val = E(0);
    if (a < g.kh) {
      const int64_t ih = ih0 + a * g.dh, iw = iw0 + b * g.dw;
      if (ih >= 0 && ih < g.h && iw >= 0 && iw < g.w) val = xn[(ih * g.w + iw) * g.c + c];
    }
    e[i] = val;
    if (++c == g.c) {
      c = 0;
      if (++b == g.kw) {
        b = 0;
        ++a;
      }
    }
  }
  *reinterpret_cast<uint4*>(buf + r * g.kp + k0) = *reinterpret_cast<const uint4*>(e);
}

template <typename E>
hipError_t launch_unfold_t(const void* x, const UnfoldGeo& g, void* buf, hipStream_t s) {
  constexpr int VE = 16 / sizeof(E);
  if (g.c % VE == 0) {
    const int64_t total = g.rows * (g.kp / VE);
    hipLaunchKernelGGL((unfold_vec_kernel<E>), dim3(unsigned((total + 255) / 256)), dim3(256), 0, s,
                       static_cast<const E*>(x), g, static_cast<E*>(buf), total);
  } else {
    const int64_t total = g.rows * (g.kp / VE);
    hipLaunchKernelGGL((unfold_gather_kernel<E>), dim3(unsigned((total + 255) / 256)), dim3(256), 0,
                       s, static_cast<const E*>(x), g, static_cast<E*>(buf), total);
  }
  return hipGetLastError();
}

}  // namespace

int unfold_launch(int dtype, const void* x, int64_t h, int64_t w, int64_t c, int64_t oh,
                  int64_t ow, int64_t kh, int64_t kw, int32_t sh, int32_t sw, int32_t ph,
                  int32_t pw, int32_t dh, int32_t dw, int64_t m0, int64_t rows, int64_t kp,
                  void* buf, void* stream) {
  if (rows <= 0) return hipSuccess;
  const UnfoldGeo g{h, w, c, oh, ow, kh, kw, sh, sw, ph, pw, dh, dw, m0, rows, kp};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return dtype == CNHWC_F32 ? launch_unfold_t<float>(x, g, buf, s)
                            : launch_unfold_t<uint16_t>(x, g, buf, s);
}

}  // namespace cnhwc
