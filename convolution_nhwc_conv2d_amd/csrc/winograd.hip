// Winograd F(6x6,3x3) transforms for gfx950: filter transform, input
// transform and output transform.  The batched GEMMs between them run on the
// MFMA core in gemm.hip.
//
// MLX PR "Bound winograd conv2d working set by tiling the batch", Problem: the
// Winograd conv2d keeps the (padded) input and two GEMM workspaces alive -- an
// input transform into tile-position-major GEMM operands, batched GEMMs over
// the tile positions, and an output transform.  Here the padded copy is never
// made: the input transform reads the NHWC image directly and treats every
// position outside it as zero.  Workspace layouts (fp32 for every input dtype):
//   U [64][O][Cs]       transformed filter, Cs = C rounded up to 8 (zeros)
//   V [64][rows][Cs]    transformed input, rows = images * tiles_per_image
//   M [64][rows][O]     GEMM result per tile position
// Tile r of image n covers input rows 6*ty - ph .. +7 and columns
// 6*tx - pw .. +7 and produces output rows 6*ty .. 6*ty+5 (cropped).
//
// The matrices come from gen_winograd.py (Toom-Cook over 0, +-1, +-2, +-1/2,
// inf).  Products with zero entries are skipped at compile time; every sum
// runs in a fixed order, and each (tile, channel) is handled by exactly one
// thread, so the transforms are elementwise over tiles: their bits do not
// depend on how the batch is tiled.
#include <hip/hip_runtime.h>

#include "wino_f63_api.hpp"
#include "device_common.hpp"
#include "winograd_f63.h"

namespace cnhwc {
namespace {

template <typename E, bool BF16>
__global__ __launch_bounds__(256) void wino_filter_kernel(const E* __restrict__ w, int64_t ldo,
                                                          int64_t O, int64_t C, int64_t Cs,
                                                          float* __restrict__ U) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= O * Cs) return;
  const int64_t o = t / Cs, c = t - o * Cs;
  float g[3][3];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b)
      g[a][b] = c < C ? to_f32<E, BF16>(w[o * ldo + (a * 3 + b) * C + c]) : 0.0f;
  // t1 = G g (8x3), column by column
  float t1[8][3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    float col[3] = {g[0][b], g[1][b], g[2][b]};
    float res[8];
    cmatvec(kWinoG, col, res);
#pragma unroll
    for (int i = 0; i < 8; ++i) t1[i][b] = res[i];
  }
  const int64_t plane = O * Cs;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float row[3] = {t1[i][0], t1[i][1], t1[i][2]};
    float res[8];
    cmatvec(kWinoG, row, res);  // (t1 G^T)[i][j] = sum_b t1[i][b] G[j][b]
#pragma unroll
    for (int j = 0; j < 8; ++j) U[(i * 8 + j) * plane + o * Cs + c] = res[j];
  }
}

template <typename E, bool BF16>
__global__ __launch_bounds__(256) void wino_input_kernel(const E* __restrict__ x, int64_t H,
                                                         int64_t W, int64_t C, int64_t Cs,
                                                         int32_t ph, int32_t pw, int64_t TH,
                                                         int64_t TW, float* __restrict__ V,
                                                         int64_t plane, int64_t total) {
  const int64_t t = xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t r = t / Cs, c = t - r * Cs;
  const int64_t T = TH * TW;
  const int64_t n = r / T, rr = r - n * T;
  const int64_t ty = rr / TW, tx = rr - ty * TW;
  const int64_t ih0 = ty * 6 - ph, iw0 = tx * 6 - pw;
  const E* __restrict__ img = x + n * H * W * C + c;
  const bool cin = c < C;
  // column transform first: t1[a][j] = sum_i BT[a][i] d[i][j]
  float t1[8][8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t iw = iw0 + j;
    const bool wok = cin && iw >= 0 && iw < W;
    float col[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t ih = ih0 + i;
      col[i] = (wok && ih >= 0 && ih < H) ? to_f32<E, BF16>(img[(ih * W + iw) * C]) : 0.0f;
    }
    float res[8];
    cmatvec(kWinoBT, col, res);
#pragma unroll
    for (int a = 0; a < 8; ++a) t1[a][j] = res[a];
  }
  // row transform: v[a][b] = sum_j t1[a][j] BT[b][j]
  float* __restrict__ out = V + r * Cs + c;
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    float res[8];
    cmatvec(kWinoBT, t1[a], res);
#pragma unroll
    for (int b = 0; b < 8; ++b) out[(a * 8 + b) * plane] = res[b];
  }
}

template <typename E, bool BF16>
__global__ __launch_bounds__(256) void wino_output_kernel(const float* __restrict__ Mt,
                                                          int64_t plane, int64_t OH, int64_t OW,
                                                          int64_t O, int64_t TH, int64_t TW,
                                                          E* __restrict__ y, float* __restrict__ acc,
                                                          int32_t epi, int64_t total) {
  const int64_t t = xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t r = t / O, o = t - r * O;
  const int64_t T = TH * TW;
  const int64_t n = r / T, rr = r - n * T;
  const int64_t ty = rr / TW, tx = rr - ty * TW;
  const float* __restrict__ src = Mt + r * O + o;
  // t1[i][b] = sum_a AT[i][a] m[a][b]  (6x8)
  float t1[6][8];
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    float col[8];
#pragma unroll
    for (int a = 0; a < 8; ++a) col[a] = src[(a * 8 + b) * plane];
    float res[6];
    cmatvec(kWinoAT, col, res);
#pragma unroll
    for (int i = 0; i < 6; ++i) t1[i][b] = res[i];
  }
#pragma unroll
  for (int i = 0; i < 6; ++i) {
    const int64_t oh = ty * 6 + i;
    float res[6];
    cmatvec(kWinoAT, t1[i], res);  // Y[i][j] = sum_b t1[i][b] AT[j][b]
    if (oh < OH) {
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int64_t ow = tx * 6 + j;
        if (ow < OW) {
          const int64_t idx = ((n * OH + oh) * OW + ow) * O + o;
          const float v = res[j];
          if (epi == kEpiStore) {
            // y is written once and not read here again: stream it past the caches
            __builtin_nontemporal_store(from_f32<E, BF16>(v), &y[idx]);
          } else if (epi == kEpiAccFirst) {
            acc[idx] = v;
          } else if (epi == kEpiAccMid) {
            acc[idx] = acc[idx] + v;
          } else {
            __builtin_nontemporal_store(from_f32<E, BF16>(acc[idx] + v), &y[idx]);
          }
        }
      }
    }
  }
}

inline unsigned blocks_for(int64_t total) { return unsigned((total + 255) / 256); }


}  // namespace

int wino_filter_launch(int dtype, const void* w, int64_t ldo, int64_t o, int64_t c, int64_t cs,
                       float* u, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(blocks_for(o * cs));
  if (dtype == CNHWC_F32)
    hipLaunchKernelGGL((wino_filter_kernel<float, false>), grid, dim3(256), 0, s,
                       static_cast<const float*>(w), ldo, o, c, cs, u);
  else if (dtype == CNHWC_F16)
    hipLaunchKernelGGL((wino_filter_kernel<uint16_t, false>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), ldo, o, c, cs, u);
  else
    hipLaunchKernelGGL((wino_filter_kernel<uint16_t, true>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), ldo, o, c, cs, u);
  return hipGetLastError();
}

int wino_input_launch(int dtype, const void* x, int64_t nb, int64_t h, int64_t w, int64_t c,
                      int64_t cs, int32_t ph, int32_t pw, int64_t th, int64_t tw, float* v,
                      int64_t plane, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t total = nb * th * tw * cs;
  if (total == 0) return hipSuccess;
  const dim3 grid(blocks_for(total));
  if (dtype == CNHWC_F32)
    hipLaunchKernelGGL((wino_input_kernel<float, false>), grid, dim3(256), 0, s,
                       static_cast<const float*>(x), h, w, c, cs, ph, pw, th, tw, v, plane, total);
  else if (dtype == CNHWC_F16)
    hipLaunchKernelGGL((wino_input_kernel<uint16_t, false>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), h, w, c, cs, ph, pw, th, tw, v, plane, total);
  else
    hipLaunchKernelGGL((wino_input_kernel<uint16_t, true>), grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), h, w, c, cs, ph, pw, th, tw, v, plane, total);
  return hipGetLastError();
}

int wino_output_launch(int dtype, const float* m, int64_t plane, int64_t nb, int64_t oh,
                       int64_t ow, int64_t o, int64_t th, int64_t tw, void* y, float* acc,
                       int32_t epi, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t total = nb * th * tw * o;
  if (total == 0) return hipSuccess;
  const dim3 grid(blocks_for(total));
  if (dtype == CNHWC_F32)
    hipLaunchKernelGGL((wino_output_kernel<float, false>), grid, dim3(256), 0, s, m, plane, oh, ow,
                       o, th, tw, static_cast<float*>(y), acc, epi, total);
  else if (dtype == CNHWC_F16)
    hipLaunchKernelGGL((wino_output_kernel<uint16_t, false>), grid, dim3(256), 0, s, m, plane, oh,
                       ow, o, th, tw, static_cast<uint16_t*>(y), acc, epi, total);
  else
    hipLaunchKernelGGL((wino_output_kernel<uint16_t, true>), grid, dim3(256), 0, s, m, plane, oh,
                       ow, o, th, tw, static_cast<uint16_t*>(y), acc, epi, total);
  return hipGetLastError();
}

}  // namespace cnhwc
