// Winograd F(4x4,3x3) for fp16/bf16 convs on gfx950: the transforms of the
// half-precision Winograd path.  The 36 tile-position GEMMs between them run
// on the fp16 matrix cores (gemm_lds.hip, 256-row tiles, fp32 results).
//
// MLX PR "Bound winograd conv2d working set by tiling the batch", Problem:
// the Winograd conv2d is an input transform into tile-position-major GEMM
// operands, batched GEMMs over the tile positions and an output transform.
// MLX PR "Decompose small kernel-depth 3D convs into 2D convs", Change: a 3D
// conv with a small kernel depth is a sum over its depth taps of per-frame 2D
// convs.  Here those taps are summed inside the GEMM (K = KD * Cs, the rows of
// tap kd shifted by kd * dd frames), so a 3D conv runs one output transform.
//
// Precision.  Half-precision storage of F(6x6,3x3) operands is too coarse for
// a 1e-2 relative bound; F(4x4,3x3) with fp16 V and U (11-bit significands)
// and fp32 M stays well inside it.  fp16's range is the risk: |B^T d B| can
// reach 100 max|d|.  So the transformed operands are scaled by powers of two
// picked on the device from max|x| and max|w| (kWino4VBound, kWino4UBound):
//   V = fp16(B^T (sx d) B),  U = fp16(G (sw g) G^T),  y = (A^T M A) / (sx sw)
// with sx * 100 max|x| < 2^15 and sw * max|g| < 2^15, so no transformed value
// can overflow, for any finite input (bf16 inputs included), and the largest
// ones use fp16's top binade.  Scaling by a power of two is exact: it changes
// no bit of a normal result.  The scales
// come from the whole x and w before the batch loop, so batch tiles see the
// same scales and tiled runs keep the untiled bits.
//
// Workspace (elements): partial maxima, then the scales {sx, sw} and 1/(sx sw)
// as two powers of two,
//   U [36][KD*Cs/32][O][32]   fp16, Cs = C rounded up to 32 (zero channels)
//   V [36][rows][Cs]          fp16, rows = (image or frame) * tiles, frames padded by pd
//   M [36][rows'][O]    fp32, rows' = output images or frames * tiles
//   tap masks [KD][O]   nonzero 3x3 taps of each (o, kd) filter slice (uint32)
//   tile masks [rows][P] nonzero pixels of each 6x6 input tile, in parts
// The masks make an output whose products are all zero exactly zero (see
// wino_mask.hpp); in 3D an output's window spans the KD frames its taps read.
// Tile (ty, tx) covers input rows 4 ty - ph .. +5 and columns 4 tx - pw .. +5
// and produces output rows 4 ty .. 4 ty + 3 (cropped).
// U is K-chunk-major: each position's plane holds its 32-element K chunks one
// after another, each as O rows of 32 elements (64 bytes), so the GEMM's load
// of one chunk for 16 consecutive filter rows reads 1 KB of whole 128-byte
// lines; row-major rows would give each load half of each of 16 lines and
// bring every line into the vector L1 twice.  V stays row-major: written
// K-chunk-major, the input transform's stores (one tile's 64-byte pieces in
// eight chunk planes per wavefront) cost more than its GEMM loads gain.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.hpp"
#include "device_common.hpp"
#include "wino_mask.hpp"
#include "winograd_f43.h"

namespace cnhwc {
namespace {

constexpr int kT = kWinoHM + 2;  // 6x6 input tiles

// Loads outside the image read this zero block instead, so every load of the
// input transform is issued unconditionally (no branch per pixel: the
// compiler can put all of a thread's loads in flight at once).
__device__ __align__(16) uint32_t g_wino_h_zero[4] = {0u, 0u, 0u, 0u};

// |h| as integer bits, NaN mapped to 0 (a NaN must not pick the scale; it
// propagates through the conv itself).  Order of |h| == order of these bits.
template <bool BF16>
__device__ __forceinline__ uint32_t abs_bits(uint32_t h) {
  const uint32_t a = h & 0x7fffu;
  constexpr uint32_t kInf = BF16 ? 0x7f80u : 0x7c00u;
  return a > kInf ? 0u : a;
}

template <bool BF16>
__device__ __forceinline__ float abs_bits_to_f32(uint32_t a) {
  if constexpr (BF16) return __builtin_bit_cast(float, a << 16);
  else return static_cast<float>(__builtin_bit_cast(_Float16, uint16_t(a)));
}

// Max over the 256 threads of a block; the result is valid in thread 0.
__device__ __forceinline__ uint32_t block_max(uint32_t v, uint32_t* sm) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, uint32_t(__shfl_xor(int(v), off)));
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) v = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
  return v;
}

// blockIdx.y = 0: x, 1: w.  Block b of a tensor's nb blocks strides over its
// 16-byte vectors and writes the largest |element| (as bits) to partial[y][b].
template <bool BF16>
__global__ __launch_bounds__(256) void wino_h_absmax_kernel(const uint16_t* __restrict__ x,
                                                            int64_t nx, int32_t nbx,
                                                            const uint16_t* __restrict__ w,
                                                            int64_t nw, int32_t nbw,
                                                            uint32_t* __restrict__ partial) {
  __shared__ uint32_t sm[4];
  const bool is_w = blockIdx.y == 1;
  const int32_t nb = is_w ? nbw : nbx;
  if (int32_t(blockIdx.x) >= nb) return;  // whole block: no barrier is skipped by part of it
  const uint16_t* __restrict__ src = is_w ? w : x;
  const int64_t n = is_w ? nw : nx;
  const int64_t nvec = n / 8;
  const uint4* __restrict__ vec = reinterpret_cast<const uint4*>(src);
  uint32_t m = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < nvec; i += int64_t(nb) * 256) {
    const uint4 q = vec[i];
    const uint32_t words[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      m = max(m, max(abs_bits<BF16>(words[k] & 0xffffu), abs_bits<BF16>(words[k] >> 16)));
  }
  if (blockIdx.x == 0)
    for (int64_t i = nvec * 8 + threadIdx.x; i < n; i += 256) m = max(m, abs_bits<BF16>(src[i]));
  m = block_max(m, sm);
  if (threadIdx.x == 0) partial[blockIdx.y * kWinoHSlots + blockIdx.x] = m;
}

// Exponent e of the scale 2^e for a tensor with largest |element| a whose
// transformed values are bounded by bound * a: with a < 2^k and bound <= 2^kb,
// e = 15 - kb - k gives 2^e * bound * a < 2^15, two below fp16's largest
// finite value 65504, which leaves room for the rounding of the fp32
// transform arithmetic.  Zero and non-finite maxima take 2^0.  |e| <= 126
// keeps 2^e and 2^-e normal fp32 numbers; every finite fp16 or bf16 tensor
// gets its full scale except bf16 maxima below about 2^-112 (then the top of
// its range sits lower, still without overflow).
__device__ __forceinline__ int scale_exp(float a, float bound) {
  if (!(a > 0.0f) || !(a < __builtin_huge_valf())) return 0;
  int k, kb;
  frexpf(a, &k);       // a in [2^(k-1), 2^k)
  frexpf(bound, &kb);  // bound < 2^kb
  const int e = 15 - kb - k;
  return e < -126 ? -126 : (e > 126 ? 126 : e);
}

// The scales from the partial maxima (every thread of the block takes part;
// the result is valid in every thread): {sx, sw} and 1/(sx sw) split in two.
template <bool BF16>
__device__ __forceinline__ void block_scales(const uint32_t* __restrict__ partial, int32_t nbx,
                                             int32_t nbw, uint32_t* sm, float (&s)[4]) {
  uint32_t mx = 0, mw = 0;
  for (int i = threadIdx.x; i < nbx; i += 256) mx = max(mx, partial[i]);
  for (int i = threadIdx.x; i < nbw; i += 256) mw = max(mw, partial[kWinoHSlots + i]);
  mx = block_max(mx, sm);
  __syncthreads();  // sm is reused
  mw = block_max(mw, sm);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int ex = scale_exp(abs_bits_to_f32<BF16>(mx), kWino4VBound);
    const int ew = scale_exp(abs_bits_to_f32<BF16>(mw), kWino4UBound);
    // 2^-(ex+ew) is undone in two halves (it may not be an fp32 itself); each
    // intermediate lies between the GEMM's fp32 result and the final value,
    // so it overflows only if y does
    const int et = -(ex + ew), eh = et / 2;
    sm[0] = __builtin_bit_cast(uint32_t, ldexpf(1.0f, ex));
    sm[1] = __builtin_bit_cast(uint32_t, ldexpf(1.0f, ew));
    sm[2] = __builtin_bit_cast(uint32_t, ldexpf(1.0f, eh));
    sm[3] = __builtin_bit_cast(uint32_t, ldexpf(1.0f, et - eh));
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = __builtin_bit_cast(float, sm[i]);
}

// U[p][o][kd*Cs + c] = fp16((G (sw g) G^T)_p), g = w[o][kd][.][.][c]; zero for c >= C.
// Every block first reduces the partial maxima to the scales (block 0 also
// stores them for the input and output transforms, which run after it).
// Workgroups [0, nfb) transform the filter; the workgroups after them compute
// the tap masks, one wavefront per (o, kd) slice.
template <bool BF16>
__global__ __launch_bounds__(256) void wino_h_filter_kernel(const uint16_t* __restrict__ w,
                                                            int64_t O, int64_t KD, int64_t C,
                                                            int64_t Cs,
                                                            const uint32_t* __restrict__ partial,
                                                            int32_t nbx, int32_t nbw,
                                                            float* __restrict__ scales,
                                                            uint16_t* __restrict__ U, int64_t nfb,
                                                            uint32_t* __restrict__ wm) {
  if (int64_t(blockIdx.x) >= nfb) {  // whole workgroups: uniform branch, no barrier below
    const int64_t sl = (int64_t(blockIdx.x) - nfb) * 4 + (threadIdx.x >> 6);  // o * KD + kd
    if (sl >= O * KD) return;
    const uint32_t bits = tap_mask_of(w + sl * 9 * C, C, [](uint16_t v) { return (v & 0x7fffu) != 0u; });
    const int64_t o = sl / KD, kd = sl - o * KD;
    if ((threadIdx.x & 63) == 0) wm[kd * O + o] = bits;
    return;
  }
  __shared__ uint32_t sm[4];
  float sc[4];
  block_scales<BF16>(partial, nbx, nbw, sm, sc);
  if (blockIdx.x == 0 && threadIdx.x < 4) scales[threadIdx.x] = sc[threadIdx.x];
  const int64_t ku = KD * Cs;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t >= O * ku) return;
  const int64_t o = t / ku, r = t - o * ku;
  const int64_t kd = r / Cs, c = r - kd * Cs;
  const uint16_t* __restrict__ g0 = w + (o * KD + kd) * 9 * C + c;
  // scaled as it is loaded (exact): the fp32 transform then stays below 2^15
  const float s = sc[1];
  float g[3][3];
#pragma unroll
  for (int a = 0; a < 3; ++a)
#pragma unroll
    for (int b = 0; b < 3; ++b) g[a][b] = c < C ? s * to_f32<uint16_t, BF16>(g0[(a * 3 + b) * C]) : 0.0f;
  float t1[kT][3];  // G g
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const float col[3] = {g[0][b], g[1][b], g[2][b]};
    float res[kT];
    cmatvec(kWino4G, col, res);
#pragma unroll
    for (int i = 0; i < kT; ++i) t1[i][b] = res[i];
  }
  const int64_t plane = O * ku;
  uint16_t* __restrict__ out = U + (r >> 5) * (O * 32) + o * 32 + (r & 31);  // K-chunk-major
#pragma unroll
  for (int i = 0; i < kT; ++i) {
    const float row[3] = {t1[i][0], t1[i][1], t1[i][2]};
    float res[kT];
    cmatvec(kWino4G, row, res);  // (t1 G^T)[i][j]
#pragma unroll
    for (int j = 0; j < kT; ++j) out[(i * kT + j) * plane] = f32_to_f16_bits(res[j]);
  }
}

// V[p][r][c] = fp16((B^T (sx d) B)_p) for tile row r = (image, ty, tx).  Images
// are the frames fp of nb elements with Dp frames each; frame fp reads input
// frame fp - pd (zero outside [0, D)); 2D convs have D = Dp = 1, pd = 0.
// VEC channels per thread (4 when C % 4 == 0, 2 when C is even: 8- or 4-byte
// loads and stores).  Besides V it writes the tile's nonzero-pixel mask (bit
// i * 6 + j for pixel (i, j)): with WAVE (Cs / VEC % 64 == 0) every wavefront
// holds channels of one tile and builds its part from one ballot per pixel;
// otherwise the workgroup ORs its threads' masks.
template <bool BF16, int VEC, bool WAVE>
__global__ __launch_bounds__(256, 3) void wino_h_input_kernel(
    const uint16_t* __restrict__ x, int64_t D, int64_t Dp, int32_t pd, int64_t H, int64_t W,
    int64_t C, int64_t Cs, int32_t ph, int32_t pw, int64_t TH, int64_t TW,
    const float* __restrict__ scales, uint16_t* __restrict__ V, int64_t plane, int64_t total,
    uint64_t* __restrict__ tm, int64_t parts) {
  const int64_t blk = xcd_block(blockIdx.x, gridDim.x);
  const int64_t t = blk * 256 + threadIdx.x;
  const int64_t groups = Cs / VEC;
  uint64_t pix = 0;  // nonzero pixels (WAVE: of the wavefront's channels, uniform; else this thread's)
  if (t < total) {
  const int64_t r = t / groups, c = (t - r * groups) * VEC;
  const int64_t T = TH * TW;
  const int64_t im = r / T, rr = r - im * T;
  const int64_t n = im / Dp, f = im - n * Dp - pd;
  const bool fok = f >= 0 && f < D;
  const int64_t ty = rr / TW, tx = rr - ty * TW;
  const int64_t ih0 = ty * kWinoHM - ph, iw0 = tx * kWinoHM - pw;
  const uint16_t* __restrict__ img = x + (n * D + (fok ? f : 0)) * H * W * C + c;
  const bool cin = fok && c < C;  // VEC > 1 only for C % VEC == 0: c < C implies c + VEC - 1 < C
  // Inputs are scaled as they are loaded (exact), so the fp32 transform stays
  // below 2^15 even where 100 max|x| would overflow fp32 (bf16 inputs).
  const float s = scales[0];
  // every load first (unconditional: outside the image they read a zero
  // block), so that all of them are in flight before the first is used
  using Raw = typename std::conditional<VEC == 4, uint2, typename std::conditional<VEC == 2, uint32_t,
                                                                                   uint16_t>::type>::type;
  Raw raw[kT][kT];
#pragma unroll
  for (int j = 0; j < kT; ++j) {
    const int64_t iw = iw0 + j;
    const bool wok = cin && iw >= 0 && iw < W;
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      const int64_t ih = ih0 + i;
      const bool ok = wok && ih >= 0 && ih < H;
      raw[i][j] = *reinterpret_cast<const Raw*>(ok ? img + (ih * W + iw) * C
                                                   : reinterpret_cast<const uint16_t*>(g_wino_h_zero));
    }
  }
  // column transform first: t1[v][a][j] = sum_i BT[a][i] d[i][j]
  float t1[VEC][kT][kT];
#pragma unroll
  for (int j = 0; j < kT; ++j) {
    float col[VEC][kT];
#pragma unroll
    for (int i = 0; i < kT; ++i) {
      uint32_t nz;  // nonzero bits of this pixel's VEC channels (sign bits dropped)
      if constexpr (VEC == 4) {
        const uint2 q = raw[i][j];
        col[0][i] = s * to_f32<uint16_t, BF16>(uint16_t(q.x & 0xffffu));
        col[1][i] = s * to_f32<uint16_t, BF16>(uint16_t(q.x >> 16));
        col[2][i] = s * to_f32<uint16_t, BF16>(uint16_t(q.y & 0xffffu));
        col[3][i] = s * to_f32<uint16_t, BF16>(uint16_t(q.y >> 16));
        nz = (q.x | q.y) & 0x7fff7fffu;
      } else if constexpr (VEC == 2) {
        const uint32_t q = raw[i][j];
        col[0][i] = s * to_f32<uint16_t, BF16>(uint16_t(q & 0xffffu));
        col[1][i] = s * to_f32<uint16_t, BF16>(uint16_t(q >> 16));
        nz = q & 0x7fff7fffu;
      } else {
        const uint16_t h = raw[i][j];
        col[0][i] = s * to_f32<uint16_t, BF16>(h);
        nz = h & 0x7fffu;
      }
      // WAVE: one ballot per pixel (the mask stays in scalar registers)
      if constexpr (WAVE) pix |= uint64_t(__ballot(nz != 0u) != 0ull) << (i * kT + j);
      else pix |= uint64_t(nz != 0u) << (i * kT + j);
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float res[kT];
      cmatvec(kWino4BT, col[v], res);
#pragma unroll
      for (int a = 0; a < kT; ++a) t1[v][a][j] = res[a];
    }
  }
  // row transform: v[a][b] = sum_j t1[a][j] BT[b][j], rounded to fp16
  uint16_t* __restrict__ out = V + r * Cs + c;
#pragma unroll
  for (int a = 0; a < kT; ++a) {
    float res[VEC][kT];
#pragma unroll
    for (int v = 0; v < VEC; ++v) cmatvec(kWino4BT, t1[v][a], res[v]);
#pragma unroll
    for (int b = 0; b < kT; ++b) {
      if constexpr (VEC == 4) {
        const uint2 q = make_uint2(uint32_t(f32_to_f16_bits(res[0][b])) |
                                       (uint32_t(f32_to_f16_bits(res[1][b])) << 16),
                                   uint32_t(f32_to_f16_bits(res[2][b])) |
                                       (uint32_t(f32_to_f16_bits(res[3][b])) << 16));
        *reinterpret_cast<uint2*>(out + (a * kT + b) * plane) = q;
      } else if constexpr (VEC == 2) {
        const uint32_t q = uint32_t(f32_to_f16_bits(res[0][b])) |
                           (uint32_t(f32_to_f16_bits(res[1][b])) << 16);
        *reinterpret_cast<uint32_t*>(out + (a * kT + b) * plane) = q;
      } else {
        out[(a * kT + b) * plane] = f32_to_f16_bits(res[0][b]);
      }
    }
  }
  if constexpr (WAVE) {
    if ((threadIdx.x & 63) == 0) tm[r * parts + (c / VEC) / 64] = pix;
  }
  }
  if constexpr (!WAVE) store_block_masks(pix, t < total, t, blk, groups, total / groups, tm, parts);
}

// y[im][oh][ow][o] = (A^T M A)[oh - 4 ty][ow - 4 tx] / (sx sw), cropped to
// [OH, OW], for output image or frame im.  VEC output channels per thread
// (2 when O is even).
// Outputs whose window (over the KD frames its taps read) meets no nonzero
// pixel under a nonzero tap store an exact zero.  Output frame od of element n
// reads input rows of padded frame od + kd * dd (Dp frames per element); the
// input transform wrote their masks with g threads per tile row in `parts`
// parts.  2D: OD = Dp = KD = 1.
template <bool BF16, int VEC>
__global__ __launch_bounds__(256) void wino_h_output_kernel(const float* __restrict__ Mt,
                                                            int64_t plane, int64_t OH,
                                                            int64_t OW, int64_t O, int64_t TH,
                                                            int64_t TW,
                                                            const float* __restrict__ scales,
                                                            uint16_t* __restrict__ y,
                                                            int64_t total,
                                                            const uint64_t* __restrict__ tm,
                                                            int64_t g, int64_t parts,
                                                            const uint32_t* __restrict__ wm,
                                                            int64_t OD, int64_t Dp, int64_t KD,
                                                            int64_t dd) {
  const int64_t t = xcd_block(blockIdx.x, gridDim.x) * 256 + threadIdx.x;
  if (t >= total) return;
  const int64_t groups = O / VEC;
  const int64_t r = t / groups, o = (t - r * groups) * VEC;
  const int64_t T = TH * TW;
  const int64_t im = r / T, rr = r - im * T;
  const int64_t ty = rr / TW, tx = rr - ty * TW;
  uint64_t hits[VEC];
  {
    const int64_t n = im / OD, od = im - n * OD;
    const bool wave = g % 64 == 0;
    // a tile whose pixels are all nonzero in every frame the taps read (the
    // usual case away from padding and zero regions): every output sees a
    // nonzero pixel under each nonzero tap, and an all-zero filter yields an
    // exact zero through U = 0 anyway, so the tap masks are not needed
    uint64_t all = ~0ull;
    for (int64_t kd = 0; kd < KD; ++kd)
      all &= load_tile_mask(tm, (n * Dp + od + kd * dd) * T + rr, g, wave, parts);
    constexpr uint64_t kFull = (1ull << (kT * kT)) - 1;
#pragma unroll
    for (int v = 0; v < VEC; ++v) hits[v] = (all & kFull) == kFull ? ~0ull : 0ull;
    if ((all & kFull) != kFull) {
      for (int64_t kd = 0; kd < KD; ++kd) {
        const uint64_t m = load_tile_mask(tm, (n * Dp + od + kd * dd) * T + rr, g, wave, parts);
#pragma unroll
        for (int v = 0; v < VEC; ++v) hits[v] |= window_hits<kT>(m, wm[kd * O + o + v]);
      }
    }
  }
  // M is read once: non-temporal loads keep it from displacing what L2 holds
  // for the other kernels' data (12% faster at C = O = 256 and 1024 -> 1024,
  // 3-4% at the largest video conv)
  const float* __restrict__ src = Mt + r * O + o;
  // t1[v][i][b] = sum_a AT[i][a] m[a][b]  (4x6)
  float t1[VEC][kWinoHM][kT];
#pragma unroll
  for (int b = 0; b < kT; ++b) {
    float col[VEC][kT];
#pragma unroll
    for (int a = 0; a < kT; ++a) {
      if constexpr (VEC == 2) {
        const v2f q = __builtin_nontemporal_load(reinterpret_cast<const v2f*>(src + (a * kT + b) * plane));
        col[0][a] = q.x;
        col[1][a] = q.y;
      } else {
        col[0][a] = __builtin_nontemporal_load(src + (a * kT + b) * plane);
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      float res[kWinoHM];
      cmatvec(kWino4AT, col[v], res);
#pragma unroll
      for (int i = 0; i < kWinoHM; ++i) t1[v][i][b] = res[i];
    }
  }
  const float inv_a = scales[2], inv_b = scales[3];
  // WHOLE: the tile lies inside the output, so its stores need no bounds tests
  auto finish = [&](auto whole_c) {
    constexpr bool WHOLE = decltype(whole_c)::value;
#pragma unroll
    for (int i = 0; i < kWinoHM; ++i) {
      const int64_t oh = ty * kWinoHM + i;
      float res[VEC][kWinoHM];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        cmatvec(kWino4AT, t1[v][i], res[v]);  // Y[i][j]
#pragma unroll
        for (int j = 0; j < kWinoHM; ++j)
          res[v][j] = (hits[v] >> (i * kT + j)) & 1u ? (res[v][j] * inv_a) * inv_b : 0.0f;  // exact
      }
      if (WHOLE || oh < OH) {
#pragma unroll
        for (int j = 0; j < kWinoHM; ++j) {
          const int64_t ow = tx * kWinoHM + j;
          if (WHOLE || ow < OW) {
            uint16_t* dst = y + ((im * OH + oh) * OW + ow) * O + o;
            // y is written once and not read here again: stream it past the caches
            if constexpr (VEC == 2) {
              const uint32_t q = uint32_t(from_f32<uint16_t, BF16>(res[0][j])) |
                                 (uint32_t(from_f32<uint16_t, BF16>(res[1][j])) << 16);
              __builtin_nontemporal_store(q, reinterpret_cast<uint32_t*>(dst));
            } else {
              __builtin_nontemporal_store(from_f32<uint16_t, BF16>(res[0][j]), dst);
            }
          }
        }
      }
    }
  };
  if (ty * kWinoHM + kWinoHM <= OH && tx * kWinoHM + kWinoHM <= OW) finish(std::true_type{});
  else finish(std::false_type{});
}

inline unsigned blocks_for(int64_t total) { return unsigned((total + 255) / 256); }

}  // namespace

int wino_h_absmax_launch(int dtype, const void* x, int64_t nx, const void* w, int64_t nw,
                         uint32_t* partial, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int32_t nbx = wino_h_absmax_blocks(nx), nbw = wino_h_absmax_blocks(nw);
  const dim3 grid{unsigned(nbx > nbw ? nbx : nbw), 2u, 1u};
  const uint16_t* xs = static_cast<const uint16_t*>(x);
  const uint16_t* ws = static_cast<const uint16_t*>(w);
  if (dtype == CNHWC_BF16)
    hipLaunchKernelGGL((wino_h_absmax_kernel<true>), grid, dim3(256), 0, s, xs, nx, nbx, ws, nw, nbw,
                       partial);
  else
    hipLaunchKernelGGL((wino_h_absmax_kernel<false>), grid, dim3(256), 0, s, xs, nx, nbx, ws, nw, nbw,
                       partial);
  return hipGetLastError();
}

int wino_h_filter_launch(int dtype, const void* w, int64_t o, int64_t kd, int64_t c, int64_t cs,
                         const uint32_t* partial, int64_t nx, int64_t nw, float* scales, uint16_t* u,
                         uint32_t* wm, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t total = o * kd * cs;
  const int64_t nfb = int64_t(blocks_for(total));
  const dim3 grid(unsigned(nfb + (o * kd + 3) / 4));
  const int32_t nbx = wino_h_absmax_blocks(nx), nbw = wino_h_absmax_blocks(nw);
  const uint16_t* ws = static_cast<const uint16_t*>(w);
  if (dtype == CNHWC_BF16)
    hipLaunchKernelGGL((wino_h_filter_kernel<true>), grid, dim3(256), 0, s, ws, o, kd, c, cs, partial, nbx,
                       nbw, scales, u, nfb, wm);
  else
    hipLaunchKernelGGL((wino_h_filter_kernel<false>), grid, dim3(256), 0, s, ws, o, kd, c, cs, partial, nbx,
                       nbw, scales, u, nfb, wm);
  return hipGetLastError();
}

int wino_h_input_launch(int dtype, const void* x, int64_t nb, int64_t d, int64_t dp, int32_t pd,
                        int64_t h, int64_t w, int64_t c, int64_t cs, int32_t ph, int32_t pw,
                        int64_t th, int64_t tw, const float* scales, uint16_t* v, int64_t plane,
                        uint64_t* tm, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int vec = int(wino_h_vec(c));
  const int64_t g = cs / vec;
  const int64_t total = nb * dp * th * tw * g;
  if (total == 0) return hipSuccess;
  const dim3 grid(blocks_for(total));
  const int64_t parts = wino_mask_parts(g);
  const bool wave = g % 64 == 0;
  const uint16_t* xs = static_cast<const uint16_t*>(x);
#define CNHWC_WINO_H_INPUT(B, VEC, WAVE)                                                        \
  hipLaunchKernelGGL((wino_h_input_kernel<B, VEC, WAVE>), grid, dim3(256), 0, s, xs, d, dp, pd, \
                     h, w, c, cs, ph, pw, th, tw, scales, v, plane, total, tm, parts)
#define CNHWC_WINO_H_INPUT_W(B, VEC)         \
  do {                                       \
    if (wave) CNHWC_WINO_H_INPUT(B, VEC, true); \
    else CNHWC_WINO_H_INPUT(B, VEC, false);   \
  } while (0)
  if (dtype == CNHWC_BF16) {
    if (vec == 4) CNHWC_WINO_H_INPUT_W(true, 4);
    else if (vec == 2) CNHWC_WINO_H_INPUT_W(true, 2);
    else CNHWC_WINO_H_INPUT_W(true, 1);
  } else {
    if (vec == 4) CNHWC_WINO_H_INPUT_W(false, 4);
    else if (vec == 2) CNHWC_WINO_H_INPUT_W(false, 2);
    else CNHWC_WINO_H_INPUT_W(false, 1);
  }
#undef CNHWC_WINO_H_INPUT_W
#undef CNHWC_WINO_H_INPUT
  return hipGetLastError();
}

int wino_h_output_launch(int dtype, const float* m, int64_t plane, int64_t nimg, int64_t oh,
                         int64_t ow, int64_t o, int64_t th, int64_t tw, const float* scales,
                         void* y, const uint64_t* tm, int64_t c, int64_t cs, const uint32_t* wm,
                         int64_t od, int64_t dp, int64_t kd, int64_t dd, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int vec = o % 2 == 0 ? 2 : 1;  // 4 per thread measured 3-15% slower (fewer waves in flight)
  const int64_t total = nimg * th * tw * (o / vec);
  if (total == 0) return hipSuccess;
  const dim3 grid(blocks_for(total));
  const int64_t g = cs / wino_h_vec(c);  // threads per tile row of the input transform
  const int64_t parts = wino_mask_parts(g);
  uint16_t* ys = static_cast<uint16_t*>(y);
#define CNHWC_WINO_H_OUTPUT(B, VEC)                                                              \
  hipLaunchKernelGGL((wino_h_output_kernel<B, VEC>), grid, dim3(256), 0, s, m, plane, oh, ow, o, \
                     th, tw, scales, ys, total, tm, g, parts, wm, od, dp, kd, dd)
  if (dtype == CNHWC_BF16) {
    if (vec == 2) CNHWC_WINO_H_OUTPUT(true, 2);
    else CNHWC_WINO_H_OUTPUT(true, 1);
  } else {
    if (vec == 2) CNHWC_WINO_H_OUTPUT(false, 2);
    else CNHWC_WINO_H_OUTPUT(false, 1);
  }
#undef CNHWC_WINO_H_OUTPUT
  return hipGetLastError();
}

}  // namespace cnhwc
