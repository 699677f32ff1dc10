// Device side of the zero-window masks of both Winograd forms.
//
// An output whose every product x * w is zero (its window holds zeros, or
// padding, wherever its filter does not) is exactly zero.  The transforms,
// though, round every value of a tile at the scale of the largest ones in
// it, so such an output would otherwise carry rounding residue from nonzero
// pixels elsewhere in its tile.  The input transform records which pixels of
// each tile are nonzero in any channel (bit i * S + j for tile pixel (i, j),
// S the tile side), the filter transform which taps of each output channel's
// filter are nonzero in any channel (bit kh * 3 + kw), and the output
// transform stores exactly zero for every output whose window meets no
// nonzero pixel under a nonzero tap.  (An output whose products vanish only
// because the nonzero channels of its pixels and of its taps never coincide
// is not caught; it keeps the tile-relative rounding error.)
//
// Tile masks are written in parts, with neither atomics nor a clearing pass:
// every thread builds the mask of its own channels (one bit per pixel, no
// cross-lane step inside the load loop, so the loads stay free to overlap),
// and the G threads of a tile row (launch threads r * G .. r * G + G - 1)
// either fill whole wavefronts (G % 64 == 0: each wavefront ORs its lanes
// and writes part (t % G) / 64) or share workgroups of 256 (each workgroup
// holding some of the row's threads ORs them in LDS and writes part
// b - (r * G) / 256, b the workgroup).  The output
// transform ORs exactly the parts that were written.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace cnhwc {

// Number of parts of tile row r's mask (P = the parts slot count per row in
// wavefront mode).
__device__ __forceinline__ int64_t mask_parts_of(int64_t r, int64_t g, bool wave, int64_t p) {
  return wave ? p : ((r + 1) * g - 1) / 256 - (r * g) / 256 + 1;
}

// Nonzero-pixel mask of tile row r.
__device__ __forceinline__ uint64_t load_tile_mask(const uint64_t* __restrict__ tm, int64_t r,
                                                   int64_t g, bool wave, int64_t p) {
  const int64_t n = mask_parts_of(r, g, wave, p);
  const uint64_t* __restrict__ src = tm + r * p;
  uint64_t m = 0;
  for (int64_t q = 0; q < n; ++q) m |= src[q];
  return m;
}

// OR of a per-thread mask over the 64 lanes of the wavefront (every lane
// gets the result).
__device__ __forceinline__ uint64_t wave_or(uint64_t m) {
  uint32_t lo = uint32_t(m), hi = uint32_t(m >> 32);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    lo |= uint32_t(__shfl_xor(int(lo), off));
    hi |= uint32_t(__shfl_xor(int(hi), off));
  }
  return (uint64_t(hi) << 32) | lo;
}

// Workgroup mode: OR the per-thread masks of each tile row among the 256
// threads of logical workgroup b and store one part per row.  Every thread of
// the workgroup calls this (it holds barriers); `live` threads carry a mask.
// G >= 8 keeps the rows of one workgroup within kMaskSlots.
constexpr int kMaskSlots = 34;
__device__ __forceinline__ void store_block_masks(uint64_t m, bool live, int64_t t, int64_t b,
                                                  int64_t g, int64_t rows,
                                                  uint64_t* __restrict__ tm, int64_t p) {
  __shared__ unsigned long long slots[kMaskSlots];
  const int64_t r0 = (b * 256) / g;
  if (threadIdx.x < kMaskSlots) slots[threadIdx.x] = 0ull;
  __syncthreads();
  if (live && m) atomicOr(&slots[t / g - r0], static_cast<unsigned long long>(m));
  __syncthreads();
  const int64_t r = r0 + threadIdx.x;
  const int64_t r_last = (b * 256 + 255) / g;
  if (threadIdx.x < kMaskSlots && r <= r_last && r < rows)
    tm[r * p + (b - (r * g) / 256)] = slots[threadIdx.x];
}

// Bit i * S + j of the result is set iff tile output (i, j) has a nonzero
// pixel (i + kh, j + kw) under a nonzero tap (kh, kw) of a 3x3 filter.
template <int S>
__device__ __forceinline__ uint64_t window_hits(uint64_t pix, uint32_t taps) {
  uint64_t z = 0;
#pragma unroll
  for (int kh = 0; kh < 3; ++kh)
#pragma unroll
    for (int kw = 0; kw < 3; ++kw)
      if ((taps >> (kh * 3 + kw)) & 1u) z |= pix >> (kh * S + kw);
  return z;
}

// Tap mask of one filter slice (one output channel, or one (o, kd) pair in
// 3D), computed by a whole wavefront: bit kh * 3 + kw is set iff some channel
// c of g0[(kh * 3 + kw) * C + c] is nonzero (nz tests one raw element).  The
// result is uniform across the wavefront.
template <typename E, typename NZ>
__device__ __forceinline__ uint32_t tap_mask_of(const E* __restrict__ g0, int64_t C, NZ nz) {
  const int64_t lane = threadIdx.x & 63;
  uint32_t bits = 0;
#pragma unroll
  for (int tap = 0; tap < 9; ++tap) {
    bool any = false;
    for (int64_t c = lane; c < C; c += 64) any = any || nz(g0[tap * C + c]);
    if (__ballot(any) != 0ull) bits |= 1u << tap;
  }
  return bits;
}

}  // namespace cnhwc
