// Implicit-GEMM conv for 3x3, stride-1, dilation-1 filters in fp16/bf16 on
// gfx950, with the im2col fragments built from input patches staged in LDS.
//
// The conv is the GEMM C[M x N] = A[M x K] * B[N x K]^T of the implicit
// gather (MLX PR "Bound winograd conv2d working set by tiling the batch",
// Fix: the scratch-free implicit GEMM; MLX PR "Use the explicit gemm for wide
// convs on neural accelerators", intro: the wide half-precision convs; MLX PR
// "Decompose small kernel-depth 3D convs into 2D convs", Change: the per-frame
// convs and, here, the native 3D conv with its depth taps in K).  Each row of
// A is one output pixel's 3x3 window; neighbouring pixels share 6 of its 9
// taps.  The gather of the 256-row tile kernel (gemm_lds.hip) fetches every
// input pixel once per tap; here:
//  - a workgroup's 256 output rows are a BH x BW block of one output image
//    (or frame) and its 256 columns 256 output channels; 4 wavefronts, each a
//    128 x 128 quadrant (16 accumulating 32x32 blocks);
//  - per 64-channel chunk the block's (BH + 2) x (BW + 2) input patch goes
//    from global memory straight into LDS once (global_load_lds_dwordx4, 128
//    bytes per pixel, zero outside the image), and all nine taps read their
//    A fragments from it, shifted by the tap; only the weight rows of each tap
//    (32 KB) stream per tap;
//  - the weight rows of tap t + 2 and a slice of the next chunk's patch are
//    loaded while tap t runs (two weight stages, two patch buffers), with one
//    barrier per tap.
// That is 36 KB of global-to-LDS traffic per tap of 8.4 MFLOP, against 64 KB
// for the per-tap gather.
//
// K order.  Every output adds its products in the order (depth tap, 64-channel
// chunk, kh, kw, 16-channel MFMA step), 16 at a time: a fixed order per tile
// configuration, so the bits depend on the data and the plan only.  (The
// per-tap gather of the other configurations orders K as (depth tap, kh, kw,
// channel); the two differ in rounding only.)
//
// LDS layouts: patch pixel p at 128 p, its 16-byte piece c (8 channels) at
// physical piece c ^ ((p >> 1) & 7); weight row r of a stage at 128 r, piece
// c at c ^ ((r >> 1) & 7).  Sixteen consecutive rows (or pixels) of one
// logical piece then hit sixteen distinct bank groups.  A lane's LDS
// destination is fixed by its lane index, so the swizzle is applied on the
// global side.
//
// MFMA: v_mfma_f32_32x32x16_{f16,bf16} with the weight fragment as the first
// operand, so each accumulator block is the transposed (channels x pixels)
// 32x32 block; in 16-channel step s of a chunk, lanes 0..31 supply channels
// 16 s + 0..7 and lanes 32..63 16 s + 8..15 of their row.
//
// Workgroups are persistent (at most one per CU, each walking a list of
// tiles, see the kernel), and each tile's results leave through LDS in
// whole-line stores.
#include <hip/hip_runtime.h>

#include <atomic>
#include <type_traits>

#include "internal.hpp"
#include "device_common.hpp"

namespace cnhwc {
namespace {

constexpr int kThreads = 256;
constexpr int kBN = 256;                                 // output channels per tile
constexpr int kRowB = 128;                               // bytes of one row (pixel) per 64-channel chunk
constexpr int kPatchLoads = 11;                          // 1 KB loads per wavefront per patch
constexpr int kPatchBytes = 4 * kPatchLoads * 1024;      // 44 KB: up to 352 pixels
constexpr int kBStage = kBN * kRowB;                     // 32 KB of weight rows per tap
constexpr int kBLoads = kBStage / (4 * 1024);            // 8 per wavefront
constexpr int kTaps = 9;
// Patch loads issued while tap t runs (prefix sums in kSliceStart): all 11 by tap 5.
constexpr int kSlice[kTaps] = {2, 2, 2, 2, 2, 1, 0, 0, 0};
constexpr int kSliceStart[kTaps] = {0, 2, 4, 6, 8, 10, 11, 11, 11};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gvec_ptr;
__device__ u32x4 g_patch_zero16 = {0u, 0u, 0u, 0u};
template <typename T>
__device__ __forceinline__ gvec_ptr gvec(const T* p) {
  return (gvec_ptr)(p);
}

// The patch buffers and the weight stages are two LDS objects, so the compiler
// tags each fragment read with the object it reads; the loads into LDS address
// them through an opaque integer (no tag), and the explicit vmcnt waits and
// barriers below order the two.
__shared__ __attribute__((aligned(1024))) uint8_t g_patch[2 * kPatchBytes];
__shared__ __attribute__((aligned(1024))) uint8_t g_wring[2 * kBStage];

typedef void __attribute__((address_space(3)))* lds_ptr;
__device__ __forceinline__ uint32_t lds_base(const uint8_t* p) {
  typedef const uint8_t __attribute__((address_space(3)))* lds_cptr;
  uint32_t v = uint32_t(reinterpret_cast<uintptr_t>((lds_cptr)p));
  asm volatile("" : "+s"(v));  // opaque to constant folding; emits no instruction
  return v;
}
__device__ __forceinline__ lds_ptr lds_addr(uint32_t a) { return reinterpret_cast<lds_ptr>(uintptr_t(a)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// The same, and every LDS read of this wavefront complete (lgkmcnt(0)).
template <int N>
__device__ __forceinline__ void wait_vmcnt_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}
__device__ __forceinline__ void block_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Row tiles are grouped kGroupM at a time, so that the workgroups of one XCD
// running together share input rows.
constexpr int64_t kGroupM = 8;
constexpr int kMaxDevices = 64;

// Physical 16-byte piece of logical piece c in LDS row (pixel) r is
// c ^ swz(r).  A 128-byte row covers half of the 64 four-byte banks, so rows
// r and r + 1 cover the two halves; with swz(r) = (r >> 1) & 7 any 16
// consecutive rows of one logical piece (the lanes a 16-byte read serves
// together) land on 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

struct Frag {
  uint4 a[4];
  uint4 b[4];
};

template <int V>
using ic = std::integral_constant<int, V>;

// Where a row tile sits: frame f (image, or n * OD + od in 3D), its first
// output row and column, and the first output channel of its column tile.
struct TileGeo {
  int32_t f, img, od, oh0, ow0, n0;
};

// BW: block width (output columns); the block is (256 / BW) x BW pixels.
//
// Persistent: the grid holds at most one workgroup per CU, and each workgroup
// walks a fixed list of tiles.  Tile t of n is assigned as follows: the 8 XCDs
// take contiguous ranges of tile indices; the kx workgroups of XCD x (those
// with blockIdx.x % 8 == x) take every kx-th tile of its range, so the tiles
// an XCD runs at one time are consecutive and share input rows and weights in
// its L2.  The load sequence runs on across tiles: during a tile's last
// (depth tap, chunk) iteration, the patch slices and the first two weight
// stages that are loaded are the next tile's, so a tile starts with its
// operands in LDS.  The loads of a workgroup's last iteration, which have no
// next tile, read a zero vector into buffers that are never read.
template <bool BF16, bool D3, int BW>
__global__ __launch_bounds__(kThreads, 1) void gemm_patch_kernel(const GemmParams p) {
  constexpr int BH = 256 / BW;
  constexpr int PW = BW + 2, PH = BH + 2, PPIX = PH * PW;
  static_assert(PPIX * kRowB <= kPatchBytes, "the patch fits its buffer");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t N = p.N, C = p.c, H = p.h, W = p.w, OH = p.oh, OW = p.ow;
  const int64_t KD = D3 ? p.kd : 1, D = D3 ? p.d : 1;
  const int32_t OD = D3 ? int32_t(p.od) : 1;

  // ---- this workgroup's tiles (32-bit indices: the tile count is below 2^31)
  const int32_t tby = int32_t((OH + BH - 1) / BH), tbx = int32_t((OW + BW - 1) / BW);
  const int32_t frames = int32_t(p.M / (OH * OW));
  const int32_t mt = frames * tby * tbx, nt = int32_t((N + kBN - 1) / kBN);
  const int32_t ntiles = mt * nt;
  const int32_t G = int32_t(gridDim.x), xcd = int32_t(blockIdx.x) % 8, kw8 = int32_t(blockIdx.x) / 8;
  const int32_t kx = G / 8 + (xcd < G % 8 ? 1 : 0);
  const int32_t q8 = ntiles / 8, r8 = ntiles % 8;
  const int32_t xs = xcd < r8 ? xcd * (q8 + 1) : r8 * (q8 + 1) + (xcd - r8) * q8;
  const int32_t xl = q8 + (xcd < r8 ? 1 : 0);
  if (kw8 >= xl) return;
  const int32_t my_tiles = (xl - kw8 + kx - 1) / kx;
  auto tile_geo = [&](int32_t j) {
    const int32_t t = xs + kw8 + j * kx;
    const int32_t group = t / (int32_t(kGroupM) * nt);
    const int32_t first_m = group * int32_t(kGroupM);
    const int32_t gsz = mt - first_m < int32_t(kGroupM) ? mt - first_m : int32_t(kGroupM);
    const int32_t tg = t - group * (int32_t(kGroupM) * nt);
    const int32_t mtile = first_m + tg % gsz;
    TileGeo g;
    g.n0 = (tg / gsz) * kBN;
    g.f = mtile / (tby * tbx);
    const int32_t rb = mtile - g.f * (tby * tbx);
    const int32_t by = rb / tbx;
    g.oh0 = by * BH;
    g.ow0 = (rb - by * tbx) * BW;
    g.img = g.f / OD;
    g.od = g.f - g.img * OD;
    return g;
  };
  const uint16_t* __restrict__ X = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* __restrict__ Bw = reinterpret_cast<const uint16_t*>(p.b);
  const gvec_ptr zero = gvec(&g_patch_zero16);

  // ---- patch load slots: slot j of this wavefront is 1 KB load q = 11 wave
  // + j, pixels 8 q .. 8 q + 7; lane l holds pixel 8 q + l / 8, physical
  // piece l % 8, i.e. logical piece (l % 8) ^ swz(pixel).  Offsets are within
  // one input frame (-1: outside the image or past the patch), for the tile
  // whose patches are being loaded (pg).
  int32_t poff[kPatchLoads];  // a frame has fewer than 2^31 elements (gemm_patch_ok)
  TileGeo pg;
  auto set_patch_tile = [&](const TileGeo& g) {
    pg = g;
#pragma unroll
    for (int j = 0; j < kPatchLoads; ++j) {
      const int pix = 8 * (wave * kPatchLoads + j) + (lane >> 3);
      const int lpc = (lane & 7) ^ swz(pix);
      const int py = pix / PW, px = pix - (pix / PW) * PW;
      const int32_t iy = g.oh0 - p.ph + py, ix = g.ow0 - p.pw + px;
      const bool ok = pix < PPIX && iy >= 0 && iy < H && ix >= 0 && ix < W;
      poff[j] = ok ? (iy * int32_t(W) + ix) * int32_t(C) + lpc * 8 : -1;
    }
  };
  // ---- weight load slots: slot j holds row (8 wave + j) * 8 + l / 8 of the
  // tile's 256, logical piece (l % 8) ^ swz(row), for the column tile whose
  // weights are being loaded.
  const uint16_t* brow[kBLoads];  // null: a row past O
  auto set_weight_tile = [&](int32_t n0) {
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
      const int rl = (wave * kBLoads + j) * 8 + (lane >> 3);  // row within the tile
      const int64_t row = int64_t(n0) + rl;
      const int lpc = (lane & 7) ^ swz(rl);
      brow[j] = row < N ? Bw + row * p.ldb + lpc * 8 : nullptr;
    }
  };

  const int64_t nchunk = C / 64;
  const int64_t nit = KD * nchunk;          // (depth tap, chunk) iterations per tile
  const int64_t nsteps = nit * kTaps;
  const uint32_t patch_lds = lds_base(g_patch) + wave * (kPatchLoads * 1024);
  const uint32_t w_lds = lds_base(g_wring) + wave * (kBLoads * 1024);

  // Weight rows of the tile's step ls (ls >= nsteps: the next tile's step
  // ls - nsteps; `real` false: no next tile, a zero vector) into the stage of
  // global step gs.
  auto issue_w = [&](int64_t ls, int64_t gs, bool real) {
    const uint32_t dst = w_lds + uint32_t(gs & 1) * kBStage;
    ls = ls < nsteps ? ls : ls - nsteps;
    const int64_t it = ls / kTaps, tap = ls - it * kTaps;
    const int64_t kd = it / nchunk, cc = it - kd * nchunk;
    const int64_t koff = (kd * kTaps + tap) * C + cc * 64;
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
      const gvec_ptr src = (real && brow[j]) ? gvec(brow[j] + koff) : zero;
      __builtin_amdgcn_global_load_lds(src, lds_addr(dst + j * 1024), 16, 0, 0);
    }
  };
  // Patch slots [j0, j0 + cnt) of iteration it of tile pg into the buffer of
  // global iteration gi (`real` false: a zero vector).
  auto issue_patch = [&](int64_t it, int64_t gi, bool real, int j0, int cnt) {
    const uint32_t dst = patch_lds + uint32_t(gi & 1) * kPatchBytes;
    const int64_t kd = it / nchunk, cc = it - kd * nchunk;
    int64_t base = 0;
    bool fok = real;
    if constexpr (D3) {
      const int64_t id = int64_t(pg.od) * p.sd - p.pd + kd * p.dd;
      fok = fok && id >= 0 && id < D;
      base = (int64_t(pg.img) * D + (fok ? id : 0)) * H * W * C;
    } else {
      base = int64_t(pg.f) * H * W * C;
    }
    const uint16_t* xf = X + base + cc * 64;
#pragma unroll
    for (int j = 0; j < kPatchLoads; ++j) {
      if (j >= j0 && j < j0 + cnt) {  // compile-time after unrolling at each call site
        const gvec_ptr src = (fok && poff[j] >= 0) ? gvec(xf + poff[j]) : zero;
        __builtin_amdgcn_global_load_lds(src, lds_addr(dst + j * 1024), 16, 0, 0);
      }
    }
  };

  // ---- fragment reads.  A: block i's row wm*128 + 32 i + (l & 31) is pixel
  // (py, px) of the block; tap (kh, kw) reads patch pixel (py + kh, px + kw).
  const int frow = lane & 31, khalf = lane >> 5;
  int pb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = wm * 128 + i * 32 + frow;
    pb[i] = (r / BW) * PW + (r % BW);
  }
  // B: block j's lane l supplies weight row wn*128 + 32 j + perm(l & 31), perm
  // swapping bits 2 and 3 (a permutation within each 16 rows, so the reads
  // stay conflict-free); with the operands swapped in the MFMA (below) each
  // lane's accumulators then hold 8 consecutive output channels of one pixel.
  const int brow_l = (frow & 0x13) | ((frow & 4) << 1) | ((frow & 8) >> 1);
  uint32_t rb_off[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + brow_l;
      rb_off[s][j] = uint32_t(r * kRowB + (((2 * s + khalf) ^ swz(r)) << 4));
      asm volatile("" : "+v"(rb_off[s][j]));
    }
  int pbl[4];  // pb, re-derived opaquely every iteration: the compiler would otherwise
              // hoist all 144 tap-shifted fragment addresses out of the loop
  auto read = [&](int buf, int wstage, int tap, int s, Frag& fr) {
    const int shift = (tap / 3) * PW + tap % 3;
    const uint8_t* pbase = g_patch + buf * kPatchBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int px = pbl[i] + shift;
      const uint32_t off = uint32_t(px * kRowB + (((2 * s + khalf) ^ swz(px)) << 4));
      fr.a[i] = *reinterpret_cast<const uint4*>(pbase + off);
    }
    const uint8_t* wbase = g_wring + wstage * kBStage;
#pragma unroll
    for (int j = 0; j < 4; ++j) fr.b[j] = *reinterpret_cast<const uint4*>(wbase + rb_off[s][j]);
  };

  v16f acc[4][4];
  auto mma = [&](const Frag& fr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16<BF16>(fr.b[j], fr.a[i], acc[i][j]);
  };
  auto interleave = [&]() {  // 16 MFMAs with the 8 fragment reads of the next step between them
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // ---- prologue: the first tile's first patch and the weights of its steps
  // 0 and 1; wait for the first two everywhere.
  TileGeo cur = tile_geo(0);
  set_patch_tile(cur);
  set_weight_tile(cur.n0);
  issue_patch(0, 0, true, 0, kPatchLoads);
  issue_w(0, 0, true);
  issue_w(1, 1, true);
  wait_vmcnt<kBLoads>();
  block_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frag f0, f1;
#pragma unroll
  for (int i = 0; i < 4; ++i) pbl[i] = pb[i];
  read(0, 0, 0, 0, f0);

  // One tap of local iteration it (global iteration gi, global step g = 9 gi
  // + T): its four 16-channel MFMA steps; before the last, wait until step g
  // + 1's weights (and, at the end of an iteration, the next patch) have
  // landed everywhere, then load step g + 2's weights into the stage just
  // read and a slice of the next iteration's patch, and read step g + 1's
  // first fragments.  In the tile's last iteration the loads are the next
  // tile's (nx: it exists), and from tap 7 on its weights.
  auto tap_step = [&](auto tap_c, int64_t it, int64_t gi, bool last, bool nx, const TileGeo& ng) {
    constexpr int T = decltype(tap_c)::value;
    const int64_t g = gi * kTaps + T;
    const int buf = int(gi & 1), ws = int(g & 1);
    read(buf, ws, T, 1, f1);
    mma(f0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read(buf, ws, T, 2, f0);
    mma(f1);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    read(buf, ws, T, 3, f1);
    mma(f0);
    interleave();
    __builtin_amdgcn_sched_barrier(0);
    // loads issued after step g + 1's weights: the patch slice of the step before
    wait_vmcnt_lds<(T == 0 ? 0 : kSlice[T == 0 ? 0 : T - 1])>();
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (T == 7) {
      if (last && nx) set_weight_tile(ng.n0);
    }
    const int64_t ls = it * kTaps + T + 2;
    issue_w(ls, g + 2, ls < nsteps || nx);
    if constexpr (kSlice[T] > 0) issue_patch(last ? 0 : it + 1, gi + 1, !last || nx, kSliceStart[T], kSlice[T]);
    constexpr int TN = (T + 1) % kTaps;
    read(T + 1 == kTaps ? (buf ^ 1) : buf, ws ^ 1, TN, 0, f0);
    mma(f1);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
      __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);  // VALU
    }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the next step's first reads are done
  };

  uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
  float* __restrict__ accbuf = p.acc;
  const int epi = p.epi;
  const bool vec = (p.ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
                   (accbuf == nullptr || (reinterpret_cast<uintptr_t>(accbuf) & 15) == 0);
  int64_t gi = 0;  // global iteration: patch buffer gi & 1
  for (int32_t jt = 0;; ++jt) {
    const bool nx = jt + 1 < my_tiles;
    const TileGeo ng = nx ? tile_geo(jt + 1) : cur;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    for (int64_t it = 0; it < nit; ++it, ++gi) {
      const bool last = it + 1 == nit;
      if (last && nx) set_patch_tile(ng);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pbl[i] = pb[i];
        asm volatile("" : "+v"(pbl[i]));
      }
      tap_step(ic<0>{}, it, gi, last, nx, ng);
      tap_step(ic<1>{}, it, gi, last, nx, ng);
      tap_step(ic<2>{}, it, gi, last, nx, ng);
      tap_step(ic<3>{}, it, gi, last, nx, ng);
      tap_step(ic<4>{}, it, gi, last, nx, ng);
      tap_step(ic<5>{}, it, gi, last, nx, ng);
      tap_step(ic<6>{}, it, gi, last, nx, ng);
      tap_step(ic<7>{}, it, gi, last, nx, ng);
      tap_step(ic<8>{}, it, gi, last, nx, ng);
    }

    // ---- epilogue through LDS, in the patch buffer of the tile's last
    // iteration (every wavefront passed the barrier after its last read of
    // it; the next tile's patch is in the other buffer).  acc[i][j] is the
    // transposed 32x32 block (output channels x pixels): lane l, register r
    // holds output channel 32 j + 16 (r / 8) + 8 (l / 32) + r % 8 of pixel
    // 32 i + l % 32 of the wavefront's quadrant (the B row permutation above),
    // so four consecutive registers are four consecutive channels of one
    // pixel and go to LDS in one 16-byte write.  Rounds of 32 pixels x 64
    // channels; each pixel row is then read back 8 channels per lane and
    // stored in whole lines.
    int el = lane;  // opaque copy: the address arithmetic stays inside the tile loop
    asm volatile("" : "+v"(el));
    const int h8 = 8 * (el >> 5), erow = el & 31;
    constexpr int kEpRowB = 64 * 4 + 16;  // 64 fp32 + 16 B: 16 consecutive rows hit 16 bank groups
    static_assert(4 * 32 * kEpRowB <= kPatchBytes, "the epilogue rows fit one patch buffer");
    float* e32 = reinterpret_cast<float*>(g_patch + int((gi - 1) & 1) * kPatchBytes + wave * (32 * kEpRowB));
    const int rl = el >> 3, cl = (el & 7) * 8;
    // WHOLE: the tile lies inside the output (all of its pixels and 256
    // channels), the 16-byte path applies and the epilogue stores y, so the
    // stores need no per-lane tests.
    auto round = [&](auto i_c, auto jp_c, auto whole_c) {  // compile-time indices into acc
      constexpr int i = decltype(i_c)::value, jp = decltype(jp_c)::value;
      constexpr bool WHOLE = decltype(whole_c)::value;
      const int ep_k = WHOLE ? int(kEpiStore) : epi;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
          for (int qq = 0; qq < 2; ++qq) {
            const v16f& a = acc[i][2 * jp + jj];
            const int r0 = 8 * hh + 4 * qq;
            *reinterpret_cast<float4*>(e32 + erow * (kEpRowB / 4) + 32 * jj + 16 * hh + h8 + 4 * qq) =
                make_float4(a[r0], a[r0 + 1], a[r0 + 2], a[r0 + 3]);
          }
      for (int gq = 0; gq < 4; ++gq) {
        const int rr = gq * 8 + rl;
        const float4 lo = *reinterpret_cast<const float4*>(e32 + rr * (kEpRowB / 4) + cl);
        const float4 hi = *reinterpret_cast<const float4*>(e32 + rr * (kEpRowB / 4) + cl + 4);
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        const int trow = wm * 128 + i * 32 + rr;  // row of the tile: pixel (trow / BW, trow % BW)
        const int64_t oh = cur.oh0 + trow / BW, ow = cur.ow0 + trow % BW;
        const int64_t col = int64_t(cur.n0) + wn * 128 + 64 * jp + cl;
        if (!WHOLE && (oh >= OH || ow >= OW || col >= N)) continue;
        const int64_t idx = ((int64_t(cur.f) * OH + oh) * OW + ow) * p.ldc + col;
        if (WHOLE || (vec && col + 8 <= N)) {
          if (ep_k == kEpiAccFirst || ep_k == kEpiAccMid) {
            float4* dst = reinterpret_cast<float4*>(accbuf + idx);
            if (ep_k == kEpiAccMid) {
              const float4 a0 = dst[0], a1 = dst[1];
              v[0] += a0.x; v[1] += a0.y; v[2] += a0.z; v[3] += a0.w;
              v[4] += a1.x; v[5] += a1.y; v[6] += a1.z; v[7] += a1.w;
            }
            dst[0] = make_float4(v[0], v[1], v[2], v[3]);
            dst[1] = make_float4(v[4], v[5], v[6], v[7]);
          } else {
            if (ep_k == kEpiAccLast) {
              const float4* src = reinterpret_cast<const float4*>(accbuf + idx);
              const float4 a0 = src[0], a1 = src[1];
              v[0] = a0.x + v[0]; v[1] = a0.y + v[1]; v[2] = a0.z + v[2]; v[3] = a0.w + v[3];
              v[4] = a1.x + v[4]; v[5] = a1.y + v[5]; v[6] = a1.z + v[6]; v[7] = a1.w + v[7];
            }
            uint4 o;
            o.x = uint32_t(from_f32<uint16_t, BF16>(v[0])) | (uint32_t(from_f32<uint16_t, BF16>(v[1])) << 16);
            o.y = uint32_t(from_f32<uint16_t, BF16>(v[2])) | (uint32_t(from_f32<uint16_t, BF16>(v[3])) << 16);
            o.z = uint32_t(from_f32<uint16_t, BF16>(v[4])) | (uint32_t(from_f32<uint16_t, BF16>(v[5])) << 16);
            o.w = uint32_t(from_f32<uint16_t, BF16>(v[6])) | (uint32_t(from_f32<uint16_t, BF16>(v[7])) << 16);
            const u32x4 ov = {o.x, o.y, o.z, o.w};  // written once: stored past L2
            __builtin_nontemporal_store(ov, reinterpret_cast<u32x4*>(out + idx));
          }
        } else {
          for (int q = 0; q < 8 && col + q < N; ++q) {
            const float x = v[q];
            if (epi == kEpiStore) {
              out[idx + q] = from_f32<uint16_t, BF16>(x);
            } else if (epi == kEpiAccFirst) {
              accbuf[idx + q] = x;
            } else if (epi == kEpiAccMid) {
              accbuf[idx + q] = accbuf[idx + q] + x;
            } else {
              out[idx + q] = from_f32<uint16_t, BF16>(accbuf[idx + q] + x);
            }
          }
        }
      }
    };
    auto rounds = [&](auto whole_c) {
      round(ic<0>{}, ic<0>{}, whole_c);
      round(ic<0>{}, ic<1>{}, whole_c);
      round(ic<1>{}, ic<0>{}, whole_c);
      round(ic<1>{}, ic<1>{}, whole_c);
      round(ic<2>{}, ic<0>{}, whole_c);
      round(ic<2>{}, ic<1>{}, whole_c);
      round(ic<3>{}, ic<0>{}, whole_c);
      round(ic<3>{}, ic<1>{}, whole_c);
    };
    if (vec && epi == kEpiStore && cur.oh0 + BH <= OH && cur.ow0 + BW <= OW && int64_t(cur.n0) + 256 <= N)
      rounds(std::true_type{});
    else
      rounds(std::false_type{});
    if (!nx) break;
    cur = ng;
  }
  wait_vmcnt<0>();  // the trailing zero loads land before the workgroup ends
}

// Compute units of the current device (one persistent workgroup each).
int cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <bool BF16, bool D3>
hipError_t launch_bw(const GemmParams& p, hipStream_t s) {
  const int bw = int(patch_block_w(p.oh, p.ow));
  const int64_t tiles = patch_row_tiles(p.M / (p.oh * p.ow), p.oh, p.ow) * ((p.N + kBN - 1) / kBN);
  const int64_t wgs = tiles < cu_count() ? tiles : cu_count();
  const dim3 grid{unsigned(wgs), 1u, 1u};
  if (bw == 8) hipLaunchKernelGGL((gemm_patch_kernel<BF16, D3, 8>), grid, dim3(kThreads), 0, s, p);
  else if (bw == 32) hipLaunchKernelGGL((gemm_patch_kernel<BF16, D3, 32>), grid, dim3(kThreads), 0, s, p);
  else hipLaunchKernelGGL((gemm_patch_kernel<BF16, D3, 16>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool gemm_patch_ok(const GemmParams& p) {
  if (p.dtype == CNHWC_F32 || p.a_mode != kAImplicit || p.batch != 1 || p.ksplit > 1) return false;
  if (p.kh != 3 || p.kw != 3 || p.sh != 1 || p.sw != 1 || p.dh != 1 || p.dw != 1) return false;
  if (p.c % 64 != 0 || p.ldb % 8 != 0 || p.a_seg_len != 0) return false;
  if (p.kd > 0 && p.K != p.kd * 9 * p.c) return false;
  if (p.kd == 0 && p.K != 9 * p.c) return false;
  if (p.M % (p.oh * p.ow) != 0) return false;
  // 32-bit element offsets within one input frame
  if (p.h * p.w * p.c >= (int64_t(1) << 31)) return false;
  const int64_t tiles = patch_row_tiles(p.M / (p.oh * p.ow), p.oh, p.ow) * ((p.N + kBN - 1) / kBN);
  return tiles < (int64_t(1) << 31);
}

int gemm_patch_launch(const GemmParams& p, void* stream) {
  if (!gemm_patch_ok(p)) return hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool d3 = p.kd > 0;
  if (p.dtype == CNHWC_BF16) return d3 ? launch_bw<true, true>(p, s) : launch_bw<true, false>(p, s);
  return d3 ? launch_bw<false, true>(p, s) : launch_bw<false, false>(p, s);
}

}  // namespace cnhwc
