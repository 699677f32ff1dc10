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
// MFMA: v_mfma_f32_32x32x16_{f16,bf16}; in 16-channel step s of a chunk,
// lanes 0..31 supply channels 16 s + 0..7 and lanes 32..63 16 s + 8..15 of
// their row.
#include <hip/hip_runtime.h>

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

// Workgroups go round-robin to the 8 XCDs; XCD x takes one contiguous range
// of tile indices (a bijection on [0, n)).
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t n) {
  constexpr int64_t kXcd = 8;
  const int64_t x = bid % kXcd, k = bid / kXcd;
  const int64_t q = n / kXcd, r = n % kXcd;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}
constexpr int64_t kGroupM = 8;

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

// BW: block width (output columns); the block is (256 / BW) x BW pixels.
template <bool BF16, bool D3, int BW>
__global__ __launch_bounds__(kThreads, 1) void gemm_patch_kernel(const GemmParams p) {
  constexpr int BH = 256 / BW;
  constexpr int PW = BW + 2, PH = BH + 2, PPIX = PH * PW;
  static_assert(PPIX * kRowB <= kPatchBytes, "the patch fits its buffer");
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t N = p.N, C = p.c, H = p.h, W = p.w, OH = p.oh, OW = p.ow;
  const int64_t OD = D3 ? p.od : 1, KD = D3 ? p.kd : 1, D = D3 ? p.d : 1;
  const int64_t frames = p.M / (OH * OW);  // output images (2D) or frames n * OD + od (3D)

  // ---- tile: (frame, block row, block column) x column tile, in groups of
  // kGroupM row tiles per XCD range so that concurrent workgroups share rows.
  const int64_t tby = (OH + BH - 1) / BH, tbx = (OW + BW - 1) / BW;
  const int64_t mt = frames * tby * tbx, nt = (N + kBN - 1) / kBN;
  const int64_t t = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t group = t / (kGroupM * nt);
  const int64_t first_m = group * kGroupM;
  const int64_t gsz = mt - first_m < kGroupM ? mt - first_m : kGroupM;
  const int64_t tg = t - group * (kGroupM * nt);
  const int64_t mtile = first_m + tg % gsz;
  const int64_t n0 = (tg / gsz) * kBN;
  const int64_t f = mtile / (tby * tbx);
  const int64_t rb = mtile - f * (tby * tbx);
  const int64_t by = rb / tbx, bx = rb - by * tbx;
  const int64_t oh0 = by * BH, ow0 = bx * BW;
  const int64_t img = f / OD, od = f - img * OD;  // input element and output frame
  const uint16_t* __restrict__ X = reinterpret_cast<const uint16_t*>(p.a);
  const uint16_t* __restrict__ Bw = reinterpret_cast<const uint16_t*>(p.b);
  const gvec_ptr zero = gvec(&g_patch_zero16);

  // ---- patch load slots: slot j of this wavefront is 1 KB load q = 11 wave
  // + j, pixels 8 q .. 8 q + 7; lane l holds pixel 8 q + l / 8, physical
  // piece l % 8, i.e. logical piece (l % 8) ^ (pixel & 7).  Offsets are within
  // one input frame (-1: outside the image or past the patch).
  int32_t poff[kPatchLoads];  // a frame has fewer than 2^31 elements (gemm_patch_ok)
#pragma unroll
  for (int j = 0; j < kPatchLoads; ++j) {
    const int pix = 8 * (wave * kPatchLoads + j) + (lane >> 3);
    const int lpc = (lane & 7) ^ swz(pix);
    const int py = pix / PW, px = pix - (pix / PW) * PW;
    const int64_t iy = oh0 - p.ph + py, ix = ow0 - p.pw + px;
    const bool ok = pix < PPIX && iy >= 0 && iy < H && ix >= 0 && ix < W;
    poff[j] = ok ? int32_t((iy * W + ix) * C + lpc * 8) : -1;
  }
  // ---- weight load slots: slot j holds row (8 wave + j) * 8 + l / 8 of the
  // tile's 256, logical piece (l % 8) ^ (row & 7) (row & 7 == l / 8).
  const uint16_t* brow[kBLoads];  // null: a row past O
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int rl = (wave * kBLoads + j) * 8 + (lane >> 3);  // row within the tile
    const int64_t row = n0 + rl;
    const int lpc = (lane & 7) ^ swz(rl);
    brow[j] = row < N ? Bw + row * p.ldb + lpc * 8 : nullptr;
  }

  const int64_t nchunk = C / 64;
  const int64_t nit = KD * nchunk;          // (depth tap, chunk) iterations
  const int64_t nsteps = nit * kTaps;
  const uint32_t patch_lds = lds_base(g_patch) + wave * (kPatchLoads * 1024);
  const uint32_t w_lds = lds_base(g_wring) + wave * (kBLoads * 1024);

  // Weight rows of global step g into stage g & 1 (past the end the rows
  // wrap around to real data, loaded into a stage that is never read again;
  // the stage still follows the unwrapped g, which keeps it off the stage in
  // use).
  auto issue_w = [&](int64_t g) {
    const uint32_t dst = w_lds + uint32_t(g & 1) * kBStage;
    g = g < nsteps ? g : g - nsteps;
    const int64_t it = g / kTaps, tap = g - it * kTaps;
    const int64_t kd = it / nchunk, cc = it - kd * nchunk;
    const int64_t koff = (kd * kTaps + tap) * C + cc * 64;
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) {
      const gvec_ptr src = brow[j] ? gvec(brow[j] + koff) : zero;
      __builtin_amdgcn_global_load_lds(src, lds_addr(dst + j * 1024), 16, 0, 0);
    }
  };
  // Patch slots [j0, j0 + cnt) of iteration it into buffer it & 1 (past the
  // end the data wraps around; the buffer follows the unwrapped it).
  auto issue_patch = [&](int64_t it, int j0, int cnt) {
    const uint32_t dst = patch_lds + uint32_t(it & 1) * kPatchBytes;
    it = it < nit ? it : it - nit;
    const int64_t kd = it / nchunk, cc = it - kd * nchunk;
    int64_t base = 0;
    bool fok = true;
    if constexpr (D3) {
      const int64_t id = od * p.sd - p.pd + kd * p.dd;
      fok = id >= 0 && id < D;
      base = (img * D + (fok ? id : 0)) * H * W * C;
    } else {
      base = f * H * W * C;
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
  uint32_t rb_off[4][4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 128 + j * 32 + frow;
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
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  auto mma = [&](const Frag& fr) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16<BF16>(fr.a[i], fr.b[j], acc[i][j]);
  };
  auto interleave = [&]() {  // 16 MFMAs with the 8 fragment reads of the next step between them
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // ---- prologue: iteration 0's patch, the weights of steps 0 and 1; wait for
  // the first two everywhere.
  issue_patch(0, 0, kPatchLoads);
  issue_w(0);
  issue_w(1);
  wait_vmcnt<kBLoads>();
  block_barrier();
  __builtin_amdgcn_sched_barrier(0);
  Frag f0, f1;
#pragma unroll
  for (int i = 0; i < 4; ++i) pbl[i] = pb[i];
  read(0, 0, 0, 0, f0);

  // One tap of iteration it (global step g = 9 it + T): its four 16-channel
  // MFMA steps; before the last, wait until step g + 1's weights (and, at the
  // end of an iteration, the next patch) have landed everywhere, then load
  // step g + 2's weights into the stage just read and a slice of the next
  // iteration's patch, and read step g + 1's first fragments.
  auto tap_step = [&](auto tap_c, int64_t it) {
    constexpr int T = decltype(tap_c)::value;
    const int64_t g = it * kTaps + T;
    const int buf = int(it & 1), ws = int(g & 1);
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
    issue_w(g + 2);
    if constexpr (kSlice[T] > 0) issue_patch(it + 1, kSliceStart[T], kSlice[T]);
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
  for (int64_t it = 0; it < nit; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pbl[i] = pb[i];
      asm volatile("" : "+v"(pbl[i]));
    }
    tap_step(ic<0>{}, it);
    tap_step(ic<1>{}, it);
    tap_step(ic<2>{}, it);
    tap_step(ic<3>{}, it);
    tap_step(ic<4>{}, it);
    tap_step(ic<5>{}, it);
    tap_step(ic<6>{}, it);
    tap_step(ic<7>{}, it);
    tap_step(ic<8>{}, it);
  }
  wait_vmcnt<0>();  // the trailing loads must land before LDS is reused

  // ---- epilogue through LDS, one 32-row slice of the wavefront's quadrant at
  // a time (layout as in gemm_lds.hip): D[row][col] of a 32x32 block sits in
  // lane l, register r at row = 8 (r / 4) + 4 (l / 32) + r % 4, col = l % 32.
  block_barrier();  // every wavefront has finished its LDS reads
  constexpr int WN = 128, EP = WN + 4;
  float* ep = reinterpret_cast<float*>(g_patch + wave * (32 * EP * 4));
  static_assert(4 * 32 * EP * 4 <= 2 * kPatchBytes, "the epilogue slices fit the patch buffers");
  uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out);
  float* __restrict__ accbuf = p.acc;
  const int epi = p.epi;
  const bool vec = (p.ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
                   (accbuf == nullptr || (reinterpret_cast<uintptr_t>(accbuf) & 15) == 0);
  constexpr int LPR = WN / 8, RPG = 64 / LPR;
  const int rl = lane / LPR, cl = (lane % LPR) * 8;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EP + 32 * j + (lane & 31)] = acc[i][j][r];
    for (int g = 0; g < 32 / RPG; ++g) {
      const int rr = g * RPG + rl;
      const int trow = wm * 128 + i * 32 + rr;  // row of the tile: pixel (trow / BW, trow % BW)
      const int64_t oh = oh0 + trow / BW, ow = ow0 + trow % BW;
      const int64_t col = n0 + wn * WN + cl;
      const float4 lo = *reinterpret_cast<const float4*>(ep + rr * EP + cl);
      const float4 hi = *reinterpret_cast<const float4*>(ep + rr * EP + cl + 4);
      float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      if (oh >= OH || ow >= OW || col >= N) continue;
      const int64_t idx = ((f * OH + oh) * OW + ow) * p.ldc + col;
      if (vec && col + 8 <= N) {
        if (epi == kEpiAccFirst || epi == kEpiAccMid) {
          float4* dst = reinterpret_cast<float4*>(accbuf + idx);
          if (epi == kEpiAccMid) {
            const float4 a0 = dst[0], a1 = dst[1];
            v[0] += a0.x; v[1] += a0.y; v[2] += a0.z; v[3] += a0.w;
            v[4] += a1.x; v[5] += a1.y; v[6] += a1.z; v[7] += a1.w;
          }
          dst[0] = make_float4(v[0], v[1], v[2], v[3]);
          dst[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
          if (epi == kEpiAccLast) {
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
          *reinterpret_cast<uint4*>(out + idx) = o;
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
  }
}

template <bool BF16, bool D3>
hipError_t launch_bw(const GemmParams& p, hipStream_t s) {
  const int bw = int(patch_block_w(p.oh, p.ow));
  const int64_t tiles = patch_row_tiles(p.M / (p.oh * p.ow), p.oh, p.ow) * ((p.N + kBN - 1) / kBN);
  const dim3 grid{unsigned(tiles), 1u, 1u};
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
