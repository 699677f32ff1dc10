// Large-tile fp16/bf16 MFMA GEMM for gfx950 with direct global -> LDS loads.
//
// C[M x N] = A[M x K] * B[N x K]^T for the implicit-GEMM conv (MLX PR "Bound
// winograd conv2d working set by tiling the batch", Fix: the scratch-free
// fallback; MLX PR "Use the explicit gemm for wide convs on neural
// accelerators", intro: the wide-channel convs) and the per-tap 2D convs of the
// 3D decomposition (MLX PR "Decompose small kernel-depth 3D convs into 2D
// convs", Change).  A is gathered from the NHWC image (or read as dense rows
// after an unfold), B is the weight rows [O][KH][KW][C], K-contiguous.
//
// Why a second GEMM core: with 64 x 64 wavefront tiles the MFMA fragments read
// from LDS alone take about one LDS cycle per matrix-core cycle, and staging
// the operands through registers into LDS adds half as much again, more than
// one CU's LDS can serve.  Here:
//  - a workgroup of 4 wavefronts owns a 256 x 256 output tile, each wavefront
//    a 128 x 128 quadrant (16 accumulating 32x32 blocks, 256 fp32 per lane),
//    which halves the LDS bytes read per MFMA;
//  - operands go from global memory straight into LDS
//    (global_load_lds_dwordx4: lane l's 16 bytes land at the wave's LDS base
//    + 16 l), so no VGPRs and no ds_write are spent on staging;
//  - K advances in chunks of 32 elements (64-byte LDS rows) through a ring of
//    four LDS stages: while a chunk feeds the matrix cores up to three more
//    are in flight, and one barrier per chunk orders reuse of a stage (the
//    implicit gather with C % 64 == 0 uses 64-element chunks in two stages
//    instead: whole 128-byte lines per load);
//  - each chunk's loads, their address arithmetic and the fragment reads are
//    interleaved with the MFMAs (scheduling groups), and the loop body is one
//    basic block, so the matrix cores are not left idle while they issue.
// LDS rows hold four (eight) 16-byte pieces, the piece index XOR-ed with bits
// of the row (see piece()), so the 8 lanes served per LDS cycle (8
// consecutive rows, same logical piece) hit 8 distinct 16-byte bank groups.
// Since a lane's LDS destination is fixed by its lane index, the swizzle is
// applied on the global side: lane l fetches the logical piece that belongs
// at its slot.
//
// MFMA: v_mfma_f32_32x32x16_{f16,bf16}; in K step q (0..1, or 0..3 with
// 64-element chunks) of a chunk, lanes 0..31 supply k = 16 q + 0..7 and lanes
// 32..63 k = 16 q + 8..15 of their row.  Every output adds its K products 16
// at a time in ascending K whatever the chunk size, so the result does not
// depend on the chunk form, on M, on the grid or on the launch a row is in.
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "device_common.hpp"

namespace cnhwc {
namespace {

constexpr int kBM = 256;  // tile rows
constexpr int kThreads = 256;

// Physical 16-byte piece of logical piece c in LDS row r, so that 16
// consecutive rows of one logical piece (the lanes a 16-byte LDS read serves
// together) hit 16 distinct 16-byte bank groups of the 64 four-byte banks:
// 64-byte rows (4 pieces, four rows per 256-byte bank line) XOR bits 2..3 of
// the row; 128-byte rows (8 pieces, two rows per bank line) XOR bits 1..3.
template <int PIECES>
__device__ __forceinline__ int piece(int r, int c) {
  if constexpr (PIECES == 4) return c ^ ((r >> 2) & 3);
  else return c ^ ((r >> 1) & 7);
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gvec_ptr;
__device__ u32x4 g_lds_zero16 = {0u, 0u, 0u, 0u};
template <typename T>
__device__ __forceinline__ gvec_ptr gvec(const T* p) {
  return (gvec_ptr)(p);
}

constexpr int64_t kGroupM = 8;

// Bijection on [0, n): the workgroups dispatched to XCD x (ids x, x + 8, ...)
// get one contiguous range of tile indices.
__device__ __forceinline__ int64_t xcd_tile(int64_t bid, int64_t n) {
  constexpr int64_t kXcd = 8;
  const int64_t x = bid % kXcd, k = bid / kXcd;
  const int64_t q = n / kXcd, r = n % kXcd;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + k;
}

// Tile shapes.  4 wavefronts in a 2 x 2 grid; each owns (kBM/2) x (BN/2).
//  - 256 x 256, 4 stages of 32-element K chunks, one workgroup per CU
//    (128 KB of LDS);
//  - the same tile with 2 stages of 64-element chunks (same LDS) for the
//    implicit gather with C % 64 == 0: every load brings a whole 128-byte
//    line of its row, half the line requests per byte;
//  - 256 x 128, 3 stages, two workgroups per CU (72 KB each): the other
//    workgroup's MFMAs cover one workgroup's waits for its loads.
// All three add the K products 16 at a time in ascending K, so they give the
// same bits.
template <int BN_, int NS_, int OCC_, int KB_ = 32>
struct LdsTile {
  static constexpr int BN = BN_, NS = NS_, OCC = OCC_;
  static constexpr int KB = KB_;                 // K chunk in elements
  static constexpr int ROWB = KB * 2;            // bytes of one row per chunk
  static constexpr int PIECES = ROWB / 16;       // 16-byte pieces per LDS row
  static constexpr int STEPS = KB / 16;          // MFMA K steps per chunk
  static constexpr int RPL = 64 * 16 / ROWB;     // rows one wavefront load instruction fills
  static constexpr int WN = BN / 2;              // wavefront tile columns
  static constexpr int FN = WN / 32;             // 32x32 accumulators per 32-row group
  static constexpr int LOADS_A = kBM * ROWB / (kThreads * 16);  // 16-byte loads per thread per chunk
  static constexpr int LOADS_B = BN * ROWB / (kThreads * 16);
  static constexpr int LOADS = LOADS_A + LOADS_B;
  static constexpr int RING_A = NS * kBM * ROWB, RING_B = NS * BN * ROWB;
};
using Tile256 = LdsTile<256, 4, 1>;
using Tile256W = LdsTile<256, 2, 1, 64>;
using Tile128 = LdsTile<128, 3, 2>;
static_assert(Tile256W::RING_A == Tile256::RING_A && Tile256W::RING_B == Tile256::RING_B,
              "the two 256 x 256 forms share one ring");

// Each tile shape's stage ring lives in two LDS objects, A rows and B rows:
// the compiler then tags every fragment read with the object it reads.  The
// loads into LDS address the ring through a plain integer LDS address (see
// lds_addr), which carries no such tag, so the compiler adds no wait of its
// own before a fragment read; the explicit vmcnt waits and barriers below
// order them.
__shared__ __attribute__((aligned(1024))) uint8_t g_ring_a[Tile256::RING_A];
__shared__ __attribute__((aligned(1024))) uint8_t g_ring_b[Tile256::RING_B];
__shared__ __attribute__((aligned(1024))) uint8_t g_ring_a2[Tile128::RING_A];
__shared__ __attribute__((aligned(1024))) uint8_t g_ring_b2[Tile128::RING_B];
template <class T>
__device__ __forceinline__ uint8_t* ring_a_obj() {
  if constexpr (T::BN == 256) return g_ring_a;
  else return g_ring_a2;
}
template <class T>
__device__ __forceinline__ uint8_t* ring_b_obj() {
  if constexpr (T::BN == 256) return g_ring_b;
  else return g_ring_b2;
}

typedef void __attribute__((address_space(3)))* lds_ptr;
__device__ __forceinline__ uint32_t lds_base(const uint8_t* p) {
  typedef const uint8_t __attribute__((address_space(3)))* lds_cptr;
  uint32_t v = uint32_t(reinterpret_cast<uintptr_t>((lds_cptr)p));
  asm volatile("" : "+s"(v));  // opaque to constant folding; emits no instruction
  return v;
}
__device__ __forceinline__ lds_ptr lds_addr(uint32_t a) {
  return reinterpret_cast<lds_ptr>(uintptr_t(a));
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
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

// Workgroup barrier that the compiler may not move memory accesses across
// (the signal fences emit no instruction and no wait; the LDS ordering
// itself comes from the explicit vmcnt waits before each barrier).
__device__ __forceinline__ void block_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int FN>
struct Frag {
  uint4 a[4];
  uint4 b[FN];
};

// D3: the implicit A operand is a 3D NDHWC gather (depth window as well).
template <class T, bool BF16, bool IMPLICIT, bool D3 = false>
__global__ __launch_bounds__(kThreads, T::OCC) void gemm_lds_kernel(const GemmParams p) {
  constexpr int kBN = T::BN, kStages = T::NS, kLoadsB = T::LOADS_B, kLoads = T::LOADS;
  constexpr int WN = T::WN, FN = T::FN;
  constexpr int kBK = T::KB, kRowBytes = T::ROWB, kStageBytes = kBM * T::ROWB;
  constexpr int kLoadsA = T::LOADS_A, kRowsPerLoad = T::RPL, kSteps = T::STEPS, kPieces = T::PIECES;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t M = p.M, N = p.N, K = p.K;

  // Tile order: workgroups are dealt round-robin to the 8 XCDs (one L2
  // each).  XCD x takes a contiguous range of tile indices, walked in groups
  // of kGroupM row tiles: the 32 workgroups an XCD runs at once then cover
  // about 8 row tiles x 4 column tiles and share their A and B rows in L2.
  const int64_t mt = (M + kBM - 1) / kBM, nt = (N + kBN - 1) / kBN;
  const int64_t t_all = xcd_tile(blockIdx.x, gridDim.x);
  const int64_t bz = t_all / (mt * nt);
  const int64_t t = t_all - bz * (mt * nt);
  const int64_t group = t / (kGroupM * nt);
  const int64_t first_m = group * kGroupM;
  const int64_t gsz = mt - first_m < kGroupM ? mt - first_m : kGroupM;
  const int64_t tg = t - group * (kGroupM * nt);
  const int64_t m0 = (first_m + tg % gsz) * kBM;
  const int64_t n0 = (tg / gsz) * kBN;
  const uint16_t* __restrict__ A = reinterpret_cast<const uint16_t*>(p.a) + bz * p.stride_a;
  const uint16_t* __restrict__ B = reinterpret_cast<const uint16_t*>(p.b) + bz * p.stride_b;

  // ---- this lane's load slots: row lane / kPieces of each block of
  // kRowsPerLoad rows (16 rows of 64 bytes, or 8 of 128), piece slot
  // lane % kPieces, holding the logical piece the row swizzle puts there (the
  // swizzle is its own inverse).  The swizzle depends on the row modulo 16:
  // with 16-row blocks that is the same for every block (kin), with 8-row
  // blocks it alternates from block to block (kin_of).
  const int lrow = lane / kPieces;
  auto kin_of = [&](int row_in_tile) { return piece<kPieces>(row_in_tile, lane % kPieces) * 8; };
  const int kin = kin_of(lrow);  // element offset of the piece within the chunk (16-row blocks)

  int64_t a_off[kLoadsA];
  int32_t a_ih0[kLoadsA], a_iw0[kLoadsA], a_id0[kLoadsA];
#pragma unroll
  for (int j = 0; j < kLoadsA; ++j) {
    const int rt = (wave * kLoadsA + j) * kRowsPerLoad + lrow;  // row within the tile
    const int64_t m = m0 + rt;
    const int kin_j = kin_of(rt);
    a_id0[j] = 0;
    if (!IMPLICIT) {
      a_off[j] = m < M ? m * p.lda + kin_j : -1;
      a_ih0[j] = a_iw0[j] = 0;
    } else if (m < M) {
      const int64_t hw = p.oh * p.ow;
      int64_t n, r;
      if constexpr (D3) {
        const int64_t dhw = p.od * hw;
        n = m / dhw;
        r = m - n * dhw;
        const int64_t od = r / hw;
        r -= od * hw;
        a_id0[j] = int32_t(od * p.sd - p.pd);
      } else {
        n = m / hw;
        r = m - n * hw;
      }
      const int64_t oh = r / p.ow;
      const int64_t ow = r - oh * p.ow;
      a_ih0[j] = int32_t(oh * p.sh - p.ph);
      a_iw0[j] = int32_t(ow * p.sw - p.pw);
      const int64_t depth = D3 ? p.d : 1;
      a_off[j] = n * depth * p.h * p.w * p.c +
                 ((int64_t(a_id0[j]) * p.h + a_ih0[j]) * p.w + a_iw0[j]) * p.c + kin_j;
    } else {
      a_off[j] = 0;
      a_ih0[j] = -0x40000000;
      a_iw0[j] = -0x40000000;
      a_id0[j] = -0x40000000;
    }
  }
  int64_t b_off[kLoadsB];
#pragma unroll
  for (int j = 0; j < kLoadsB; ++j) {
    const int rt = (wave * kLoadsB + j) * kRowsPerLoad + lrow;
    const int64_t n = n0 + rt;
    b_off[j] = n < N ? n * p.ldb + kin_of(rt) : -1;
  }

  // ---- K position of the next chunk to issue (implicit: C is a multiple of
  // the chunk, 32 or 64 elements, so a chunk never straddles two taps and its
  // tap is wave-uniform).  Chunks past
  // the end are issued too (dense: as zero loads), so every wait count is
  // fixed.
  int64_t k_next = 0;
  int32_t t_c = 0, t_kh = 0, t_kw = 0, t_kd = 0;
  // segmented dense A: K position within the segment, and the row shift of
  // the segments passed so far (a_seg_len == 0 never wraps)
  int64_t seg_k = 0, seg_off = 0;
  // dense operands: element offset of the next chunk (row-major: k_next;
  // K-chunk-major: chunk index x a_kstep / b_kstep)
  const int64_t a_step = p.a_kstep ? p.a_kstep : kBK, b_step = p.b_kstep ? p.b_kstep : kBK;
  int64_t a_k = 0, b_k = 0;
  const gvec_ptr zero = gvec(&g_lds_zero16);

  const uint32_t ring_a = lds_base(ring_a_obj<T>()) + wave * (kLoadsA * 64 * 16);
  const uint32_t ring_b = lds_base(ring_b_obj<T>()) + wave * (kLoadsB * 64 * 16);
  auto issue = [&](int stg) {
    const uint32_t sa = ring_a + stg * kStageBytes;
    const uint32_t sb = ring_b + stg * (kBN * kRowBytes);
    if constexpr (IMPLICIT) {
      // Branch-free, so the address arithmetic can be interleaved with the
      // MFMAs.  Chunks past the end wrap around to tap 0 and load real data,
      // which lands in stages that are never read again.
      const int32_t dhh = t_kh * p.dh, dww = t_kw * p.dw, ddd = D3 ? t_kd * p.dd : 0;
      const int64_t tap_off = ((int64_t(ddd) * p.h + dhh) * p.w + dww) * p.c + t_c;
#pragma unroll
      for (int j = 0; j < kLoadsA; ++j) {
        bool ok = (uint32_t(a_ih0[j] + dhh) < uint32_t(p.h)) &
                  (uint32_t(a_iw0[j] + dww) < uint32_t(p.w));
        if constexpr (D3) ok = ok & (uint32_t(a_id0[j] + ddd) < uint32_t(p.d));
        const gvec_ptr src = ok ? gvec(A + a_off[j] + tap_off) : zero;
        __builtin_amdgcn_global_load_lds(src, lds_addr(sa + j * (64 * 16)), 16, 0, 0);
      }
      const int64_t kb = k_next < K ? k_next : 0;
#pragma unroll
      for (int j = 0; j < kLoadsB; ++j) {
        const gvec_ptr src = b_off[j] >= 0 ? gvec(B + b_off[j] + kb) : zero;
        __builtin_amdgcn_global_load_lds(src, lds_addr(sb + j * (64 * 16)), 16, 0, 0);
      }
      t_c += kBK;
      const bool wc = t_c == p.c;
      t_c = wc ? 0 : t_c;
      t_kw += wc ? 1 : 0;
      const bool ww = t_kw == p.kw;
      t_kw = ww ? 0 : t_kw;
      t_kh += ww ? 1 : 0;
      if constexpr (D3) {
        const bool wh = t_kh == p.kh;
        t_kh = wh ? 0 : t_kh;
        t_kd += wh ? 1 : 0;
        t_kd = t_kd == p.kd ? 0 : t_kd;
      } else {
        t_kh = t_kh == p.kh ? 0 : t_kh;
      }
    } else {
      static_assert(kRowsPerLoad == 16, "dense A uses 16-row load blocks: kin is every slot's offset");
      const bool k_in = k_next + kin < K;
#pragma unroll
      for (int j = 0; j < kLoadsA; ++j) {
        const gvec_ptr src = (a_off[j] >= 0 && k_in) ? gvec(A + a_off[j] + a_k + seg_off) : zero;
        __builtin_amdgcn_global_load_lds(src, lds_addr(sa + j * (64 * 16)), 16, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < kLoadsB; ++j) {
        const gvec_ptr src = (b_off[j] >= 0 && k_in) ? gvec(B + b_off[j] + b_k) : zero;
        __builtin_amdgcn_global_load_lds(src, lds_addr(sb + j * (64 * 16)), 16, 0, 0);
      }
      seg_k += kBK;
      const bool sw = seg_k == p.a_seg_len;
      seg_k = sw ? 0 : seg_k;
      seg_off += sw ? p.a_seg_jump : 0;
      a_k += a_step;
      b_k += b_step;
    }
    k_next += kBK;
  };

  // ---- fragment reads: lane's A rows wm*128 + 32 i + (lane & 31), B rows
  // wn*128 + 32 j + (lane & 31), logical piece 2 q + (lane >> 5), physical
  // piece piece<kPieces>(row, that) (it depends on the row modulo 16 only, so
  // it is the same for all four 32-row groups).
  // Each read is addressed as ring + (offset + stage base) with the offsets
  // precomputed and kept opaque, so the compiler sees every fragment read as a
  // read of its ring object (and tags it so).
  const int frow = lane & 31;
  const int khalf = lane >> 5;
  uint32_t ra_off[kSteps][4], rb_off[kSteps][FN];
#pragma unroll
  for (int q = 0; q < kSteps; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t ph = uint32_t(piece<kPieces>(frow, 2 * q + khalf) << 4);
      ra_off[q][i] = uint32_t((wm * 128 + i * 32 + frow) * kRowBytes) + ph;
      asm volatile("" : "+v"(ra_off[q][i]));
      if (i < FN) {
        rb_off[q][i] = uint32_t((wn * WN + i * 32 + frow) * kRowBytes) + ph;
        asm volatile("" : "+v"(rb_off[q][i]));
      }
    }
  auto read = [&](int stg, int q, Frag<FN>& f) {
    const uint32_t sa = uint32_t(stg * kStageBytes), sb = uint32_t(stg * kBN * kRowBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const uint4*>(ring_a_obj<T>() + (ra_off[q][i] + sa));
#pragma unroll
    for (int j = 0; j < FN; ++j) f.b[j] = *reinterpret_cast<const uint4*>(ring_b_obj<T>() + (rb_off[q][j] + sb));
  };

  v16f acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto mma = [&](const Frag<FN>& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma_32x32x16<BF16>(f.a[i], f.b[j], acc[i][j]);
  };

  const int64_t nk = (K + kBK - 1) / kBK;
  Frag<FN> f0, f1;
  // step q's MFMAs with the fragment reads of step q + 1 interleaved
  auto step_with_reads = [&]() {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
  };
  if constexpr (kBK == 64) {
    static_assert(kStages == 2 && FN == 4 && kSteps == 4, "the 64-element form is the 256 x 256 tile");
    // Two stages.  Prologue: both filled; wait for chunk 0 everywhere.
    issue(0);
    issue(1);
    wait_vmcnt<kLoads>();
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read(0, 0, f0);
    // Chunk kc sits in stage cur, its K step 0 fragments in f0.  After its
    // step 2 every wavefront holds step 3 in f1; once chunk kc + 1 has landed
    // everywhere (the only loads in flight) the barrier lets stage cur take
    // chunk kc + 2 while step 3 runs, so each chunk has a whole chunk period
    // to arrive.
    int cur = 0;
    for (int64_t kc = 0; kc < nk; ++kc) {
      const int nxt = cur ^ 1;
      read(cur, 1, f1);
      mma(f0);
      step_with_reads();
      __builtin_amdgcn_sched_barrier(0);
      read(cur, 2, f0);
      mma(f1);
      step_with_reads();
      __builtin_amdgcn_sched_barrier(0);
      read(cur, 3, f1);
      mma(f0);
      step_with_reads();
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lds<0>();
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // the chunk after next and the next chunk's K step 0 reads, interleaved
      // with step 3's MFMAs: one load into LDS per MFMA
      issue(cur);
      read(nxt, 0, f0);
      mma(f1);
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);  // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 1);  // VALU
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      cur = nxt;
    }
  } else {
    // Prologue: chunks 0 .. kStages-2 in flight; wait for chunk 0 everywhere.
  #pragma unroll
    for (int i = 0; i < kStages - 1; ++i) issue(i);
    wait_vmcnt<(kStages - 2) * kLoads>();
    block_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read(0, 0, f0);

    // Chunk kc sits in stage cur; its K step 0 fragments are already in f0.
    // Mid-chunk: wait until chunk kc + 1 has landed everywhere.  After that
    // barrier every wavefront has also issued all MFMAs of chunk kc - 1, so its
    // reads are done and stage cur - 1 can take chunk kc + kStages - 1.
    int cur = 0;
    for (int64_t kc = 0; kc < nk; ++kc) {
      const int nxt = cur + 1 == kStages ? 0 : cur + 1;
      const int prv = cur == 0 ? kStages - 1 : cur - 1;
      // K step 1 reads interleaved with K step 0 MFMAs
      read(cur, 1, f1);
      mma(f0);
      if constexpr (FN == 4) {
  #pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // two MFMAs
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
      } else {
  #pragma unroll
        for (int g = 0; g < 4 + FN; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<(kStages - 3) * kLoads>();
      block_barrier();
      __builtin_amdgcn_sched_barrier(0);
      // The next chunk's loads and K step 0 reads interleaved with K step 1
      // MFMAs: per MFMA one load into LDS and its address arithmetic, and a
      // fragment read every other MFMA.
      issue(prv);
      read(nxt, 0, f0);
      mma(f1);
      if constexpr (FN == 4) {
  #pragma unroll
        for (int g = 0; g < 8; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);  // VALU
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
          __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);  // VALU
        }
      } else {
  #pragma unroll
        for (int g = 0; g < kLoads; ++g) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 1);  // load into LDS
          __builtin_amdgcn_sched_group_barrier(0x002, 8, 1);  // VALU
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);  // LDS read
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      // The next chunk's step 0 reads were issued 16 MFMAs ago and are done;
      // saying so here lets the loop head wait for its own reads only.
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      cur = nxt;
    }
  }
  wait_vmcnt<0>();  // the trailing zero loads must land before LDS is reused

  // ---- epilogue through LDS, one 32-row slice of the wavefront's quadrant
  // at a time.  D[row][col] of a 32x32 block sits in lane l, register r at
  // row = 8 (r / 4) + 4 (l / 32) + r % 4, col = l % 32; the slice is written to
  // the wavefront's own LDS area and read back as 8 consecutive columns per
  // lane, 16 lanes per row, so global stores are 16-byte and row-contiguous.
  block_barrier();  // every wavefront has finished its LDS reads
  constexpr int EP = WN + 4;     // padded slice row (floats)
  static_assert(32 * EP * 4 <= T::RING_B / 2, "an epilogue slice fits half a ring");
  float* ep = reinterpret_cast<float*>(wave < 2 ? ring_a_obj<T>() + (wave & 1) * (T::RING_A / 2)
                                                : ring_b_obj<T>() + (wave & 1) * (T::RING_B / 2));
  uint16_t* __restrict__ out = reinterpret_cast<uint16_t*>(p.out) + bz * p.stride_out;
  float* __restrict__ accbuf = p.acc ? p.acc + bz * p.stride_out : nullptr;
  const int epi = p.epi;
  const bool vec = (p.ldc % 8) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0 &&
                   (accbuf == nullptr || (reinterpret_cast<uintptr_t>(accbuf) & 15) == 0);
  constexpr int LPR = WN / 8;      // lanes per slice row (8 columns each)
  constexpr int RPG = 64 / LPR;    // slice rows per group of 64 lanes
  const int rl = lane / LPR;       // row within a group
  const int cl = (lane % LPR) * 8; // first column of this lane's 8
  // One pass over the quadrant for epilogue EPI (-1: any, read from p.epi).
  // WHOLE: the tile lies inside M x N and the 16-byte path applies to every
  // lane, so the stores need no per-lane tests.  16-bit outputs are stored
  // non-temporally (written once; 4% faster on the C_out 4096 unfold GEMM);
  // fp32 rows stay plain stores (non-temporal ones made the Winograd GEMMs up
  // to 37% slower).
  auto pass = [&](auto epi_c, auto whole_c) {
    constexpr int EPI = decltype(epi_c)::value;
    constexpr bool WHOLE = decltype(whole_c)::value;
    const int ep_k = EPI >= 0 ? EPI : epi;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          ep[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * EP + 32 * j + (lane & 31)] = acc[i][j][r];
      for (int g = 0; g < 32 / RPG; ++g) {
        const int rr = g * RPG + rl;
        const int64_t row = m0 + wm * 128 + i * 32 + rr;
        const int64_t col = n0 + wn * WN + cl;
        const float4 lo = *reinterpret_cast<const float4*>(ep + rr * EP + cl);
        const float4 hi = *reinterpret_cast<const float4*>(ep + rr * EP + cl + 4);
        float v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
        if (!WHOLE && (row >= M || col >= N)) continue;
        const int64_t idx = row * p.ldc + col;
        if (WHOLE || (vec && col + 8 <= N)) {
          if (ep_k == kEpiAccFirst || ep_k == kEpiAccMid) {
            f32x4* dst = reinterpret_cast<f32x4*>(accbuf + idx);
            if (ep_k == kEpiAccMid) {
              const f32x4 a0 = dst[0], a1 = dst[1];
              v[0] += a0.x; v[1] += a0.y; v[2] += a0.z; v[3] += a0.w;
              v[4] += a1.x; v[5] += a1.y; v[6] += a1.z; v[7] += a1.w;
            }
            dst[0] = f32x4{v[0], v[1], v[2], v[3]};
            dst[1] = f32x4{v[4], v[5], v[6], v[7]};
          } else {
            if (ep_k == kEpiAccLast) {
              const float4* src = reinterpret_cast<const float4*>(accbuf + idx);
              const float4 a0 = src[0], a1 = src[1];
              v[0] = a0.x + v[0]; v[1] = a0.y + v[1]; v[2] = a0.z + v[2]; v[3] = a0.w + v[3];
              v[4] = a1.x + v[4]; v[5] = a1.y + v[5]; v[6] = a1.z + v[6]; v[7] = a1.w + v[7];
            }
            const u32x4 o = {
                uint32_t(from_f32<uint16_t, BF16>(v[0])) | (uint32_t(from_f32<uint16_t, BF16>(v[1])) << 16),
                uint32_t(from_f32<uint16_t, BF16>(v[2])) | (uint32_t(from_f32<uint16_t, BF16>(v[3])) << 16),
                uint32_t(from_f32<uint16_t, BF16>(v[4])) | (uint32_t(from_f32<uint16_t, BF16>(v[5])) << 16),
                uint32_t(from_f32<uint16_t, BF16>(v[6])) | (uint32_t(from_f32<uint16_t, BF16>(v[7])) << 16)};
            __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(out + idx));
          }
        } else {
          for (int t = 0; t < 8 && col + t < N; ++t) {
            const float x = v[t];
            if (ep_k == kEpiStore) {
              out[idx + t] = from_f32<uint16_t, BF16>(x);
            } else if (ep_k == kEpiAccFirst) {
              accbuf[idx + t] = x;
            } else if (ep_k == kEpiAccMid) {
              accbuf[idx + t] = accbuf[idx + t] + x;
            } else {
              out[idx + t] = from_f32<uint16_t, BF16>(accbuf[idx + t] + x);
            }
          }
        }
      }
    }
  };
  const bool whole = vec && m0 + kBM <= M && n0 + kBN <= N;
  if (whole && epi == kEpiAccFirst) pass(std::integral_constant<int, kEpiAccFirst>{}, std::true_type{});
  else if (whole && epi == kEpiStore) pass(std::integral_constant<int, kEpiStore>{}, std::true_type{});
  else pass(std::integral_constant<int, -1>{}, std::false_type{});
}

template <class T, bool BF16>
hipError_t launch_lds(const GemmParams& p, hipStream_t s) {
  const int64_t tiles = ((p.M + kBM - 1) / kBM) * ((p.N + T::BN - 1) / T::BN) * p.batch;
  const dim3 grid{unsigned(tiles), 1u, 1u};
  if (p.a_mode == kADense) {
    if constexpr (T::KB == 64) return hipErrorInvalidValue;  // the wide form gathers only
    else hipLaunchKernelGGL((gemm_lds_kernel<T, BF16, false>), grid, dim3(kThreads), 0, s, p);
  } else if (p.kd > 0)  // native 3D gather
    hipLaunchKernelGGL((gemm_lds_kernel<T, BF16, true, true>), grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL((gemm_lds_kernel<T, BF16, true>), grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

template <class T>
hipError_t launch_tile(const GemmParams& p, hipStream_t s) {
  return p.dtype == CNHWC_BF16 ? launch_lds<T, true>(p, s) : launch_lds<T, false>(p, s);
}

}  // namespace

bool gemm_lds_ok(const GemmParams& p) {
  if (p.dtype == CNHWC_F32 || p.K <= 0) return false;
  if (p.config != kCfgH_256x256 && p.config != kCfgH_256x128L) return false;
  const int64_t bn = p.config == kCfgH_256x256 ? 256 : 128;
  if (((p.M + kBM - 1) / kBM) * ((p.N + bn - 1) / bn) * p.batch >= (int64_t(1) << 31)) return false;
  if (p.K % 8 != 0 || p.ldb % 8 != 0) return false;
  if (p.a_seg_len < 0 || p.a_seg_len % 32 != 0) return false;  // a chunk never straddles segments
  if (p.a_kstep % 8 != 0 || p.b_kstep % 8 != 0) return false;  // 16-byte pieces stay aligned
  if (p.a_mode == kADense) return p.lda % 8 == 0 && p.a_seg_jump % 8 == 0;
  if (p.a_seg_len != 0 || p.a_kstep != 0 || p.b_kstep != 0) return false;
  return p.c % 32 == 0;  // a chunk never straddles two taps
}

namespace {
// The 256 x 256 tile takes 64-element chunks for the implicit gather when a
// chunk never straddles two taps (C % 64 == 0): measured 3-5% faster on the
// large implicit GEMMs, with the same bits.  Dense A (unfold rows, Winograd
// operands) keeps 32-element chunks, where the wide form measured 2-9% slower.
bool wide_chunks_ok(const GemmParams& p) {
  return p.config == kCfgH_256x256 && p.a_mode != kADense && p.c % 64 == 0;
}
}  // namespace

int gemm_lds_launch(const GemmParams& p, void* stream) {
  if (!gemm_lds_ok(p)) return hipErrorInvalidValue;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.config == kCfgH_256x128L) return launch_tile<Tile128>(p, s);
  return wide_chunks_ok(p) ? launch_tile<Tile256W>(p, s) : launch_tile<Tile256>(p, s);
}

}  // namespace cnhwc
