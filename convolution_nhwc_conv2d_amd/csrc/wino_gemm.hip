// Persistent fp32 MFMA kernel for the Winograd tile-position GEMMs
// M_p = V_p * U_p^T (MLX PR "Bound winograd conv2d working set by tiling the
// batch", Problem: the batched GEMMs between the input and output transforms).
//
// These GEMMs have a short K (C, e.g. 192), a narrow N (O, e.g. 96) and a very
// long M (images x tiles, e.g. 295,840 rows per position).  One workgroup of 8
// wavefronts runs per CU and owns a contiguous row range of one position p:
//  - the whole U_p (O x C fp32, at most 96 x 192 = 72 KB) is loaded into LDS
//    once; it is the only shared data, so after that single barrier the
//    wavefronts never synchronise again;
//  - each wavefront owns 32-row blocks (all O columns) and streams its own rows
//    of V_p straight from global memory into MFMA operand registers, 32 K
//    values per chunk, the loads of the chunk two steps ahead in flight while
//    the current one feeds the matrix cores (v_mfma_f32_32x32x2f32);
//  - a finished block's result is stored after the next chunk's loads are
//    issued; a wavefront that waits on its stores is covered by the other
//    wavefront sharing its SIMD.
// MFMA k assignment: in chunk kc, step q (0..3), sub-step s (0..3), lanes of
// half h (0/1) supply k = 32*kc + 16*h + 4*q + s.  Each lane thus reads 64
// contiguous bytes of its row per chunk.  The order depends on C and O only,
// so batch tiling never changes a bit.  K = C must be a multiple of 32 (at most
// 192) so a block's chunks unroll completely and every LDS and global address
// is a per-block base plus an immediate offset.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "wino_f63_api.hpp"
#include "device_common.hpp"

namespace cnhwc {
namespace {

constexpr int kResMaxChunks = 6;   // K up to 192 resident
constexpr int kResThreads = 512;   // 8 wavefronts
constexpr int kResWaves = kResThreads / 64;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gvec_ptr;
__device__ u32x4 g_res_zero16 = {0u, 0u, 0u, 0u};
template <typename T>
__device__ __forceinline__ gvec_ptr gvec(const T* p) {
  return (gvec_ptr)(p);
}

__device__ __forceinline__ int swz(int r, int c) { return (c ^ r ^ (r >> 3)) & 7; }

template <int BN, int NCH>
__global__ __launch_bounds__(kResThreads) void wino_gemm_resident_kernel(
    const float* __restrict__ V, const float* __restrict__ U, float* __restrict__ Mout,
    int64_t rows, int64_t O, int64_t v_plane, int64_t m_plane, int32_t wg_per_p) {
  constexpr int FN = BN / 32;
  constexpr int64_t Cs = 32 * NCH;  // K, a whole number of 32-wide chunks
  __shared__ __attribute__((aligned(16))) float lds_u[NCH * BN * 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p = int(blockIdx.x) / wg_per_p;
  const int part = int(blockIdx.x) - p * wg_per_p;
  const float* __restrict__ A = V + int64_t(p) * v_plane;
  const float* __restrict__ B = U + int64_t(p) * O * Cs;
  float* __restrict__ C = Mout + int64_t(p) * m_plane;
  const gvec_ptr zero = gvec(&g_res_zero16);

  // ---- U_p -> LDS, [chunk][row][32 floats], 16-byte pieces swizzled by row;
  // zeros past O.  Every thread takes part, then the one barrier.
  for (int idx = tid; idx < NCH * BN * 8; idx += kResThreads) {
    const int kc = idx / (BN * 8);
    const int r = (idx >> 3) % BN;
    const int v = idx & 7;
    const gvec_ptr src = r < O ? gvec(B + r * Cs + kc * 32 + v * 4) : zero;
    *reinterpret_cast<u32x4*>(&lds_u[(kc * BN + r) * 32 + swz(r, v) * 4]) = *src;
  }
  __syncthreads();

  // ---- this wavefront's 32-row blocks: the workgroup's share of the blocks of
  // position p, dealt round-robin to its 8 wavefronts
  const int64_t nblk = (rows + 31) / 32;
  const int64_t per = (nblk + wg_per_p - 1) / wg_per_p;
  const int64_t b_begin = part * per;
  const int64_t b_end = b_begin + per < nblk ? b_begin + per : nblk;
  const int64_t first = b_begin + wave;
  if (first >= b_end) return;  // no barrier below: a wavefront may leave early
  const int64_t nmine = (b_end - first + kResWaves - 1) / kResWaves;

  const int i = lane & 31;  // row within the block / column within a 32-column group
  const int h = lane >> 5;  // k half

  // LDS byte offsets of this lane's B pieces (step q, column group j) within a chunk
  int boff[4][FN];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = i + 32 * j;
      boff[q][j] = (r * 32 + swz(r, 4 * h + q) * 4) * 4;
    }
  const char* lu = reinterpret_cast<const char*>(lds_u);

  // Row pointer of a block: rows past the end are clamped to the last row (in
  // bounds; their results are never stored, and rows do not mix in the MFMA).
  auto rowptr = [&](int64_t blk) {
    int64_t m = blk * 32 + i;
    m = m < rows ? m : rows - 1;
    return A + m * Cs + 16 * h;
  };
  // A operand of chunk kc: 4 x 16 bytes at k = 32kc + 16h + 4q
  auto load_a = [&](const float* rp, int kc, u32x4 (&a)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) a[q] = *gvec(rp + kc * 32 + 4 * q);
  };

  v16f acc[FN];
  // one chunk: B fragments from the resident U_p, 4 steps x 4 sub-steps x FN MFMAs;
  // the block's first MFMA per accumulator starts from zero
  auto compute = [&](const u32x4 (&a)[4], int kc, bool first_chunk) {
    const char* base = lu + kc * BN * 128;
    u32x4 b0[FN], b1[FN];
    auto read_b = [&](int q, u32x4 (&b)[FN]) {
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = *reinterpret_cast<const u32x4*>(base + boff[q][j]);
    };
    auto mma = [&](const u32x4& av, const u32x4 (&b)[FN], bool zero_start) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const v16f cin = (zero_start && s == 0) ? v16f{} : acc[j];
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(v4f, av)[s],
                                                        __builtin_bit_cast(v4f, b[j])[s], cin, 0, 0, 0);
        }
    };
    read_b(0, b0);
    read_b(1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[0], b0, first_chunk);
    __builtin_amdgcn_sched_barrier(0);
    read_b(2, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[1], b1, false);
    __builtin_amdgcn_sched_barrier(0);
    read_b(3, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[2], b0, false);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[3], b1, false);
  };

  // D[row][col] of a 32x32 block: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32
  // A whole block (all 32 rows, O == BN) stores without per-element tests:
  // 48 plain stores instead of 48 branches around them (about 3% of the
  // kernel at 40 x 512 x 512, 192 -> 96).  Only a position's last block can
  // be partial.
  auto store_block = [&](int64_t blk) {
    float* cp = C + (blk * 32 + h * 4) * O + i;
    const bool full = blk * 32 + 32 <= rows;
    if (full && O == BN) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = (r >> 2) * 8 + (r & 3);
          __builtin_nontemporal_store(acc[j][r], &cp[rr * O + 32 * j]);  // streamed: read once, later
        }
      return;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = (r >> 2) * 8 + (r & 3);
        if (32 * j + i < O && (full || blk * 32 + h * 4 + rr < rows))
          __builtin_nontemporal_store(acc[j][r], &cp[rr * O + 32 * j]);
      }
  };

  // Blocks in order.  Three operand sets: chunk c of a block lives in set
  // (c + PAR) % 3, and the loads of the chunk two steps ahead (possibly in the
  // next block) are issued before each chunk's MFMAs.  Those loads are
  // unconditional: past the wavefront's last block they re-read rows it
  // already holds (rpn and rpn2 fall back to valid rows), so the number of
  // loads in flight is the same on every path and each chunk's wait leaves
  // the later chunks' loads outstanding (a load skipped on one path would
  // make the compiler wait for all of them before the block's last chunk).
  u32x4 a0[4], a1[4], a2[4];
  auto set = [&](int k) -> u32x4 (&)[4] { return k == 0 ? a0 : (k == 1 ? a1 : a2); };
  int64_t b = 0;
  const float* rp = rowptr(first);
  const float* rpn = nmine > 1 ? rowptr(first + kResWaves) : rp;
  load_a(rp, 0, a0);
  if (NCH > 1) load_a(rp, 1, a1);
  else if (nmine > 1) load_a(rpn, 0, a1);
  auto block = [&](auto par_tag) {
    constexpr int PAR = decltype(par_tag)::value;
    const int64_t blk = first + b * kResWaves;
    const bool has_next = b + 1 < nmine;
    const bool has_next2 = b + 2 < nmine;
    const float* rpn2 = has_next2 ? rowptr(blk + 2 * kResWaves) : rpn;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      // chunk c + 2 of this block, or chunk c + 2 - NCH of the next one(s)
      const int ahead = c + 2;
      if (ahead < NCH) {
        load_a(rp, ahead, set((ahead + PAR) % 3));
      } else if (ahead - NCH < NCH) {
        load_a(rpn, ahead - NCH, set((ahead + PAR) % 3));
      } else {
        load_a(rpn2, ahead - 2 * NCH, set((ahead + PAR) % 3));
      }
      compute(set((c + PAR) % 3), c, c == 0);
    }
    store_block(blk);
    rp = rpn;
    rpn = rpn2;
    ++b;
    return has_next;
  };
  while (true) {
    if (!block(std::integral_constant<int, 0>{})) break;
    if constexpr (NCH % 3 != 0) {
      if (!block(std::integral_constant<int, NCH % 3>{})) break;
      if (!block(std::integral_constant<int, (2 * NCH) % 3>{})) break;
    }
  }
}

}  // namespace

bool wino_gemm_resident_ok(int64_t cs, int64_t o) {
  return cs % 32 == 0 && cs <= kResMaxChunks * 32 && o <= 96;
}

int wino_gemm_resident_launch(const float* v, const float* u, float* m, int64_t rows, int64_t o,
                              int64_t cs, int64_t v_plane, int64_t m_plane, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (rows <= 0) return hipSuccess;
  if (!wino_gemm_resident_ok(cs, o)) return hipErrorInvalidValue;
  // one workgroup per CU: 256 workgroups over the 64 tile positions
  const int wg_per_p = 4;
  const dim3 grid(unsigned(kWinoP * wg_per_p));
  const int nch = int(cs / 32);
  const int bn = o <= 32 ? 32 : (o <= 64 ? 64 : 96);
#define CNHWC_RES_LAUNCH(BN_, NCH_)                                                          \
  if (bn == BN_ && nch == NCH_)                                                              \
    hipLaunchKernelGGL((wino_gemm_resident_kernel<BN_, NCH_>), grid, dim3(kResThreads), 0, s, v, u, \
                       m, rows, o, v_plane, m_plane, wg_per_p);
  CNHWC_RES_LAUNCH(32, 1) CNHWC_RES_LAUNCH(32, 2) CNHWC_RES_LAUNCH(32, 3)
  CNHWC_RES_LAUNCH(32, 4) CNHWC_RES_LAUNCH(32, 5) CNHWC_RES_LAUNCH(32, 6)
  CNHWC_RES_LAUNCH(64, 1) CNHWC_RES_LAUNCH(64, 2) CNHWC_RES_LAUNCH(64, 3)
  CNHWC_RES_LAUNCH(64, 4) CNHWC_RES_LAUNCH(64, 5) CNHWC_RES_LAUNCH(64, 6)
  CNHWC_RES_LAUNCH(96, 1) CNHWC_RES_LAUNCH(96, 2) CNHWC_RES_LAUNCH(96, 3)
  CNHWC_RES_LAUNCH(96, 4) CNHWC_RES_LAUNCH(96, 5) CNHWC_RES_LAUNCH(96, 6)
#undef CNHWC_RES_LAUNCH
  return hipGetLastError();
}

}  // namespace cnhwc
