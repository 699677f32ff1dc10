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
//    values per chunk, the next chunk's loads in flight while the current one
//    feeds the matrix cores (v_mfma_f32_32x32x2f32);
//  - a finished block's result is stored after the next chunk's loads are
//    issued; a wavefront that waits on its stores is covered by the other
//    wavefront sharing its SIMD.
// MFMA k assignment: in chunk kc, step q (0..3), sub-step s (0..3), lanes of
// half h (0/1) supply k = 32*kc + 16*h + 4*q + s.  Each lane thus reads 64
// contiguous bytes of its row per chunk.  The order depends on C and O only,
// so batch tiling never changes a bit.
#include <hip/hip_runtime.h>

#include "internal.hpp"
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

template <int BN>
__global__ __launch_bounds__(kResThreads) void wino_gemm_resident_kernel(
    const float* __restrict__ V, const float* __restrict__ U, float* __restrict__ Mout,
    int64_t rows, int64_t O, int64_t Cs, int64_t v_plane, int64_t m_plane, int32_t wg_per_p) {
  constexpr int FN = BN / 32;
  __shared__ __attribute__((aligned(16))) float lds_u[kResMaxChunks * BN * 32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int p = int(blockIdx.x) / wg_per_p;
  const int part = int(blockIdx.x) - p * wg_per_p;
  const int nch = int((Cs + 31) / 32);
  const float* __restrict__ A = V + int64_t(p) * v_plane;
  const float* __restrict__ B = U + int64_t(p) * O * Cs;
  float* __restrict__ C = Mout + int64_t(p) * m_plane;
  const gvec_ptr zero = gvec(&g_res_zero16);

  // ---- U_p -> LDS, [chunk][row][32 floats], 16-byte pieces swizzled by row;
  // zeros past O or C.  Every thread takes part, then the one barrier.
  for (int idx = tid; idx < nch * BN * 8; idx += kResThreads) {
    const int kc = idx / (BN * 8);
    const int r = (idx >> 3) % BN;
    const int v = idx & 7;
    const int64_t k = int64_t(kc) * 32 + v * 4;
    const gvec_ptr src = (r < O && k < Cs) ? gvec(B + r * Cs + k) : zero;
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

  // A operand of one chunk: 4 x 16 bytes of row (blk*32 + i), k = 32kc + 16h + 4q
  auto load_a = [&](int64_t blk, int kc, u32x4 (&a)[4]) {
    const int64_t m = blk * 32 + i;
    const int64_t k0 = int64_t(kc) * 32 + h * 16;
    const float* row = A + m * Cs;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = k0 + 4 * q;
      const gvec_ptr src = (m < rows && k < Cs) ? gvec(row + k) : zero;
      a[q] = *src;
    }
  };

  v16f acc[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

  // one chunk: B fragments from the resident U_p, 4 steps x 4 sub-steps x FN MFMAs
  auto compute = [&](const u32x4 (&a)[4], int kc) {
    const float* lu = lds_u + kc * BN * 32;
    u32x4 b0[FN], b1[FN];
    auto read_b = [&](int q, u32x4 (&b)[FN]) {
      const int cl = 4 * h + q;  // logical 16-byte piece of the 128-byte row slice
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = i + 32 * j;
        b[j] = *reinterpret_cast<const u32x4*>(lu + r * 32 + swz(r, cl) * 4);
      }
    };
    auto mma = [&](const u32x4& av, const u32x4 (&b)[FN]) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(v4f, av)[s],
                                                        __builtin_bit_cast(v4f, b[j])[s], acc[j], 0,
                                                        0, 0);
    };
    read_b(0, b0);
    read_b(1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[0], b0);
    __builtin_amdgcn_sched_barrier(0);
    read_b(2, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[1], b1);
    __builtin_amdgcn_sched_barrier(0);
    read_b(3, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[2], b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(a[3], b1);
  };

  // D[row][col] of a 32x32 block: lane l, register r -> row 8*(r/4) + 4*(l/32) + r%4, col l%32
  auto store_block = [&](const v16f (&res)[FN], int64_t blk) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = blk * 32 + (r >> 2) * 8 + h * 4 + (r & 3);
        const int64_t col = j * 32 + i;
        if (row < rows && col < O) C[row * O + col] = res[j][r];
      }
  };

  // (blk, kc): the chunk being computed; (lblk, lkc): the next chunk to load.
  // Unrolled by two so the two operand register sets stay static.
  int64_t blk = first, lblk = first, left = nmine;  // `left`: blocks not yet finished
  int kc = 0, lkc = 0;
  auto step = [&](const u32x4 (&cur)[4], u32x4 (&nxt)[4]) -> bool {
    if (++lkc == nch) {
      lkc = 0;
      lblk += kResWaves;
    }
    const bool more = !(left == 1 && kc == nch - 1);
    if (more) load_a(lblk, lkc, nxt);
    compute(cur, kc);
    if (kc == nch - 1) {
      store_block(acc, blk);
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
      --left;
      blk += kResWaves;
      kc = 0;
    } else {
      ++kc;
    }
    return more;
  };

  u32x4 a0[4], a1[4];
  load_a(lblk, lkc, a0);
  while (step(a0, a1) && step(a1, a0)) {
  }
}

}  // namespace

bool wino_gemm_resident_ok(int64_t cs, int64_t o) {
  return cs <= kResMaxChunks * 32 && o <= 96;
}

int wino_gemm_resident_launch(const float* v, const float* u, float* m, int64_t rows, int64_t o,
                              int64_t cs, int64_t v_plane, int64_t m_plane, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (rows <= 0) return hipSuccess;
  if (!wino_gemm_resident_ok(cs, o)) return hipErrorInvalidValue;
  // one workgroup per CU: 256 workgroups over the 64 tile positions
  const int wg_per_p = 4;
  const dim3 grid(unsigned(kWinoP * wg_per_p));
  if (o <= 32)
    hipLaunchKernelGGL((wino_gemm_resident_kernel<32>), grid, dim3(kResThreads), 0, s, v, u, m, rows,
                       o, cs, v_plane, m_plane, wg_per_p);
  else if (o <= 64)
    hipLaunchKernelGGL((wino_gemm_resident_kernel<64>), grid, dim3(kResThreads), 0, s, v, u, m, rows,
                       o, cs, v_plane, m_plane, wg_per_p);
  else
    hipLaunchKernelGGL((wino_gemm_resident_kernel<96>), grid, dim3(kResThreads), 0, s, v, u, m, rows,
                       o, cs, v_plane, m_plane, wg_per_p);
  return hipGetLastError();
}

}  // namespace cnhwc
