// MFMA GEMM core for gfx950: C[M x N] = A[M x K] * B[N x K]^T, fp32 accumulate.
//
// Used for the three dense contractions of the conv forward path:
//  - Winograd's batched GEMMs over the 64 tile positions (MLX PR "Bound
//    winograd conv2d working set by tiling the batch", Problem: the Winograd
//    path's two GEMM workspaces), A = transformed input V_p [rows x C],
//    B = transformed filter U_p [O x C];
//  - the implicit-GEMM conv, A gathered on the fly from the NHWC input
//    (same page, Fix: the scratch-free fallback), k = (kh*KW + kw)*C + c;
//  - the dense GEMM after an explicit unfold (MLX PR "Use the explicit gemm for
//    wide convs on neural accelerators", intro), A = unfold buffer.
// B rows are weight rows [O][KH][KW][C] (or strided depth slices of
// [O][KD][KH][KW][C] for the 3D decomposition of MLX PR "Decompose small
// kernel-depth 3D convs into 2D convs", Change): already K-contiguous.
//
// Design: 256 threads (4 wavefronts of 64), a BM x BN workgroup tile, BK-deep
// K chunks staged through double-buffered LDS (16-byte global loads along K,
// padded LDS rows so the 16-byte fragment reads are bank-conflict free), next
// chunk prefetched into registers while the matrix cores work on the current
// one.  fp32 uses v_mfma_f32_32x32x2f32 and fp16/bf16 v_mfma_f32_32x32x16_*.
// The K order of every output element is fixed by the configuration alone, so
// results never depend on M, on the launch a row is in, or on the grid.
#include <hip/hip_runtime.h>

#include "internal.hpp"
#include "device_common.hpp"

namespace cnhwc {
namespace {

template <int BM_, int BN_, int BK_, int WM_, int WN_, bool HALF_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_;
  static constexpr bool HALF = HALF_;
};

// A-operand gather modes (kernel template argument).
constexpr int kLoadDense = 0;     // dense rows, 16-byte vectors
constexpr int kLoadImplicit = 1;  // NHWC gather, 16-byte vectors (C % VE == 0)
constexpr int kLoadScalar = 2;    // NHWC gather element by element (any C), scalar B
constexpr int kLoadDenseScalar = 3;  // dense rows element by element, scalar B

template <class Cfg, int LOAD, bool BF16>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmParams p) {
  using E = typename std::conditional<Cfg::HALF, uint16_t, float>::type;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WM = Cfg::WM, WN = Cfg::WN;
  constexpr int VE = 16 / sizeof(E);          // elements per 16-byte vector
  constexpr int KV = BK / VE;                 // vectors per tile row
  constexpr int LDSK = BK + VE;               // padded LDS row (elements)
  constexpr int ROW_STEP = 256 / KV;          // rows covered by one pass of 256 threads
  constexpr int A_VEC = BM / ROW_STEP;
  constexpr int B_VEC = BN / ROW_STEP;
  constexpr int WAVES_N = BN / WN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(BM % ROW_STEP == 0 && BN % ROW_STEP == 0, "tile rows");
  static_assert((BM / WM) * (BN / WN) == 4, "four wavefronts");

  __shared__ __attribute__((aligned(16))) E lds_a[2][BM * LDSK];
  __shared__ __attribute__((aligned(16))) E lds_b[2][BN * LDSK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t m0 = int64_t(blockIdx.x) * BM;
  const int64_t n0 = int64_t(blockIdx.y) * BN;
  const int64_t bz = blockIdx.z;

  const E* __restrict__ A = reinterpret_cast<const E*>(p.a) + bz * p.stride_a;
  const E* __restrict__ B = reinterpret_cast<const E*>(p.b) + bz * p.stride_b;
  const int64_t M = p.M, N = p.N, K = p.K;

  const int kv = tid % KV;
  const int row0 = tid / KV;

  // ---- per-thread A-row state (rows are fixed for the whole K loop)
  int64_t a_base[A_VEC];   // dense: row offset; implicit: image offset of pixel (n, 0, 0)
  int32_t a_ih0[A_VEC], a_iw0[A_VEC];
#pragma unroll
  for (int j = 0; j < A_VEC; ++j) {
    const int64_t m = m0 + row0 + j * ROW_STEP;
    if (LOAD == kLoadDense || LOAD == kLoadDenseScalar) {
      a_base[j] = m < M ? m * p.lda : -1;
      a_ih0[j] = a_iw0[j] = 0;
    } else {
      if (m < M) {
        const int64_t hw = p.oh * p.ow;
        const int64_t n = m / hw;
        const int64_t r = m - n * hw;
        const int64_t oh = r / p.ow;
        const int64_t ow = r - oh * p.ow;
        a_base[j] = n * p.h * p.w * p.c;
        a_ih0[j] = int32_t(oh * p.sh - p.ph);
        a_iw0[j] = int32_t(ow * p.sw - p.pw);
      } else {
        a_base[j] = 0;
        a_ih0[j] = -0x40000000;  // every tap out of range -> zeros
        a_iw0[j] = -0x40000000;
      }
    }
  }
  // ---- K-position state of this thread's vector slot (implicit, vector path)
  int32_t k_c = 0, k_kh = 0, k_kw = 0;
  if (LOAD == kLoadImplicit) {
    const int64_t k0 = int64_t(kv) * VE;
    const int64_t tap = k0 / p.c;
    k_c = int32_t(k0 - tap * p.c);
    k_kh = int32_t(tap / p.kw);
    k_kw = int32_t(tap - int64_t(k_kh) * p.kw);
  }

  uint4 ra[A_VEC], rb[B_VEC];

  auto load_chunk = [&](int64_t kbase) {
    const int64_t kk = kbase + int64_t(kv) * VE;
    // A
#pragma unroll
    for (int j = 0; j < A_VEC; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (LOAD == kLoadDense) {
        if (a_base[j] >= 0 && kk < K) v = *reinterpret_cast<const uint4*>(A + a_base[j] + kk);
      } else if (LOAD == kLoadImplicit) {
        const int32_t ih = a_ih0[j] + k_kh * p.dh;
        const int32_t iw = a_iw0[j] + k_kw * p.dw;
        if (k_kh < p.kh && uint32_t(ih) < uint32_t(p.h) && uint32_t(iw) < uint32_t(p.w))
          v = *reinterpret_cast<const uint4*>(A + a_base[j] + (int64_t(ih) * p.w + iw) * p.c + k_c);
      } else if (LOAD == kLoadDenseScalar) {
        E e[VE];
#pragma unroll
        for (int t = 0; t < VE; ++t)
          e[t] = (a_base[j] >= 0 && kk + t < K) ? A[a_base[j] + kk + t] : E(0);
        v = *reinterpret_cast<const uint4*>(e);
      } else {
        E e[VE];
#pragma unroll
        for (int t = 0; t < VE; ++t) {
          e[t] = E(0);
          const int64_t k = kk + t;
          if (k < K) {
            const int64_t tap = k / p.c;
            const int64_t c = k - tap * p.c;
            const int64_t kh = tap / p.kw;
            const int64_t kw = tap - kh * p.kw;
            const int64_t ih = a_ih0[j] + kh * p.dh;
            const int64_t iw = a_iw0[j] + kw * p.dw;
            if (ih >= 0 && ih < p.h && iw >= 0 && iw < p.w)
              e[t] = A[a_base[j] + (ih * p.w + iw) * p.c + c];
          }
        }
        v = *reinterpret_cast<const uint4*>(e);
      }
      ra[j] = v;
    }
    // B
#pragma unroll
    for (int j = 0; j < B_VEC; ++j) {
      const int64_t n = n0 + row0 + j * ROW_STEP;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (LOAD == kLoadDense || LOAD == kLoadImplicit) {
        if (n < N && kk < K) v = *reinterpret_cast<const uint4*>(B + n * p.ldb + kk);
      } else {
        E e[VE];
#pragma unroll
        for (int t = 0; t < VE; ++t) e[t] = (n < N && kk + t < K) ? B[n * p.ldb + kk + t] : E(0);
        v = *reinterpret_cast<const uint4*>(e);
      }
      rb[j] = v;
    }
  };

  auto advance_k = [&]() {
    if (LOAD == kLoadImplicit) {
      k_c += BK;
      while (k_c >= p.c) {
        k_c -= int32_t(p.c);
        if (++k_kw == p.kw) { k_kw = 0; ++k_kh; }
      }
    }
  };

  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int j = 0; j < A_VEC; ++j)
      *reinterpret_cast<uint4*>(&lds_a[buf][(row0 + j * ROW_STEP) * LDSK + kv * VE]) = ra[j];
#pragma unroll
    for (int j = 0; j < B_VEC; ++j)
      *reinterpret_cast<uint4*>(&lds_b[buf][(row0 + j * ROW_STEP) * LDSK + kv * VE]) = rb[j];
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int arow = wm * WM + (lane & 31);
  const int brow = wn * WN + (lane & 31);
  const int khalf = lane >> 5;

  auto compute = [&](int buf) {
    const E* la = lds_a[buf];
    const E* lb = lds_b[buf];
    if constexpr (!Cfg::HALF) {
      // 8 K values per step: lane half h holds k = 4h..4h+3 of the step; MFMA
      // sub-step s pairs k = s (h=0) with k = 4 + s (h=1).
#pragma unroll
      for (int kq = 0; kq < BK / 8; ++kq) {
        v4f af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const v4f*>(la + (arow + i * 32) * LDSK + kq * 8 + khalf * 4);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = *reinterpret_cast<const v4f*>(lb + (brow + j * 32) * LDSK + kq * 8 + khalf * 4);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][s], bf[j][s], acc[i][j], 0, 0, 0);
      }
    } else {
      // 16 K values per MFMA: lane half h holds k = 8h..8h+7.
#pragma unroll
      for (int kq = 0; kq < BK / 16; ++kq) {
        uint4 af[FM], bf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
          af[i] = *reinterpret_cast<const uint4*>(la + (arow + i * 32) * LDSK + kq * 16 + khalf * 8);
#pragma unroll
        for (int j = 0; j < FN; ++j)
          bf[j] = *reinterpret_cast<const uint4*>(lb + (brow + j * 32) * LDSK + kq * 16 + khalf * 8);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = mfma_32x32x16<BF16>(af[i], bf[j], acc[i][j]);
      }
    }
  };

  const int64_t nk = (K + BK - 1) / BK;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int64_t kc = 0; kc < nk; ++kc) {
    const int cur = int(kc & 1);
    const bool more = kc + 1 < nk;
    if (more) {
      advance_k();
      load_chunk((kc + 1) * BK);
    }
    compute(cur);
    if (more) store_chunk(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: D[row][col] of a 32x32 block sits in lane l, register r at
  // row = 8*(r/4) + 4*(l/32) + r%4, col = l%32.
  E* __restrict__ out = reinterpret_cast<E*>(p.out) + bz * p.stride_out;
  float* __restrict__ accbuf = p.acc ? p.acc + bz * p.stride_out : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
        const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
        if (row < M && col < N) {
          const int64_t idx = row * p.ldc + col;
          const float v = acc[i][j][r];
          if (p.epi == kEpiStore) {
            out[idx] = from_f32<E, BF16>(v);
          } else if (p.epi == kEpiAccFirst) {
            accbuf[idx] = v;
          } else if (p.epi == kEpiAccMid) {
            accbuf[idx] = accbuf[idx] + v;
          } else {
            out[idx] = from_f32<E, BF16>(accbuf[idx] + v);
          }
        }
      }
}

template <class Cfg, bool BF16>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  const dim3 grid(unsigned((p.M + Cfg::BM - 1) / Cfg::BM), unsigned((p.N + Cfg::BN - 1) / Cfg::BN),
                  unsigned(p.batch));
  const int es = Cfg::HALF ? 2 : 4;
  const int ve = 16 / es;
  const bool bvec = p.ldb % ve == 0 && p.K % ve == 0;
  if (p.a_mode == kADense) {
    if (bvec && p.lda % ve == 0)
      hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadDense, BF16>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadDenseScalar, BF16>), grid, dim3(256), 0, s, p);
  } else if (p.c % ve == 0 && bvec) {
    hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadImplicit, BF16>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadScalar, BF16>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

int gemm_launch(const GemmParams& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const bool bf = p.dtype == CNHWC_BF16;
  const bool f32cfg = p.config >= kCfgF32_N32 && p.config <= kCfgF32_N128;
  if (f32cfg != (p.dtype == CNHWC_F32)) return hipErrorInvalidValue;
  switch (p.config) {
    case kCfgF32_N32: return launch_cfg<TileCfg<128, 32, 32, 32, 32, false>, false>(p, s);
    case kCfgF32_N64: return launch_cfg<TileCfg<128, 64, 32, 32, 64, false>, false>(p, s);
    case kCfgF32_N96: return launch_cfg<TileCfg<128, 96, 32, 32, 96, false>, false>(p, s);
    case kCfgF32_N128: return launch_cfg<TileCfg<128, 128, 32, 32, 128, false>, false>(p, s);
    case kCfgH_N64:
      return bf ? launch_cfg<TileCfg<128, 64, 64, 32, 64, true>, true>(p, s)
                : launch_cfg<TileCfg<128, 64, 64, 32, 64, true>, false>(p, s);
    case kCfgH_N128:
      return bf ? launch_cfg<TileCfg<128, 128, 64, 64, 64, true>, true>(p, s)
                : launch_cfg<TileCfg<128, 128, 64, 64, 64, true>, false>(p, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cnhwc
