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
// Design: one wavefront per WM x WN sub-tile (4 or 8 per workgroup) of a BM x
// BN output tile.  K is
// consumed in chunks of 128 bytes per row (32 fp32 or 64 fp16/bf16).  Each
// chunk travels global -> registers (16-byte loads along K) -> LDS -> MFMA
// fragments.  Two register staging sets keep the loads of chunk k+2 in flight
// while the matrix cores consume chunk k, so global latency is covered by two
// chunks of MFMA work; LDS is double buffered with one barrier per chunk.
// LDS rows are 128 bytes with the 16-byte chunk index XOR-swizzled by the row,
// so both the staging stores and the fragment reads are bank-conflict free
// without padding.  fp32 uses v_mfma_f32_32x32x2f32 (a 16-byte LDS read feeds
// four of them), fp16/bf16 v_mfma_f32_32x32x16_*.  The K order of every output
// element is fixed by the configuration alone, so results never depend on M,
// on the launch a row is in, or on the grid.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "internal.hpp"
#include "device_common.hpp"

namespace cnhwc {
namespace {

template <int BM_, int BN_, int WM_, int WN_, bool HALF_, int NSETS_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr int NT = 64 * (BM_ / WM_) * (BN_ / WN_);  // threads: one wavefront per WM x WN
  static constexpr bool HALF = HALF_;
  static constexpr int BK = HALF_ ? 64 : 32;  // 128 bytes of K per row
  static constexpr int NSETS = NSETS_;        // register staging sets (prefetch depth)
};

// A-operand gather modes (kernel template argument).
constexpr int kLoadDense = 0;        // dense rows, 16-byte vectors
constexpr int kLoadImplicit = 1;     // NHWC gather, 16-byte vectors (C % VE == 0)
constexpr int kLoadScalar = 2;       // NHWC gather element by element (any C), scalar B
constexpr int kLoadDenseScalar = 3;  // dense rows element by element, scalar B

// 16 zero bytes: masked lanes load from here, so the operand loads need no
// branches (padding taps, rows past M, K past the end).
// Global-address-space pointers keep the loads global_load (a generic pointer
// would turn them into flat loads, which also count against the LDS counter).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ u32x4 g_zero16 = {0u, 0u, 0u, 0u};
typedef const u32x4 __attribute__((address_space(1)))* gvec_ptr;
template <typename T>
__device__ __forceinline__ gvec_ptr gvec(const T* p) {
  return (gvec_ptr)(p);
}

// Physical 16-byte chunk of logical chunk c in LDS row r (8 chunks per row).
__device__ __forceinline__ int swz(int r, int c) { return (c ^ r ^ (r >> 3)) & 7; }

template <int NA, int NB>
struct Stage {
  u32x4 a[NA];
  u32x4 b[NB];
};

// D3: the implicit A operand is a 3D NDHWC gather (depth window as well).
template <class Cfg, int LOAD, bool BF16, bool D3 = false>
__global__ __launch_bounds__(Cfg::NT) void gemm_kernel(const GemmParams p) {
  using E = typename std::conditional<Cfg::HALF, uint16_t, float>::type;
  constexpr int BM = Cfg::BM, BN = Cfg::BN, BK = Cfg::BK, WM = Cfg::WM, WN = Cfg::WN;
  constexpr int VE = 16 / sizeof(E);  // elements per 16-byte chunk
  constexpr int ROWE = BK;            // elements per LDS row (128 bytes)
  constexpr int NT = Cfg::NT;
  constexpr int RP = NT / 8;          // rows per pass: 8 threads per 128-byte row
  constexpr int A_VEC = BM / RP;
  constexpr int B_VEC = BN / RP;
  constexpr int WAVES_N = BN / WN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(BK * sizeof(E) == 128, "128-byte rows");
  static_assert(BM % RP == 0 && BN % RP == 0, "tile rows");

  __shared__ __attribute__((aligned(16))) E lds_a[2][BM * ROWE];
  __shared__ __attribute__((aligned(16))) E lds_b[2][BN * ROWE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int64_t m0 = int64_t(blockIdx.x) * BM;
  const int64_t n0 = int64_t(blockIdx.y) * BN;
  // blockIdx.z: batch index, or the K split (then the batch is 1)
  const bool split = p.ksplit > 1;
  const int64_t bz = split ? 0 : blockIdx.z;
  const int64_t kstart = split ? int64_t(blockIdx.z) * p.kchunk : 0;

  const E* __restrict__ A = reinterpret_cast<const E*>(p.a) + bz * p.stride_a;
  const E* __restrict__ B = reinterpret_cast<const E*>(p.b) + bz * p.stride_b;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t kend = split && kstart + p.kchunk < K ? kstart + p.kchunk : K;

  const int kv = tid & 7;   // this thread's 16-byte chunk within a row
  const int row0 = tid >> 3;

  // ---- per-thread A-row state (rows are fixed for the whole K loop)
  // dense: a_off = row offset, -1 past M.  implicit: a_off = element offset of
  // the row's window origin (oh*sh - ph, ow*sw - pw) in image n (may be
  // negative: only used once the tap is known to be inside the image).
  int64_t a_off[A_VEC];
  int32_t a_ih0[A_VEC], a_iw0[A_VEC], a_id0[A_VEC];
#pragma unroll
  for (int j = 0; j < A_VEC; ++j) {
    const int64_t m = m0 + row0 + j * RP;
    a_id0[j] = 0;
    if (LOAD == kLoadDense || LOAD == kLoadDenseScalar) {
      a_off[j] = m < M ? m * p.lda : -1;
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
                 ((int64_t(a_id0[j]) * p.h + a_ih0[j]) * p.w + a_iw0[j]) * p.c;
    } else {
      a_off[j] = 0;
      a_ih0[j] = -0x40000000;  // every tap out of range -> zeros
      a_iw0[j] = -0x40000000;
      a_id0[j] = -0x40000000;
    }
  }
  // B rows
  int64_t b_off[B_VEC];
#pragma unroll
  for (int j = 0; j < B_VEC; ++j) {
    const int64_t n = n0 + row0 + j * RP;
    b_off[j] = n < N ? n * p.ldb : -1;
  }
  // ---- K position of the next chunk to load (implicit vector path)
  // (3D: the tap is (k_kd, k_kh, k_kw); past the end k_kd >= KD, 2D: k_kh >= KH)
  int32_t k_c = 0, k_kh = 0, k_kw = 0, k_kd = 0;
  if (LOAD == kLoadImplicit) {
    const int64_t k0 = kstart + int64_t(kv) * VE;
    const int64_t tap = k0 / p.c;
    k_c = int32_t(k0 - tap * p.c);
    const int64_t t2 = tap / p.kw;
    k_kw = int32_t(tap - t2 * p.kw);
    if constexpr (D3) {
      k_kd = int32_t(t2 / p.kh);
      k_kh = int32_t(t2 - int64_t(k_kd) * p.kh);
    } else {
      k_kh = int32_t(t2);
    }
  }
  auto advance_k = [&]() {
    if (LOAD == kLoadImplicit) {
      k_c += BK;
      while (k_c >= p.c) {
        k_c -= int32_t(p.c);
        if (++k_kw == p.kw) {
          k_kw = 0;
          ++k_kh;
          if (D3 && k_kh == p.kh) {
            k_kh = 0;
            ++k_kd;
          }
        }
      }
    }
  };

  const gvec_ptr zero = gvec(&g_zero16);
  using St = Stage<A_VEC, B_VEC>;
  auto load_chunk = [&](int64_t kbase, St& st) {
    const int64_t kk = kbase + int64_t(kv) * VE;
    const bool k_in = kk < K;
    if constexpr (LOAD == kLoadDense) {
#pragma unroll
      for (int j = 0; j < A_VEC; ++j) {
        const gvec_ptr ptr = (a_off[j] >= 0 && k_in) ? gvec(A + a_off[j] + kk) : zero;
        st.a[j] = *ptr;
      }
    } else if constexpr (LOAD == kLoadImplicit) {
      // one tap for the whole chunk slot: shared offset, per-row bounds
      const int32_t dhh = k_kh * p.dh, dww = k_kw * p.dw, ddd = D3 ? k_kd * p.dd : 0;
      const int64_t tap_off = ((int64_t(ddd) * p.h + dhh) * p.w + dww) * p.c + k_c;
      const bool tap_in = D3 ? k_kd < p.kd : k_kh < p.kh;
#pragma unroll
      for (int j = 0; j < A_VEC; ++j) {
        const bool ok = tap_in && uint32_t(a_ih0[j] + dhh) < uint32_t(p.h) &&
                        uint32_t(a_iw0[j] + dww) < uint32_t(p.w) &&
                        (!D3 || uint32_t(a_id0[j] + ddd) < uint32_t(p.d));
        const gvec_ptr ptr = ok ? gvec(A + a_off[j] + tap_off) : zero;
        st.a[j] = *ptr;
      }
    } else {
#pragma unroll
      for (int j = 0; j < A_VEC; ++j) {
        E e[VE];
        if (LOAD == kLoadDenseScalar) {
#pragma unroll
          for (int t = 0; t < VE; ++t)
            e[t] = (a_off[j] >= 0 && kk + t < K) ? A[a_off[j] + kk + t] : E(0);
        } else {
          // the vector's first (kd, kh, kw, c) from one division chain, the rest walked
          const int64_t tap0 = kk / p.c;
          const int64_t t2 = tap0 / p.kw;
          int64_t c = kk - tap0 * p.c;
          int64_t kw = tap0 - t2 * p.kw;
          int64_t kd = D3 ? t2 / p.kh : 0;
          int64_t kh = t2 - kd * p.kh;
#pragma unroll
          for (int t = 0; t < VE; ++t) {
            e[t] = E(0);
            if (kk + t < K) {
              const int64_t dd_ = kd * p.dd, dh_ = kh * p.dh, dw_ = kw * p.dw;
              const int64_t id = a_id0[j] + dd_;
              const int64_t ih = a_ih0[j] + dh_;
              const int64_t iw = a_iw0[j] + dw_;
              if ((!D3 || (id >= 0 && id < p.d)) && ih >= 0 && ih < p.h && iw >= 0 && iw < p.w)
                e[t] = A[a_off[j] + ((dd_ * p.h + dh_) * p.w + dw_) * p.c + c];
            }
            if (++c == p.c) {
              c = 0;
              if (++kw == p.kw) {
                kw = 0;
                if (++kh == p.kh) {
                  kh = 0;
                  ++kd;
                }
              }
            }
          }
        }
        st.a[j] = *reinterpret_cast<const u32x4*>(e);
      }
    }
    if constexpr (LOAD == kLoadDense || LOAD == kLoadImplicit) {
#pragma unroll
      for (int j = 0; j < B_VEC; ++j) {
        const gvec_ptr ptr = (b_off[j] >= 0 && k_in) ? gvec(B + b_off[j] + kk) : zero;
        st.b[j] = *ptr;
      }
    } else {
#pragma unroll
      for (int j = 0; j < B_VEC; ++j) {
        E e[VE];
#pragma unroll
        for (int t = 0; t < VE; ++t) e[t] = (b_off[j] >= 0 && kk + t < K) ? B[b_off[j] + kk + t] : E(0);
        st.b[j] = *reinterpret_cast<const u32x4*>(e);
      }
    }
  };

  auto store_chunk = [&](int buf, const St& st) {
#pragma unroll
    for (int j = 0; j < A_VEC; ++j) {
      const int r = row0 + j * RP;
      *reinterpret_cast<u32x4*>(&lds_a[buf][r * ROWE + swz(r, kv) * VE]) = st.a[j];
    }
#pragma unroll
    for (int j = 0; j < B_VEC; ++j) {
      const int r = row0 + j * RP;
      *reinterpret_cast<u32x4*>(&lds_b[buf][r * ROWE + swz(r, kv) * VE]) = st.b[j];
    }
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

  // One K chunk = 4 fragment steps; step kq reads logical 16-byte chunk
  // 2*kq + khalf of the lane's A and B rows.  Fragments are software
  // pipelined: step kq+1's LDS reads are issued before step kq's MFMAs (two
  // fragment register sets; the scheduling barriers keep the compiler from
  // sinking the reads next to their first use).
  struct Frags {
    uint4 a[FM];
    uint4 b[FN];
  };
  auto read_frags = [&](const E* la, const E* lb, int kq, Frags& f) {
    const int cl = 2 * kq + khalf;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = arow + i * 32;
      f.a[i] = *reinterpret_cast<const uint4*>(la + r * ROWE + swz(r, cl) * VE);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = brow + j * 32;
      f.b[j] = *reinterpret_cast<const uint4*>(lb + r * ROWE + swz(r, cl) * VE);
    }
  };
  auto mma = [&](const Frags& f) {
    if constexpr (!Cfg::HALF) {
      // lane half h holds k = 8kq + 4h + s; sub-step s pairs k = 8kq + s with 8kq + 4 + s
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(__builtin_bit_cast(v4f, f.a[i])[s],
                                                             __builtin_bit_cast(v4f, f.b[j])[s],
                                                             acc[i][j], 0, 0, 0);
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma_32x32x16<BF16>(f.a[i], f.b[j], acc[i][j]);
    }
  };
  auto compute = [&](int buf) {
    const E* la = lds_a[buf];
    const E* lb = lds_b[buf];
    Frags f0, f1;
    read_frags(la, lb, 0, f0);
    read_frags(la, lb, 1, f1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(la, lb, 2, f0);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    read_frags(la, lb, 3, f1);
    __builtin_amdgcn_sched_barrier(0);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    mma(f1);
  };

  // chunks of this split; kstart and the split length are multiples of BK,
  // so only the last chunk of the whole K can be partial (masked by kk < K)
  const int64_t nk = (kend - kstart + BK - 1) / BK;
  if constexpr (Cfg::NSETS == 1) {
    // ---- main loop, one staging set: chunk k+1 in flight while chunk k computes
    St s0;
    load_chunk(kstart, s0);
    store_chunk(0, s0);
    __syncthreads();
    for (int64_t kc = 0; kc < nk; ++kc) {
      const int cur = int(kc & 1);
      const bool more = kc + 1 < nk;
      if (more) {
        advance_k();
        load_chunk(kstart + (kc + 1) * BK, s0);
      }
      compute(cur);
      if (more) store_chunk(cur ^ 1, s0);
      __syncthreads();
    }
  } else {
  // ---- main loop, two staging sets: chunk k+2 in flight while chunk k computes
  St s0, s1;
  load_chunk(kstart, s0);
  store_chunk(0, s0);
  if (nk > 1) {
    advance_k();
    load_chunk(kstart + BK, s1);
  }
  __syncthreads();
  for (int64_t kc = 0; kc < nk; kc += 2) {
    if (kc + 2 < nk) {
      advance_k();
      load_chunk(kstart + (kc + 2) * BK, s0);
    }
    compute(0);
    if (kc + 1 < nk) store_chunk(1, s1);
    __syncthreads();
    if (kc + 1 >= nk) break;
    if (kc + 3 < nk) {
      advance_k();
      load_chunk(kstart + (kc + 3) * BK, s1);
    }
    compute(1);
    if (kc + 2 < nk) store_chunk(0, s0);
    __syncthreads();
  }
  }

  // ---- epilogue: D[row][col] of a 32x32 block sits in lane l, register r at
  // row = 8*(r/4) + 4*(l/32) + r%4, col = l%32.
  E* __restrict__ out = reinterpret_cast<E*>(p.out) + bz * p.stride_out;
  float* __restrict__ accbuf = p.acc ? p.acc + bz * p.stride_out : nullptr;
  // a K split stores its fp32 partial sums to its own slice (epilogue later)
  float* __restrict__ partbuf = split ? p.part + int64_t(blockIdx.z) * M * p.ldc : nullptr;
  const int epi = split ? -1 : p.epi;
  // EPI: the epilogue kind when fixed at compile time (-2: read epi).  WHOLE:
  // the tile lies inside M x N, so no element needs a bounds test.
  auto store_tile = [&](auto epi_c, auto whole_c) {
    constexpr int EPI = decltype(epi_c)::value;
    constexpr bool WHOLE = decltype(whole_c)::value;
    const int ep_k = EPI > -2 ? EPI : epi;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t row = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
          const int64_t col = n0 + wn * WN + j * 32 + (lane & 31);
          if (WHOLE || (row < M && col < N)) {
            const int64_t idx = row * p.ldc + col;
            const float v = acc[i][j][r];
            if (ep_k < 0) {
              partbuf[idx] = v;
            } else if (ep_k == kEpiStore) {
              out[idx] = from_f32<E, BF16>(v);
            } else if (ep_k == kEpiAccFirst) {
              accbuf[idx] = v;
            } else if (ep_k == kEpiAccMid) {
              accbuf[idx] = accbuf[idx] + v;
            } else {
              out[idx] = from_f32<E, BF16>(accbuf[idx] + v);
            }
          }
        }
  };
  const bool whole = m0 + BM <= M && n0 + BN <= N;
  if (whole && epi < 0) store_tile(std::integral_constant<int, -1>{}, std::true_type{});
  else if (whole && epi == kEpiStore) store_tile(std::integral_constant<int, kEpiStore>{}, std::true_type{});
  else store_tile(std::integral_constant<int, -2>{}, std::false_type{});
}

// y (or the fp32 accumulator) from the K-split partial slices: the slices are
// added in order 0, 1, ..., ksplit-1, then the epilogue of p is applied.  Each
// thread takes V consecutive columns of one row (V = 4: 16-byte slice loads;
// V divides N); NARROW: the thread index fits 32 bits, so the row and column
// come from 32-bit arithmetic.
template <typename E, bool BF16, int V, bool NARROW>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const GemmParams p) {
  using I = typename std::conditional<NARROW, uint32_t, uint64_t>::type;
  const I nv = I(p.N / V);
  const I t = I(blockIdx.x) * 256 + threadIdx.x;
  if (t >= I(p.M) * nv) return;
  const I row = t / nv;
  const int64_t col = int64_t(t - row * nv) * V;
  const int64_t idx = int64_t(row) * p.ldc + col;
  const int64_t slice = p.M * p.ldc;
  // The slices' loads go out kGroup at a time and are then added in slice
  // order, so a thread waits for one load latency per group, not per slice.
  constexpr int kGroup = 8;
  float v[V];
  if constexpr (V == 4) {
    const float4 a = *reinterpret_cast<const float4*>(p.part + idx);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    for (int s0 = 1; s0 < p.ksplit; s0 += kGroup) {
      float4 b[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (s0 + j < p.ksplit) b[j] = *reinterpret_cast<const float4*>(p.part + (s0 + j) * slice + idx);
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (s0 + j < p.ksplit) {
          v[0] += b[j].x; v[1] += b[j].y; v[2] += b[j].z; v[3] += b[j].w;
        }
    }
  } else {
    v[0] = p.part[idx];
    for (int s0 = 1; s0 < p.ksplit; s0 += kGroup) {
      float b[kGroup];
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (s0 + j < p.ksplit) b[j] = p.part[(s0 + j) * slice + idx];
#pragma unroll
      for (int j = 0; j < kGroup; ++j)
        if (s0 + j < p.ksplit) v[0] += b[j];
    }
  }
  E* __restrict__ out = reinterpret_cast<E*>(p.out);
  if (p.epi == kEpiAccFirst || p.epi == kEpiAccMid) {
    if (p.epi == kEpiAccMid) {
#pragma unroll
      for (int q = 0; q < V; ++q) v[q] = p.acc[idx + q] + v[q];
    }
#pragma unroll
    for (int q = 0; q < V; ++q) p.acc[idx + q] = v[q];
    return;
  }
  if (p.epi == kEpiAccLast) {
#pragma unroll
    for (int q = 0; q < V; ++q) v[q] = p.acc[idx + q] + v[q];
  }
  if constexpr (V == 4 && sizeof(E) == 2) {
    uint2 o;
    o.x = uint32_t(from_f32<E, BF16>(v[0])) | (uint32_t(from_f32<E, BF16>(v[1])) << 16);
    o.y = uint32_t(from_f32<E, BF16>(v[2])) | (uint32_t(from_f32<E, BF16>(v[3])) << 16);
    *reinterpret_cast<uint2*>(out + idx) = o;
  } else if constexpr (V == 4) {
    *reinterpret_cast<float4*>(out + idx) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    out[idx] = from_f32<E, BF16>(v[0]);
  }
}

template <typename E, bool BF16>
hipError_t launch_reduce(const GemmParams& p, hipStream_t s) {
  const auto aligned = [](const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) % a) == 0; };
  const bool v4 = p.N % 4 == 0 && p.ldc % 4 == 0 && aligned(p.part, 16) &&
                  (p.epi == kEpiAccFirst || p.epi == kEpiAccMid || aligned(p.out, 4 * sizeof(E))) &&
                  (p.acc == nullptr || aligned(p.acc, 16));
  const int64_t threads = p.M * (v4 ? p.N / 4 : p.N);
  const dim3 grid{unsigned((threads + 255) / 256), 1u, 1u};
  const bool narrow = threads + 256 < (int64_t(1) << 32);
  if (v4) {
    if (narrow) hipLaunchKernelGGL((splitk_reduce_kernel<E, BF16, 4, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((splitk_reduce_kernel<E, BF16, 4, false>), grid, dim3(256), 0, s, p);
  } else {
    if (narrow) hipLaunchKernelGGL((splitk_reduce_kernel<E, BF16, 1, true>), grid, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((splitk_reduce_kernel<E, BF16, 1, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <class Cfg, bool BF16>
hipError_t launch_cfg(const GemmParams& p, hipStream_t s) {
  const dim3 grid(unsigned((p.M + Cfg::BM - 1) / Cfg::BM), unsigned((p.N + Cfg::BN - 1) / Cfg::BN),
                  unsigned(p.ksplit > 1 ? p.ksplit : p.batch));
  const int ve = Cfg::HALF ? 8 : 4;
  const bool bvec = p.ldb % ve == 0 && p.K % ve == 0;
  if (p.a_mode == kADense) {
    if (bvec && p.lda % ve == 0)
      hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadDense, BF16>), grid, dim3(Cfg::NT), 0, s, p);
    else
      hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadDenseScalar, BF16>), grid, dim3(Cfg::NT), 0, s, p);
  } else if (p.kd > 0) {  // native 3D gather
    if (p.c % ve == 0 && bvec)
      hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadImplicit, BF16, true>), grid, dim3(Cfg::NT), 0, s, p);
    else
      hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadScalar, BF16, true>), grid, dim3(Cfg::NT), 0, s, p);
  } else if (p.c % ve == 0 && bvec) {
    hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadImplicit, BF16>), grid, dim3(Cfg::NT), 0, s, p);
  } else {
    hipLaunchKernelGGL((gemm_kernel<Cfg, kLoadScalar, BF16>), grid, dim3(Cfg::NT), 0, s, p);
  }
  return hipGetLastError();
}

template <class Cfg>
hipError_t launch_half(const GemmParams& p, hipStream_t s) {
  return p.dtype == CNHWC_BF16 ? launch_cfg<Cfg, true>(p, s) : launch_cfg<Cfg, false>(p, s);
}

}  // namespace

int splitk_reduce_launch(const GemmParams& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  if (p.ksplit < 2 || !p.part) return hipErrorInvalidValue;
  if (p.dtype == CNHWC_F32) return launch_reduce<float, false>(p, s);
  if (p.dtype == CNHWC_F16) return launch_reduce<uint16_t, false>(p, s);
  return launch_reduce<uint16_t, true>(p, s);
}

int gemm_launch(const GemmParams& p, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (p.M <= 0 || p.N <= 0) return hipSuccess;
  const bool f32cfg = p.config >= kCfgF32_N32 && p.config <= kCfgF32_N128;
  if (f32cfg != (p.dtype == CNHWC_F32)) return hipErrorInvalidValue;
  if (p.ksplit > 1 && (p.batch != 1 || !p.part || p.config == kCfgH_256x256 ||
                       p.config == kCfgH_256x128L || p.config == kCfgH_Patch ||
                       p.kchunk <= 0 || p.kchunk % gemm_config_bk(p.config) != 0 ||
                       (p.ksplit - 1) * p.kchunk >= p.K))
    return hipErrorInvalidValue;
  // segmented A or K-chunk-major operands: the 256-row tiles only
  if ((p.a_seg_len != 0 || p.a_seg_jump != 0 || p.a_kstep != 0 || p.b_kstep != 0) &&
      p.config != kCfgH_256x256 && p.config != kCfgH_256x128L)
    return hipErrorInvalidValue;
  if ((p.a_kstep != 0 || p.b_kstep != 0) &&
      (p.a_mode != kADense || (p.a_kstep != 0 && p.lda != 32) || (p.b_kstep != 0 && p.ldb != 32)))
    return hipErrorInvalidValue;
  switch (p.config) {
    case kCfgF32_N32: return launch_cfg<TileCfg<128, 32, 32, 32, false, 2>, false>(p, s);
    case kCfgF32_N64: return launch_cfg<TileCfg<128, 64, 32, 64, false, 1>, false>(p, s);
    case kCfgF32_N96: return launch_cfg<TileCfg<128, 96, 32, 96, false, 1>, false>(p, s);
    case kCfgF32_N128: return launch_cfg<TileCfg<128, 128, 32, 128, false, 1>, false>(p, s);
    case kCfgH_128x64: return launch_half<TileCfg<128, 64, 32, 64, true, 2>>(p, s);
    case kCfgH_128x128: return launch_half<TileCfg<128, 128, 64, 64, true, 1>>(p, s);
    case kCfgH_256x128: return launch_half<TileCfg<256, 128, 128, 64, true, 1>>(p, s);
    case kCfgH_128x256: return launch_half<TileCfg<128, 256, 64, 128, true, 1>>(p, s);
    case kCfgH_256x256:
    case kCfgH_256x128L: return gemm_lds_launch(p, stream);
    case kCfgH_Patch: return gemm_patch_launch(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cnhwc
