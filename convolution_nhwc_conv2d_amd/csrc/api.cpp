// Forward entry points: argument and plan validation, then the launch
// sequence of the planned algorithm on the caller's stream.  Nothing here
// allocates, synchronises or falls back to another algorithm.
//
// Winograd (MLX PR "Bound winograd conv2d working set by tiling the batch",
// Fix): filter transform once, then for each batch tile the input transform,
// the 64 tile-position GEMMs and the output transform, all through the one
// workspace.  Unfold (MLX PR "Use the explicit gemm for wide convs on neural
// accelerators", Notes): per row chunk, unfold into the one buffer, then GEMM.
// 3D (MLX PR "Decompose small kernel-depth 3D convs into 2D convs", Change):
// per depth tap, a 2D conv on the frame view and the weight depth slice,
// accumulated in fp32; or the native implicit GEMM; or the half-precision
// Winograd path with the depth taps summed inside its GEMMs.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

#include "internal.hpp"

namespace cnhwc {
namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool overlaps(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

cnhwc_status_t hip_status(int e) { return e == hipSuccess ? CNHWC_OK : CNHWC_ERR_HIP; }

// Optional event recording between kernel launches (timed entry points).
struct Recorder {
  void* const* events = nullptr;
  int32_t* kinds = nullptr;
  int32_t n = 0;
  hipStream_t stream = nullptr;
  void mark(int32_t kind) {
    if (!events) return;
    hipEventRecord(reinterpret_cast<hipEvent_t>(events[n]), stream);
    if (kinds) kinds[n] = kind;
    ++n;
  }
};

// Kernels launched by one 2D conv with this plan.
int64_t launches_2d(const cnhwc_plan_t& p, int32_t algo) {
  const int64_t reduce = p.split_k > 1 ? 1 : 0;  // the K-split sum after each GEMM
  if (algo == CNHWC_ALGO_IMPLICIT_GEMM) return 1 + reduce;
  if (algo == CNHWC_ALGO_UNFOLD_GEMM) return (2 + reduce) * p.n_chunks;
  if (algo == CNHWC_ALGO_WINOGRAD) return 1 + 3 * p.n_tiles;
  if (algo == CNHWC_ALGO_WINOGRAD_HALF) return 2 + 3 * p.n_tiles;
  return -1;
}

// Half-precision Winograd F(4x4,3x3) (2D, or 3D with the depth taps summed in
// the GEMMs): the max-|element| pass, the filter transform (which also turns
// the maxima into the scales),
// then per batch tile the input transform, the 36 tile-position GEMMs (fp16
// operands, fp32 results) and the output transform.
cnhwc_status_t run_wino_h(const cnhwc_conv_desc_t& d, const cnhwc_plan_t& p, const void* x,
                          const void* w, void* y, char* ws, void* stream, Recorder& rec) {
  const WinoHLayout L = wino_h_layout(d, p.out_d, p.out_h, p.out_w, p.tile_batch);
  uint32_t* partial = reinterpret_cast<uint32_t*>(ws);
  float* scales = reinterpret_cast<float*>(ws + kWinoHScaleOff);
  uint16_t* U = reinterpret_cast<uint16_t*>(ws + L.off_u);
  uint16_t* V = reinterpret_cast<uint16_t*>(ws + L.off_v);
  float* Mt = reinterpret_cast<float*>(ws + L.off_m);
  uint32_t* wm = reinterpret_cast<uint32_t*>(ws + L.off_wm);
  uint64_t* tm = reinterpret_cast<uint64_t*>(ws + L.off_tm);
  const int64_t nx = d.n * d.d * d.h * d.w * d.c;
  const int64_t nw = d.o * d.kd * d.kh * d.kw * d.c;
  rec.mark(CNHWC_KERNEL_WINO_SCALE);
  if (wino_h_absmax_launch(d.dtype, x, nx, w, nw, partial, stream) != hipSuccess) return CNHWC_ERR_HIP;
  rec.mark(CNHWC_KERNEL_WINO_FILTER);
  if (wino_h_filter_launch(d.dtype, w, d.o, d.kd, d.c, L.cs, partial, nx, nw, scales, U, wm,
                           stream) != hipSuccess)
    return CNHWC_ERR_HIP;

  GemmParams q;
  std::memset(&q, 0, sizeof(q));
  q.dtype = CNHWC_F16;  // the transformed operands are fp16 for either input dtype
  q.a_mode = kADense;
  q.epi = kEpiAccFirst;  // fp32 results
  q.config = p.kernel_config;
  q.N = d.o;
  q.K = L.ku;
  q.lda = L.cs;
  q.b = U;
  // K-chunk-major U: O rows of 32 elements per chunk, one chunk plane after another
  q.ldb = 32;
  q.b_kstep = d.o * 32;
  q.out = Mt;  // not written with kEpiAccFirst
  q.acc = Mt;
  q.ldc = d.o;
  q.batch = kWinoHP;
  q.stride_a = int64_t(L.v_plane);
  q.stride_b = d.o * L.ku;
  q.stride_out = int64_t(L.m_plane);
  if (d.kd > 1) {
    // tap kd reads the transformed rows kd * dd frames further on
    q.a_seg_len = L.cs;
    q.a_seg_jump = (int64_t(d.dil[0]) * L.t - 1) * L.cs;
  }
  const uint64_t x_elem = uint64_t(d.d) * d.h * d.w * d.c * 2;              // bytes per element
  const uint64_t y_elem = uint64_t(p.out_d) * p.out_h * p.out_w * d.o * 2;  // bytes per element
  for (int64_t n0 = 0; n0 < d.n; n0 += p.tile_batch) {
    const int64_t nb = n0 + p.tile_batch <= d.n ? p.tile_batch : d.n - n0;
    rec.mark(CNHWC_KERNEL_WINO_INPUT);
    if (wino_h_input_launch(d.dtype, static_cast<const char*>(x) + n0 * x_elem, nb, d.d, L.dp,
                            d.pad[0], d.h, d.w, d.c, L.cs, d.pad[1], d.pad[2], L.tiles_h,
                            L.tiles_w, scales, V, int64_t(L.v_plane), tm, stream) != hipSuccess)
      return CNHWC_ERR_HIP;
    rec.mark(CNHWC_KERNEL_WINO_GEMM);
    q.M = nb * p.out_d * L.t;
    q.a = V;
    if (gemm_launch(q, stream) != hipSuccess) return CNHWC_ERR_HIP;
    rec.mark(CNHWC_KERNEL_WINO_OUTPUT);
    if (wino_h_output_launch(d.dtype, Mt, int64_t(L.m_plane), nb * p.out_d, p.out_h, p.out_w, d.o,
                             L.tiles_h, L.tiles_w, scales, static_cast<char*>(y) + n0 * y_elem, tm,
                             d.c, L.cs, wm, p.out_d, L.dp, d.kd, d.dil[0], stream) != hipSuccess)
      return CNHWC_ERR_HIP;
  }
  return CNHWC_OK;
}

// One 2D conv (a full 2D call or one depth tap of a 3D call).
//   x: [n][h][w][c] (dtype), w: rows of K = kh*kw*c elements at stride ldw,
//   y: [n][oh][ow][o] (dtype), acc: fp32 rows of the same shape (epi != store).
cnhwc_status_t run_2d(const cnhwc_conv_desc_t& d, const cnhwc_plan_t& p, int32_t algo,
                      const void* x, const void* w, int64_t ldw, void* y, float* acc, int32_t epi,
                      char* ws, void* stream, Recorder& rec) {
  const uint64_t es = dtype_size(d.dtype);
  const int64_t oh = p.out_h, ow = p.out_w;
  const int64_t m_rows = d.n * oh * ow;
  const int64_t k = d.kh * d.kw * d.c;

  GemmParams g;
  std::memset(&g, 0, sizeof(g));
  g.dtype = d.dtype;
  g.epi = epi;
  g.config = p.kernel_config;
  g.N = d.o;
  g.h = d.h;
  g.w = d.w;
  g.c = d.c;
  g.oh = oh;
  g.ow = ow;
  g.kh = d.kh;
  g.kw = d.kw;
  g.sh = d.stride[1];
  g.sw = d.stride[2];
  g.ph = d.pad[1];
  g.pw = d.pad[2];
  g.dh = d.dil[1];
  g.dw = d.dil[2];
  g.batch = 1;
  // K split (plan.split_k > 1): whole K chunks per split; the partial slices
  // sit in the workspace after the unfold buffer (if any).
  g.ksplit = p.split_k;
  if (p.split_k > 1) {
    const int64_t bk = gemm_config_bk(p.kernel_config);
    g.kchunk = ceil_div(ceil_div(k, bk), p.split_k) * bk;
  }
  auto gemm = [&](int32_t kind) -> cnhwc_status_t {
    rec.mark(kind);
    if (gemm_launch(g, stream) != hipSuccess) return CNHWC_ERR_HIP;
    if (g.ksplit > 1) {
      rec.mark(CNHWC_KERNEL_SPLITK_REDUCE);
      if (splitk_reduce_launch(g, stream) != hipSuccess) return CNHWC_ERR_HIP;
    }
    return CNHWC_OK;
  };

  if (algo == CNHWC_ALGO_IMPLICIT_GEMM) {
    g.a_mode = kAImplicit;
    g.M = m_rows;
    g.K = k;
    g.a = x;
    g.b = w;
    g.ldb = ldw;
    g.out = y;
    g.ldc = d.o;
    g.acc = acc;
    g.part = reinterpret_cast<float*>(ws);
    return gemm(CNHWC_KERNEL_IMPLICIT_GEMM);
  }

  if (algo == CNHWC_ALGO_UNFOLD_GEMM) {
    const int64_t kp = unfold_kp(k, d.dtype);
    const int64_t rows = p.unfold_rows;
    g.part = reinterpret_cast<float*>(ws + align_up(uint64_t(rows) * kp * es, 256));
    for (int64_t m0 = 0; m0 < m_rows; m0 += rows) {
      const int64_t r = m0 + rows <= m_rows ? rows : m_rows - m0;
      rec.mark(CNHWC_KERNEL_UNFOLD);
      int e = unfold_launch(d.dtype, x, d.h, d.w, d.c, oh, ow, d.kh, d.kw, d.stride[1],
                            d.stride[2], d.pad[1], d.pad[2], d.dil[1], d.dil[2], m0, r, kp, ws,
                            stream);
      if (e != hipSuccess) return CNHWC_ERR_HIP;
      g.a_mode = kADense;
      g.M = r;
      g.K = k;
      g.a = ws;
      g.lda = kp;
      g.b = w;
      g.ldb = ldw;
      g.out = static_cast<char*>(y) + uint64_t(m0) * d.o * es;
      g.ldc = d.o;
      g.acc = acc ? acc + m0 * d.o : nullptr;
      const cnhwc_status_t st = gemm(CNHWC_KERNEL_UNFOLD_GEMM);
      if (st != CNHWC_OK) return st;
    }
    return CNHWC_OK;
  }

  if (algo == CNHWC_ALGO_WINOGRAD) {
    const WinoLayout L = wino_layout(d, oh, ow, p.tile_batch);
    float* U = reinterpret_cast<float*>(ws + L.off_u);
    float* V = reinterpret_cast<float*>(ws + L.off_v);
    float* Mt = reinterpret_cast<float*>(ws + L.off_m);
    uint32_t* wm = reinterpret_cast<uint32_t*>(ws + L.off_wm);
    uint64_t* tm = reinterpret_cast<uint64_t*>(ws + L.off_tm);
    rec.mark(CNHWC_KERNEL_WINO_FILTER);
    int e = wino_filter_launch(d.dtype, w, ldw, d.o, d.c, L.cs, U, wm, stream);
    if (e != hipSuccess) return CNHWC_ERR_HIP;
    const uint64_t x_elem = uint64_t(d.h) * d.w * d.c * es;  // bytes of one image
    const uint64_t y_elem = uint64_t(oh) * ow * d.o;         // elements of one output image
    for (int64_t n0 = 0; n0 < d.n; n0 += p.tile_batch) {
      const int64_t nb = n0 + p.tile_batch <= d.n ? p.tile_batch : d.n - n0;
      rec.mark(CNHWC_KERNEL_WINO_INPUT);
      e = wino_input_launch(d.dtype, static_cast<const char*>(x) + n0 * x_elem, nb, d.h, d.w, d.c,
                            L.cs, d.pad[1], d.pad[2], L.tiles_h, L.tiles_w, V, int64_t(L.v_plane),
                            tm, stream);
      if (e != hipSuccess) return CNHWC_ERR_HIP;
      rec.mark(CNHWC_KERNEL_WINO_GEMM);
      if (p.kernel_config == kCfgWinoResident) {
        e = wino_gemm_resident_launch(V, U, Mt, nb * L.t, d.o, L.cs, int64_t(L.v_plane),
                                      int64_t(L.m_plane), stream);
      } else {
        GemmParams q;
        std::memset(&q, 0, sizeof(q));
        q.dtype = CNHWC_F32;
        q.a_mode = kADense;
        q.epi = kEpiStore;
        q.config = p.kernel_config;
        q.M = nb * L.t;
        q.N = d.o;
        q.K = L.cs;
        q.a = V;
        q.lda = L.cs;
        q.b = U;
        q.ldb = L.cs;
        q.out = Mt;
        q.ldc = d.o;
        q.batch = kWinoP;
        q.stride_a = int64_t(L.v_plane);
        q.stride_b = d.o * L.cs;
        q.stride_out = int64_t(L.m_plane);
        e = gemm_launch(q, stream);
      }
      if (e != hipSuccess) return CNHWC_ERR_HIP;
      rec.mark(CNHWC_KERNEL_WINO_OUTPUT);
      e = wino_output_launch(d.dtype, Mt, int64_t(L.m_plane), nb, oh, ow, d.o, L.tiles_h,
                             L.tiles_w, static_cast<char*>(y) + n0 * y_elem * es,
                             acc ? acc + n0 * y_elem : nullptr, epi, tm, L.cs, wm, stream);
      if (e != hipSuccess) return CNHWC_ERR_HIP;
    }
    return CNHWC_OK;
  }
  return CNHWC_ERR_INTERNAL;
}

cnhwc_status_t validate(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan, int nd,
                        const void* x, const void* w, const void* y, const void* ws,
                        uint64_t ws_bytes) {
  if (!desc || !plan) return CNHWC_ERR_INVALID_ARGUMENT;
  if (desc->nd != nd) return CNHWC_ERR_INVALID_ARGUMENT;
  cnhwc_plan_t ref;
  const cnhwc_status_t st = select_impl(desc, &plan->opts, &ref);
  if (st != CNHWC_OK) return st;
  if (!plan_equal(ref, *plan)) return CNHWC_ERR_PLAN_MISMATCH;
  if (!x || !w || !y || !aligned16(x) || !aligned16(w) || !aligned16(y))
    return CNHWC_ERR_INVALID_ARGUMENT;
  const uint64_t es = dtype_size(desc->dtype);
  const uint64_t xb = uint64_t(desc->n) * desc->d * desc->h * desc->w * desc->c * es;
  const uint64_t yb = uint64_t(desc->n) * plan->out_d * plan->out_h * plan->out_w * desc->o * es;
  const uint64_t wb = uint64_t(desc->o) * desc->kd * desc->kh * desc->kw * desc->c * es;
  // the written buffers (y, the workspace) may not overlap anything else; x and w may share memory
  if (overlaps(x, xb, y, yb) || overlaps(w, wb, y, yb)) return CNHWC_ERR_INVALID_ARGUMENT;
  if (plan->workspace_bytes > 0) {
    if (ws_bytes < plan->workspace_bytes) return CNHWC_ERR_WORKSPACE_TOO_SMALL;
    if (!ws || !aligned16(ws)) return CNHWC_ERR_INVALID_ARGUMENT;
    const uint64_t wsb = plan->workspace_bytes;
    if (overlaps(ws, wsb, y, yb) || overlaps(ws, wsb, x, xb) || overlaps(ws, wsb, w, wb))
      return CNHWC_ERR_INVALID_ARGUMENT;
  }
  return CNHWC_OK;
}

// Kernels a whole forward call launches (3D: all taps).
int64_t plan_launch_count(const cnhwc_conv_desc_t& d, const cnhwc_plan_t& p) {
  if (d.nd == 3 && p.algo == CNHWC_ALGO_IMPLICIT_GEMM) return p.split_k > 1 ? 2 : 1;
  if (p.algo == CNHWC_ALGO_WINOGRAD_HALF) return launches_2d(p, p.algo);
  if (p.algo == CNHWC_ALGO_SMALL_KD) {
    const int64_t per = launches_2d(p, p.inner_algo);
    return per < 0 ? -1 : per * d.kd;
  }
  return launches_2d(p, p.algo);
}

// 2D forward body shared by the plain and timed entry points.
cnhwc_status_t fwd2d(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan, const void* x,
                     const void* w, void* y, void* workspace, uint64_t workspace_bytes,
                     void* stream, Recorder& rec) {
  const cnhwc_status_t st = validate(desc, plan, 2, x, w, y, workspace, workspace_bytes);
  if (st != CNHWC_OK) return st;
  if (rec.events && plan_launch_count(*desc, *plan) + 1 > rec.n) return CNHWC_ERR_INVALID_ARGUMENT;
  rec.n = 0;
  const cnhwc_status_t s =
      plan->algo == CNHWC_ALGO_WINOGRAD_HALF
          ? run_wino_h(*desc, *plan, x, w, y, static_cast<char*>(workspace), stream, rec)
          : run_2d(*desc, *plan, plan->algo, x, w, desc->kh * desc->kw * desc->c, y, nullptr,
                   kEpiStore, static_cast<char*>(workspace), stream, rec);
  if (s == CNHWC_OK) rec.mark(CNHWC_KERNEL_END);
  return s;
}

cnhwc_status_t fwd3d(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan, const void* x,
                     const void* w, void* y, void* workspace, uint64_t workspace_bytes,
                     void* stream, Recorder& rec) {
  const cnhwc_status_t st = validate(desc, plan, 3, x, w, y, workspace, workspace_bytes);
  if (st != CNHWC_OK) return st;
  if (plan->algo != CNHWC_ALGO_SMALL_KD && plan->algo != CNHWC_ALGO_IMPLICIT_GEMM &&
      plan->algo != CNHWC_ALGO_WINOGRAD_HALF)
    return CNHWC_ERR_INTERNAL;
  if (rec.events && plan_launch_count(*desc, *plan) + 1 > rec.n) return CNHWC_ERR_INVALID_ARGUMENT;
  rec.n = 0;
  const cnhwc_conv_desc_t& d = *desc;
  if (plan->algo == CNHWC_ALGO_WINOGRAD_HALF) {
    const cnhwc_status_t s = run_wino_h(d, *plan, x, w, y, static_cast<char*>(workspace), stream, rec);
    if (s == CNHWC_OK) rec.mark(CNHWC_KERNEL_END);
    return s;
  }
  if (plan->algo == CNHWC_ALGO_IMPLICIT_GEMM) {
    // native 3D implicit GEMM: rows (n, od, oh, ow), k = ((kd*KH + kh)*KW + kw)*C + c
    GemmParams g;
    std::memset(&g, 0, sizeof(g));
    g.dtype = d.dtype;
    g.a_mode = kAImplicit;
    g.epi = kEpiStore;
    g.config = plan->kernel_config;
    g.M = d.n * plan->out_d * plan->out_h * plan->out_w;
    g.N = d.o;
    g.K = d.kd * d.kh * d.kw * d.c;
    g.a = x;
    g.b = w;
    g.ldb = g.K;
    g.out = y;
    g.ldc = d.o;
    g.h = d.h;
    g.w = d.w;
    g.c = d.c;
    g.oh = plan->out_h;
    g.ow = plan->out_w;
    g.kh = d.kh;
    g.kw = d.kw;
    g.sh = d.stride[1];
    g.sw = d.stride[2];
    g.ph = d.pad[1];
    g.pw = d.pad[2];
    g.dh = d.dil[1];
    g.dw = d.dil[2];
    g.d = d.d;
    g.od = plan->out_d;
    g.kd = d.kd;
    g.sd = d.stride[0];
    g.pd = d.pad[0];
    g.dd = d.dil[0];
    g.batch = 1;
    g.ksplit = plan->split_k;
    if (plan->split_k > 1) {
      const int64_t bk = gemm_config_bk(plan->kernel_config);
      g.kchunk = ceil_div(ceil_div(g.K, bk), plan->split_k) * bk;
      g.part = static_cast<float*>(workspace);
    }
    rec.mark(CNHWC_KERNEL_IMPLICIT_GEMM);
    if (gemm_launch(g, stream) != hipSuccess) return CNHWC_ERR_HIP;
    if (g.ksplit > 1) {
      rec.mark(CNHWC_KERNEL_SPLITK_REDUCE);
      if (splitk_reduce_launch(g, stream) != hipSuccess) return CNHWC_ERR_HIP;
    }
    rec.mark(CNHWC_KERNEL_END);
    return CNHWC_OK;
  }
  const int64_t od = plan->out_d;
  const cnhwc_conv_desc_t f = frame_desc(d, od);
  const uint64_t es = dtype_size(d.dtype);
  const uint64_t acc_bytes =
      d.dtype == CNHWC_F32 ? 0 : align_up(uint64_t(od) * plan->out_h * plan->out_w * d.o * 4, 256);
  char* ws = static_cast<char*>(workspace);
  float* acc = d.dtype == CNHWC_F32 ? static_cast<float*>(y) : reinterpret_cast<float*>(ws);
  char* inner_ws = ws ? ws + acc_bytes : nullptr;
  const uint64_t frame_bytes = uint64_t(d.h) * d.w * d.c * es;
  const int64_t k2 = d.kh * d.kw * d.c;
  const int64_t ldw = d.kd * k2;  // weight [O][KD][KH][KW][C]: row stride of one depth slice
  for (int64_t t = 0; t < d.kd; ++t) {
    int32_t epi;
    if (d.kd == 1) epi = kEpiStore;
    else if (d.dtype == CNHWC_F32) epi = t == 0 ? kEpiStore : kEpiAccMid;
    else epi = t == 0 ? kEpiAccFirst : (t == d.kd - 1 ? kEpiAccLast : kEpiAccMid);
    const void* xt = static_cast<const char*>(x) + uint64_t(t) * frame_bytes;
    const void* wt = static_cast<const char*>(w) + uint64_t(t) * k2 * es;
    const cnhwc_status_t s =
        run_2d(f, *plan, plan->inner_algo, xt, wt, ldw, y, acc, epi, inner_ws, stream, rec);
    if (s != CNHWC_OK) return s;
  }
  rec.mark(CNHWC_KERNEL_END);
  return CNHWC_OK;
}

}  // namespace
}  // namespace cnhwc

extern "C" {

int64_t cnhwc_launch_count(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan) {
  using namespace cnhwc;
  if (!desc || !plan) return -1;
  cnhwc_plan_t ref;
  if (select_impl(desc, &plan->opts, &ref) != CNHWC_OK || !plan_equal(ref, *plan)) return -1;
  return plan_launch_count(*desc, *plan);
}

cnhwc_status_t cnhwc_conv2d_fwd(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                const void* x, const void* w, void* y, void* workspace,
                                uint64_t workspace_bytes, void* hip_stream) {
  cnhwc::Recorder rec;
  return cnhwc::fwd2d(desc, plan, x, w, y, workspace, workspace_bytes, hip_stream, rec);
}

cnhwc_status_t cnhwc_conv3d_fwd(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                const void* x, const void* w, void* y, void* workspace,
                                uint64_t workspace_bytes, void* hip_stream) {
  cnhwc::Recorder rec;
  return cnhwc::fwd3d(desc, plan, x, w, y, workspace, workspace_bytes, hip_stream, rec);
}

cnhwc_status_t cnhwc_conv2d_fwd_timed(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                      const void* x, const void* w, void* y, void* workspace,
                                      uint64_t workspace_bytes, void* hip_stream,
                                      void* const* events, int32_t n_events, int32_t* kinds) {
  if (!events || n_events < 1) return CNHWC_ERR_INVALID_ARGUMENT;
  cnhwc::Recorder rec;
  rec.events = events;
  rec.kinds = kinds;
  rec.n = n_events;
  rec.stream = reinterpret_cast<hipStream_t>(hip_stream);
  return cnhwc::fwd2d(desc, plan, x, w, y, workspace, workspace_bytes, hip_stream, rec);
}

cnhwc_status_t cnhwc_conv3d_fwd_timed(const cnhwc_conv_desc_t* desc, const cnhwc_plan_t* plan,
                                      const void* x, const void* w, void* y, void* workspace,
                                      uint64_t workspace_bytes, void* hip_stream,
                                      void* const* events, int32_t n_events, int32_t* kinds) {
  if (!events || n_events < 1) return CNHWC_ERR_INVALID_ARGUMENT;
  cnhwc::Recorder rec;
  rec.events = events;
  rec.kinds = kinds;
  rec.n = n_events;
  rec.stream = reinterpret_cast<hipStream_t>(hip_stream);
  return cnhwc::fwd3d(desc, plan, x, w, y, workspace, workspace_bytes, hip_stream, rec);
}

}  // extern "C"
