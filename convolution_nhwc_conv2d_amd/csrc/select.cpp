// Algorithm selection and memory planning: a pure host function of the
// convolution descriptor and the selection options.  No device call, no
// allocation, no environment read, no dependence on free memory.
//
// Sources (MLX pull requests):
//  - "Bound winograd conv2d working set by tiling the batch", Problem and Fix:
//    the Winograd gate (C%32, O%32, C+O >= 256 for 3x3 stride 1), the budget
//    3/4 of the working-set figure minus the conv's own tensors (input, output,
//    transformed filter), batch tiles sized from it with one reused scratch
//    set, the fallback to implicit GEMM when no element fits or tiles carry
//    too few GEMM rows, and unchanged work when the whole batch fits.  Testing:
//    the budget can be injected and a tile size forced (capped by the budget).
//  - "Use the explicit gemm for wide convs on neural accelerators", intro and
//    Notes: unfold+GEMM for wide output channels in half precision, placed
//    after the Winograd branch; the unfold tiled against a fixed buffer cap.
//    The closing review rejects dispatch on live memory, so none is used.
//  - "Decompose small kernel-depth 3D convs into 2D convs", Change: the guard
//    (idil 1, groups 1, N 1, KD <= 7, depth stride 1, dilation 1, depth pad 0,
//    channels multiple of 16) and the per-tap 2D decomposition.
#include <cstring>
#include <algorithm>

#include "internal.hpp"

namespace cnhwc {

namespace {

int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t d) {
  const int64_t span = in + 2 * p - d * (k - 1) - 1;
  return span < 0 ? 0 : span / s + 1;
}

bool valid_dtype(int32_t dt) { return dt == CNHWC_F32 || dt == CNHWC_F16 || dt == CNHWC_BF16; }

// floor(3/4 * w) without overflow.
uint64_t three_quarters(uint64_t w) { return (w / 4) * 3 + ((w % 4) * 3) / 4; }

// Bound on element counts so every byte size below fits comfortably in 63 bits.
constexpr int64_t kMaxDim = int64_t(1) << 31;
constexpr uint64_t kMaxElems = uint64_t(1) << 56;
// The implicit-GEMM gathers hold a window's origin (o * stride - pad), a tap's
// offset ((k - 1) * dil at most) and their sum in 32-bit integers, and mark
// rows past the end with an origin of -2^30.  With in + 2 * pad <= 2^30 on
// every axis all of them lie in (-2^31, 2^31) and a marked row stays out of
// range; C <= 2^30 keeps the channel position of a K chunk (at most C - 1 plus
// one chunk) in range too.  Larger convs are UNSUPPORTED.
constexpr int64_t kMaxSpan = int64_t(1) << 30;

cnhwc_status_t check_desc(const cnhwc_conv_desc_t& d, int64_t out[3]) {
  if (d.nd != 2 && d.nd != 3) return CNHWC_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(d.dtype)) return CNHWC_ERR_INVALID_ARGUMENT;
  const int64_t dims[9] = {d.n, d.d, d.h, d.w, d.c, d.o, d.kd, d.kh, d.kw};
  for (int64_t v : dims)
    if (v < 1 || v > kMaxDim) return CNHWC_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 3; ++i) {
    if (d.stride[i] < 1 || d.pad[i] < 0 || d.dil[i] < 1) return CNHWC_ERR_INVALID_ARGUMENT;
    if (d.stride[i] > (1 << 20) || d.pad[i] > (1 << 20) || d.dil[i] > (1 << 20))
      return CNHWC_ERR_INVALID_ARGUMENT;
  }
  if (d.groups != 1) return d.groups < 1 ? CNHWC_ERR_INVALID_ARGUMENT : CNHWC_ERR_UNSUPPORTED;
  if (d.nd == 2 && (d.d != 1 || d.kd != 1 || d.stride[0] != 1 || d.pad[0] != 0 || d.dil[0] != 1))
    return CNHWC_ERR_INVALID_ARGUMENT;
  const int64_t ins[3] = {d.d, d.h, d.w};
  for (int i = 0; i < 3; ++i)
    if (ins[i] + 2 * int64_t(d.pad[i]) > kMaxSpan) return CNHWC_ERR_UNSUPPORTED;
  if (d.c > kMaxSpan) return CNHWC_ERR_UNSUPPORTED;
  out[0] = out_extent(d.d, d.kd, d.stride[0], d.pad[0], d.dil[0]);
  out[1] = out_extent(d.h, d.kh, d.stride[1], d.pad[1], d.dil[1]);
  out[2] = out_extent(d.w, d.kw, d.stride[2], d.pad[2], d.dil[2]);
  if (out[0] < 1 || out[1] < 1 || out[2] < 1) return CNHWC_ERR_INVALID_ARGUMENT;
  const double ex = double(d.n) * d.d * d.h * d.w * d.c;
  const double ey = double(d.n) * out[0] * out[1] * out[2] * d.o;
  const double ew = double(d.o) * d.kd * d.kh * d.kw * d.c;
  if (ex > double(kMaxElems) || ey > double(kMaxElems) || ew > double(kMaxElems))
    return CNHWC_ERR_INVALID_ARGUMENT;
  return CNHWC_OK;
}

bool winograd_geometry(const cnhwc_conv_desc_t& d) {
  return d.nd == 2 && d.kh == 3 && d.kw == 3 && d.stride[1] == 1 && d.stride[2] == 1 &&
         d.dil[1] == 1 && d.dil[2] == 1;
}

// The channel/dtype gate AUTO applies on top of the geometry.  The pages' gate
// is C%32, O%32, C+O >= 256; on MI355X Winograd is only taken automatically
// for fp32 (fp16/bf16 implicit GEMM runs on the much faster half-precision
// matrix cores; the Winograd transforms keep fp32 tensors).
bool winograd_auto_gate(const cnhwc_conv_desc_t& d) {
  return winograd_geometry(d) && d.c % 32 == 0 && d.o % 32 == 0 && d.c + d.o >= 256 &&
         d.dtype == CNHWC_F32;
}

// Half-precision Winograd F(4x4,3x3): 3x3 taps in the image plane, stride 1 and
// dilation 1 there, fp16/bf16 only (3D: depth stride 1; any depth, depth pad
// and depth dilation).  Accuracy limits: the fp16 rounding of a tile's
// transformed values scales with the whole 6x6 tile, so an output whose 3x3
// window is mostly padding (image-plane padding of 2 or more: a corner window
// holds one real pixel of nine) can see errors of 1-3e-2 of its own
// sum |x||w|; and the rounding errors of fewer than 16 channels do not average
// down (8 channels with padding 1: up to 9e-3).  Padding <= 1 in the image
// plane and C >= 16 keep the measured error below 5e-3.
bool winograd_h_geometry(const cnhwc_conv_desc_t& d) {
  return d.dtype != CNHWC_F32 && d.kh == 3 && d.kw == 3 && d.stride[1] == 1 &&
         d.stride[2] == 1 && d.dil[1] == 1 && d.dil[2] == 1 && d.stride[0] == 1 &&
         d.pad[1] <= 1 && d.pad[2] <= 1 && d.c >= 16;
}

// AUTO's rule for the half-precision Winograd path (on top of its geometry).
// Per output pixel it moves about 11 C + 20 O bytes more than the implicit
// GEMM (fp16 V written and read, x read: C side; fp32 M written and read, y
// written: O side) and saves 13.5 KD C O of the 18 KD C O multiply-adds.  On
// MI355X (bf16/fp16, 3x3, C, O in 64..2048, 2D and 3D) it was faster in
// every measured case with KD C >= 384 and KD C O >= 13 (11 C + 20 O), by
// 1.1-2.6x, and slower in every case with C = 256 in 2D (0.7-0.96x) or
// 3D 64 -> 128 (0.78x); between 12 and 13 it depends on the implicit GEMM's
// efficiency at the shape (0.93-1.3x) and is left to the implicit GEMM.
// Below 512 GEMM rows (N OD tiles) the fixed cost of the scale and filter
// passes (about 25 us) decides: 0.66-1.02x.
bool winograd_h_auto_gate(const cnhwc_conv_desc_t& d, const int64_t out[3]) {
  const double kc = double(d.kd) * double(d.c);
  const double rows = double(d.n) * double(out[0]) * double(ceil_div(out[1], kWinoHM)) *
                      double(ceil_div(out[2], kWinoHM));
  return kc >= 384 && kc * double(d.o) >= 13.0 * (11.0 * double(d.c) + 20.0 * double(d.o)) &&
         rows >= 512;
}

// The 256-row GEMM tile for the half-precision Winograd GEMMs (rows x n x k,
// batch tile positions).  With a short K loop (k <= 1152) and n <= 512 the
// 256 x 128 tile at two workgroups per CU measured faster on nearly every
// shape (the other workgroup's MFMAs cover one's fp32 result stores; up to
// 1.2x); with longer K loops or wider n, the occupancy model of
// pick_gemm_config over the two direct-to-LDS tiles (the 256 x 256 tile: 5%
// faster on the 41x120x208 512 -> 512 video conv, K = 1536).
int32_t pick_lds_tile(int64_t rows, int64_t n, int64_t k, int64_t batch) {
  if (k <= 1152 && n <= 512) return kCfgH_256x128L;
  struct Cand { int32_t id; int64_t bn, occ; double eff; };
  const Cand cands[2] = {{kCfgH_256x256, 256, 1, 1.35}, {kCfgH_256x128L, 128, 2, 1.20}};
  constexpr int64_t kCUs = 256;
  int32_t best = kCfgH_256x256;
  double best_t = 1e300;
  for (const Cand& c : cands) {
    const int64_t tiles = ceil_div(rows, 256) * ceil_div(n, c.bn) * batch;
    const double t = double(ceil_div(tiles, kCUs * c.occ)) * double(256 * c.bn * c.occ) / c.eff;
    if (t < best_t) { best_t = t; best = c.id; }
  }
  return best;
}

void tile_rule(uint64_t ws_limit, uint64_t own, uint64_t scratch, int64_t n, int64_t rows,
               int64_t force_tile, int64_t* tile, uint64_t* budget, int32_t* fallback) {
  const uint64_t q = three_quarters(ws_limit);
  const uint64_t b = q > own ? q - own : 0;
  const uint64_t fit = scratch ? b / scratch : 0;
  int64_t t = fit > uint64_t(n) ? n : int64_t(fit);
  if (force_tile > 0) t = std::min<int64_t>(t, force_tile);
  *tile = t;
  *budget = b;
  *fallback = (t < 1) || (force_tile <= 0 && t < n && t * rows < CNHWC_MIN_TILE_ROWS);
}

// K splits for a GEMM grid too small to fill the device (tiles of gemm.hip
// only; the direct-to-LDS tiles and the Winograd GEMMs never split).  Each split
// gets a whole number of K chunks and at least 3 (at least 4 measured 13%
// slower on a single 16x16 image, 32 -> 32, with the ResNet-50 stacks
// unchanged); trailing empty splits are dropped.  Returns 1 for no split.
int32_t pick_split_k(int32_t cfg, int64_t m, int64_t n, int64_t k) {
  int64_t bm = 128, bn = 128, occ = 2;
  switch (cfg) {
    case kCfgF32_N32: bn = 32; break;
    case kCfgF32_N64: bn = 64; break;
    case kCfgF32_N96: bn = 96; break;
    case kCfgF32_N128: bn = 128; break;
    case kCfgH_128x64: bn = 64; break;
    case kCfgH_128x128: break;
    case kCfgH_256x128: bm = 256; occ = 1; break;
    case kCfgH_128x256: bn = 256; occ = 1; break;
    default: return 1;
  }
  constexpr int64_t kCUs = 256;
  const int64_t tiles = ceil_div(m, bm) * ceil_div(n, bn);
  const int64_t slots = kCUs * occ;
  if (2 * tiles > slots) return 1;
  const int64_t nk = ceil_div(k, gemm_config_bk(cfg));
  const int64_t s = std::min<int64_t>(std::min<int64_t>(slots / tiles, nk / 3), kMaxSplitK);
  if (s < 2) return 1;
  const int64_t per = ceil_div(nk, s);
  return int32_t(ceil_div(nk, per));
}

// K splits: forced, or picked.
cnhwc_status_t split_k_for(int32_t cfg, int64_t m, int64_t n, int64_t k, int32_t force,
                           int32_t* splits) {
  if (force == 0) {
    *splits = pick_split_k(cfg, m, n, k);
    return CNHWC_OK;
  }
  if (force == 1) {
    *splits = 1;
    return CNHWC_OK;
  }
  const int64_t nk = ceil_div(k, gemm_config_bk(cfg));
  if (cfg == kCfgH_256x256 || cfg == kCfgH_256x128L || cfg == kCfgH_Patch || force > nk)
    return CNHWC_ERR_NOT_APPLICABLE;
  *splits = int32_t(ceil_div(nk, ceil_div(nk, int64_t(force))));
  return CNHWC_OK;
}

// Bytes of the fp32 partial slices of a split GEMM with `rows` rows.
uint64_t split_k_bytes(int32_t splits, int64_t rows, int64_t o) {
  return splits > 1 ? align_up(uint64_t(splits) * uint64_t(rows) * uint64_t(o) * 4, 256) : 0;
}

// Tile configuration of the implicit / unfold GEMM: forced, or picked.  The
// direct-to-LDS tiles need C % 32 == 0 (implicit: a K chunk never
// straddles two taps) or K % 8 == 0 (unfold rows).
// The patch-staged implicit GEMM (gemm_patch.hip): 3x3 taps in the image
// plane at stride 1 and dilation 1 (any depth geometry), fp16/bf16, C % 64 ==
// 0, and 32-bit element offsets within one input frame.
bool patch_ok(const cnhwc_conv_desc_t& d) {
  return d.dtype != CNHWC_F32 && d.kh == 3 && d.kw == 3 && d.stride[1] == 1 && d.stride[2] == 1 &&
         d.dil[1] == 1 && d.dil[2] == 1 && d.c % 64 == 0 && d.h * d.w * d.c < (int64_t(1) << 31);
}

// Relative throughput of the patch-staged tile against the 128x128 tile's
// (the occupancy model of pick_gemm_config): measured on the C_out axis and
// video shapes of the sweeps.
constexpr double kPatchEff = 1.8;

cnhwc_status_t gemm_config_for(const cnhwc_conv_desc_t& d, const int64_t out[3], int64_t m_rows,
                               bool implicit, int32_t force, int32_t* cfg) {
  const int64_t k = d.kh * d.kw * d.c;
  const bool lds_ok = d.dtype != CNHWC_F32 && (implicit ? d.c % 32 == 0 : k % 8 == 0);
  const bool pok = implicit && patch_ok(d);
  if (force == 0) {
    *cfg = pick_gemm_config(d.dtype, m_rows, d.o, lds_ok);
    if (pok) {
      // the patch tile against the model's pick, by the same waves-of-256-CUs estimate
      constexpr int64_t kCUs = 256;
      const int64_t frames = m_rows / (out[1] * out[2]);
      const int64_t tiles = patch_row_tiles(frames, out[1], out[2]) * ceil_div(d.o, 256);
      const double t_patch = double(ceil_div(tiles, kCUs)) * 256.0 * 256.0 / kPatchEff;
      if (t_patch <= gemm_config_time(d.dtype, *cfg, m_rows, d.o)) *cfg = kCfgH_Patch;
    }
    return CNHWC_OK;
  }
  const bool f32 = force >= kCfgF32_N32 && force <= kCfgF32_N128;
  const bool half = force >= kCfgH_128x64 && force <= kCfgH_Patch;
  const bool lds = force == kCfgH_256x256 || force == kCfgH_256x128L;
  if ((d.dtype == CNHWC_F32 && !f32) || (d.dtype != CNHWC_F32 && !half) || (lds && !lds_ok) ||
      (force == kCfgH_Patch && !pok))
    return CNHWC_ERR_NOT_APPLICABLE;
  *cfg = force;
  return CNHWC_OK;
}

// Plan of the half-precision Winograd path (2D, or 3D with one batch element
// per tile), forced or under AUTO.  Returns OK with the plan, BUDGET when no
// batch element fits the budget (AUTO then falls back), NOT_APPLICABLE for a
// forced GEMM tile other than the two 256-row tiles.
cnhwc_status_t plan_winograd_h(const cnhwc_conv_desc_t& d, const int64_t out[3],
                               const cnhwc_select_opts_t& o, bool forced, cnhwc_plan_t* p) {
  const uint64_t es = dtype_size(d.dtype);
  const WinoHLayout one = wino_h_layout(d, out[0], out[1], out[2], 1);
  const uint64_t own = uint64_t(d.n) * d.d * d.h * d.w * d.c * es +
                       uint64_t(d.n) * out[0] * out[1] * out[2] * d.o * es + kWinoHHeadBytes +
                       align_up(one.u_bytes, 256) + align_up(one.wm_bytes, 256);
  // V + M + the tile masks of one element
  const uint64_t scratch = uint64_t(kWinoHP) * one.t * (one.dp * one.cs * 2 + out[0] * d.o * 4) +
                           uint64_t(one.dp) * one.t * one.mask_parts * 8;
  int64_t tb;
  uint64_t budget;
  int32_t fb;
  // 3D: one element per tile (a GEMM's rows shift by whole frames within one element)
  const int64_t force_tile = d.nd == 3 ? 1 : o.force_tile_batch;
  tile_rule(o.ws_limit_bytes, own, scratch, d.n, one.t * out[0], force_tile, &tb, &budget, &fb);
  if (tb < 1 || (!forced && fb)) return CNHWC_ERR_BUDGET;
  int32_t cfg = o.force_gemm_config;
  if (cfg != 0 && cfg != kCfgH_256x256 && cfg != kCfgH_256x128L) return CNHWC_ERR_NOT_APPLICABLE;
  // the GEMM tile depends on the untiled shape only
  if (cfg == 0) cfg = pick_lds_tile((d.nd == 3 ? 1 : d.n) * out[0] * one.t, d.o, one.ku, kWinoHP);
  const WinoHLayout lay = wino_h_layout(d, out[0], out[1], out[2], tb);
  p->algo = p->inner_algo = CNHWC_ALGO_WINOGRAD_HALF;
  p->out_d = out[0];
  p->out_h = out[1];
  p->out_w = out[2];
  p->tile_batch = tb;
  p->n_tiles = ceil_div(d.n, tb);
  p->tiles_per_image = lay.t;
  p->own_bytes = own;
  p->budget_bytes = budget;
  p->scratch_per_element = scratch;
  p->workspace_bytes = lay.total;
  p->kernel_config = cfg;
  p->split_k = 1;
  return CNHWC_OK;
}

cnhwc_status_t select_2d(const cnhwc_conv_desc_t& d, const int64_t out[3],
                         const cnhwc_select_opts_t& o, int32_t force, cnhwc_plan_t* p) {
  const uint64_t es = dtype_size(d.dtype);
  const int64_t m_rows = d.n * out[1] * out[2];
  const int64_t k = d.kh * d.kw * d.c;
  p->out_d = 1;
  p->out_h = out[1];
  p->out_w = out[2];
  p->split_k = 1;
  cnhwc_status_t st = CNHWC_OK;

  if (force != CNHWC_ALGO_AUTO && force != CNHWC_ALGO_WINOGRAD &&
      force != CNHWC_ALGO_IMPLICIT_GEMM && force != CNHWC_ALGO_UNFOLD_GEMM &&
      force != CNHWC_ALGO_WINOGRAD_HALF)
    return force == CNHWC_ALGO_SMALL_KD ? CNHWC_ERR_NOT_APPLICABLE : CNHWC_ERR_INVALID_ARGUMENT;

  // 1. Winograd (gate + budget), or forced.
  const bool try_wino = force == CNHWC_ALGO_WINOGRAD ||
                        (force == CNHWC_ALGO_AUTO && winograd_auto_gate(d));
  if (force == CNHWC_ALGO_WINOGRAD && !winograd_geometry(d)) return CNHWC_ERR_NOT_APPLICABLE;
  if (try_wino) {
    const WinoLayout one = wino_layout(d, out[1], out[2], 1);
    // own: x, y and the transformed filter (U and its tap masks)
    const uint64_t own = uint64_t(d.n) * d.h * d.w * d.c * es +
                         uint64_t(m_rows) * d.o * es + one.u_bytes + one.wm_bytes;
    // V + M + the tile masks of one element
    const uint64_t scratch =
        uint64_t(kWinoP) * one.t * (one.cs + d.o) * 4 + uint64_t(one.t) * one.mask_parts * 8;
    int64_t tb;
    uint64_t budget;
    int32_t fb;
    tile_rule(o.ws_limit_bytes, own, scratch, d.n, one.t, o.force_tile_batch, &tb, &budget, &fb);
    if (force == CNHWC_ALGO_WINOGRAD && tb < 1) return CNHWC_ERR_BUDGET;
    if (force == CNHWC_ALGO_WINOGRAD || !fb) {
      const WinoLayout lay = wino_layout(d, out[1], out[2], tb);
      p->algo = p->inner_algo = CNHWC_ALGO_WINOGRAD;
      p->tile_batch = tb;
      p->n_tiles = ceil_div(d.n, tb);
      p->tiles_per_image = lay.t;
      p->own_bytes = own;
      p->budget_bytes = budget;
      p->scratch_per_element = scratch;
      p->workspace_bytes = lay.total;
      // the GEMM configuration depends on (C, O) only, never on the batch tiling
      p->kernel_config = wino_gemm_resident_ok(lay.cs, d.o) ? int32_t(kCfgWinoResident)
                                                            : pick_gemm_config(CNHWC_F32, 0, d.o, false);
      return CNHWC_OK;
    }
  }

  // 1b. Half-precision Winograd F(4x4,3x3), forced or under its AUTO rule.
  if (force == CNHWC_ALGO_WINOGRAD_HALF) {
    if (!winograd_h_geometry(d)) return CNHWC_ERR_NOT_APPLICABLE;
    return plan_winograd_h(d, out, o, true, p);
  }
  if (force == CNHWC_ALGO_AUTO && winograd_h_geometry(d) && winograd_h_auto_gate(d, out)) {
    cnhwc_plan_t h = *p;
    if (plan_winograd_h(d, out, o, false, &h) == CNHWC_OK) {
      *p = h;
      return CNHWC_OK;
    }
  }

  // 2. Unfold + GEMM for wide half-precision convs (the explicit page's rule),
  // for half-precision convs whose implicit gather would go element by element
  // (C % 8 != 0: no 16-byte channel vectors; measured 1.3-1.9x faster above the
  // launch floor, e.g. the 3-channel stem), or forced.
  if (force == CNHWC_ALGO_UNFOLD_GEMM ||
      (force == CNHWC_ALGO_AUTO && d.dtype != CNHWC_F32 &&
       (d.o >= CNHWC_UNFOLD_MIN_COUT || d.c % 8 != 0))) {
    const int64_t kp = unfold_kp(k, d.dtype);
    int64_t rows = o.force_unfold_rows > 0
                       ? o.force_unfold_rows
                       : int64_t(CNHWC_UNFOLD_CAP_BYTES / (uint64_t(kp) * es));
    rows = std::max<int64_t>(1, std::min<int64_t>(rows, m_rows));
    p->algo = p->inner_algo = CNHWC_ALGO_UNFOLD_GEMM;
    p->unfold_rows = rows;
    p->n_chunks = ceil_div(m_rows, rows);
    st = gemm_config_for(d, out, m_rows, false, o.force_gemm_config, &p->kernel_config);
    if (st != CNHWC_OK) return st;
    st = split_k_for(p->kernel_config, m_rows, d.o, k, o.force_split_k, &p->split_k);
    if (st != CNHWC_OK) return st;
    p->workspace_bytes = align_up(uint64_t(rows) * kp * es, 256) + split_k_bytes(p->split_k, rows, d.o);
    return CNHWC_OK;
  }

  // 3. Implicit GEMM (scratch-free).
  p->algo = p->inner_algo = CNHWC_ALGO_IMPLICIT_GEMM;
  st = gemm_config_for(d, out, m_rows, true, o.force_gemm_config, &p->kernel_config);
  if (st != CNHWC_OK) return st;
  st = split_k_for(p->kernel_config, m_rows, d.o, k, o.force_split_k, &p->split_k);
  if (st != CNHWC_OK) return st;
  p->workspace_bytes = split_k_bytes(p->split_k, m_rows, d.o);
  return CNHWC_OK;
}

cnhwc_status_t select_3d(const cnhwc_conv_desc_t& d, const int64_t out[3],
                         const cnhwc_select_opts_t& o, cnhwc_plan_t* p) {
  const bool force_kd = o.force_algo == CNHWC_ALGO_SMALL_KD;
  const bool force_native = o.force_algo == CNHWC_ALGO_IMPLICIT_GEMM;
  const bool force_wh = o.force_algo == CNHWC_ALGO_WINOGRAD_HALF;
  if (o.force_algo != CNHWC_ALGO_AUTO && !force_kd && !force_native && !force_wh)
    return CNHWC_ERR_NOT_APPLICABLE;
  if ((force_native || force_wh) && o.force_inner_algo != CNHWC_ALGO_AUTO)
    return CNHWC_ERR_INVALID_ARGUMENT;

  // 0. Half-precision Winograd with the depth taps summed in the GEMM: forced,
  // or under its AUTO rule (over budget: fall through).
  if (force_wh) {
    if (!winograd_h_geometry(d)) return CNHWC_ERR_NOT_APPLICABLE;
    return plan_winograd_h(d, out, o, true, p);
  }
  if (o.force_algo == CNHWC_ALGO_AUTO && o.force_inner_algo == CNHWC_ALGO_AUTO &&
      winograd_h_geometry(d) && winograd_h_auto_gate(d, out)) {
    cnhwc_plan_t h = *p;
    if (plan_winograd_h(d, out, o, false, &h) == CNHWC_OK) {
      *p = h;
      return CNHWC_OK;
    }
  }
  // Structural requirements of the decomposition itself.
  const bool structural = d.n == 1 && d.stride[0] == 1 && d.dil[0] == 1 && d.pad[0] == 0;
  // AUTO guard: also KD <= 7, dilation 1 everywhere, channels multiple of 16.
  const bool guard = structural && d.kd <= 7 && d.dil[1] == 1 && d.dil[2] == 1 &&
                     d.c % 16 == 0 && d.o % 16 == 0;
  if (force_kd && !structural) return CNHWC_ERR_NOT_APPLICABLE;

  // 1. Depth decomposition (MLX PR "Decompose small kernel-depth 3D convs into
  // 2D convs", Change): forced, or under AUTO when the guard holds and the
  // per-frame 2D conv takes Winograd (the reason the page decomposes: the 2D
  // path has Winograd, the native 3D path does not) or an inner algorithm is
  // forced.
  if (force_kd || (!force_native && guard)) {
    const cnhwc_conv_desc_t f = frame_desc(d, out[0]);
    int64_t fo[3];
    cnhwc_status_t st = check_desc(f, fo);
    if (st != CNHWC_OK) return st;
    cnhwc_plan_t inner;
    std::memset(&inner, 0, sizeof(inner));
    st = select_2d(f, fo, o, o.force_inner_algo, &inner);
    if (st == CNHWC_OK && inner.algo == CNHWC_ALGO_WINOGRAD_HALF) {
      // its output transform has no accumulate epilogue: the frames take the
      // implicit GEMM instead (the fused 3D form above is the better use)
      std::memset(&inner, 0, sizeof(inner));
      st = select_2d(f, fo, o, CNHWC_ALGO_IMPLICIT_GEMM, &inner);
    }
    if (st != CNHWC_OK) return st;
    if (force_kd || inner.algo == CNHWC_ALGO_WINOGRAD || o.force_inner_algo != CNHWC_ALGO_AUTO) {
      *p = inner;
      p->algo = CNHWC_ALGO_SMALL_KD;
      p->inner_algo = inner.algo;
      p->out_d = out[0];
      const uint64_t acc = d.dtype == CNHWC_F32
                               ? 0
                               : align_up(uint64_t(out[0]) * out[1] * out[2] * d.o * 4, 256);
      p->workspace_bytes = acc + inner.workspace_bytes;
      return CNHWC_OK;
    }
  } else if (o.force_inner_algo != CNHWC_ALGO_AUTO) {
    return CNHWC_ERR_NOT_APPLICABLE;  // an inner algorithm needs the decomposition
  }

  // 2. Native 3D implicit GEMM: one GEMM with K = KD*KH*KW*C over the NDHWC
  // gather, any batch, depth stride, padding and dilation.  It is the page's
  // fall-through for what the guard rejects, and (all taps in one K loop, no
  // per-tap accumulator passes) the fused form of the decomposition.
  const int64_t m_rows = d.n * out[0] * out[1] * out[2];
  const int64_t k = d.kd * d.kh * d.kw * d.c;
  p->algo = p->inner_algo = CNHWC_ALGO_IMPLICIT_GEMM;
  p->out_d = out[0];
  p->out_h = out[1];
  p->out_w = out[2];
  p->split_k = 1;
  cnhwc_status_t st = gemm_config_for(d, out, m_rows, true, o.force_gemm_config, &p->kernel_config);
  if (st != CNHWC_OK) return st;
  st = split_k_for(p->kernel_config, m_rows, d.o, k, o.force_split_k, &p->split_k);
  if (st != CNHWC_OK) return st;
  p->workspace_bytes = split_k_bytes(p->split_k, m_rows, d.o);
  return CNHWC_OK;
}

}  // namespace

WinoLayout wino_layout(const cnhwc_conv_desc_t& d, int64_t oh, int64_t ow, int64_t tb) {
  WinoLayout l{};
  l.tiles_h = ceil_div(oh, kWinoM);
  l.tiles_w = ceil_div(ow, kWinoM);
  l.t = l.tiles_h * l.tiles_w;
  l.cs = wino_cs(d.c);
  l.mask_parts = wino_mask_parts(l.cs);
  const uint64_t rows = uint64_t(tb) * l.t;
  l.u_bytes = uint64_t(kWinoP) * d.o * l.cs * 4;
  l.wm_bytes = uint64_t(d.o) * 4;
  l.v_plane = rows * l.cs;
  l.m_plane = rows * d.o;
  l.off_u = 0;
  l.off_wm = align_up(l.u_bytes, 256);
  l.off_v = l.off_wm + align_up(l.wm_bytes, 256);
  l.off_m = l.off_v + align_up(kWinoP * l.v_plane * 4, 256);
  l.off_tm = l.off_m + align_up(kWinoP * l.m_plane * 4, 256);
  l.total = l.off_tm + align_up(rows * l.mask_parts * 8, 256);
  return l;
}

WinoHLayout wino_h_layout(const cnhwc_conv_desc_t& d, int64_t od, int64_t oh, int64_t ow,
                          int64_t tb) {
  WinoHLayout l{};
  l.tiles_h = ceil_div(oh, kWinoHM);
  l.tiles_w = ceil_div(ow, kWinoHM);
  l.t = l.tiles_h * l.tiles_w;
  l.cs = wino_h_cs(d.c);
  l.mask_parts = wino_mask_parts(l.cs / wino_h_vec(d.c));
  l.dp = d.d + 2 * int64_t(d.pad[0]);
  l.ku = d.kd * l.cs;
  l.u_bytes = uint64_t(kWinoHP) * d.o * l.ku * 2;
  l.wm_bytes = uint64_t(d.o) * d.kd * 4;
  const uint64_t in_rows = uint64_t(tb) * l.dp * l.t;
  l.v_plane = in_rows * l.cs;
  l.m_plane = uint64_t(tb) * od * l.t * d.o;
  l.off_u = kWinoHHeadBytes;
  l.off_wm = l.off_u + align_up(l.u_bytes, 256);
  l.off_v = l.off_wm + align_up(l.wm_bytes, 256);
  l.off_m = l.off_v + align_up(kWinoHP * l.v_plane * 2, 256);
  l.off_tm = l.off_m + align_up(kWinoHP * l.m_plane * 4, 256);
  l.total = l.off_tm + align_up(in_rows * l.mask_parts * 8, 256);
  return l;
}

cnhwc_conv_desc_t frame_desc(const cnhwc_conv_desc_t& d3, int64_t od) {
  cnhwc_conv_desc_t f = d3;
  f.nd = 2;
  f.n = od;
  f.d = 1;
  f.kd = 1;
  f.stride[0] = 1;
  f.pad[0] = 0;
  f.dil[0] = 1;
  return f;
}

namespace {
// The half-precision candidates of the occupancy model (see pick_gemm_config).
struct HalfCand { int32_t id; int64_t bm, bn, occ; double eff; };
constexpr HalfCand kHalfCands[6] = {{kCfgH_128x128, 128, 128, 2, 1.00}, {kCfgH_128x256, 128, 256, 1, 0.85},
                                    {kCfgH_256x128, 256, 128, 1, 0.80}, {kCfgH_128x64, 128, 64, 2, 0.70},
                                    {kCfgH_256x256, 256, 256, 1, 1.35}, {kCfgH_256x128L, 256, 128, 2, 1.20}};
double half_cand_time(const HalfCand& c, int64_t m_rows, int64_t n_cols) {
  constexpr int64_t kCUs = 256;
  const int64_t tiles = ceil_div(m_rows, c.bm) * ceil_div(n_cols, c.bn);
  const int64_t waves = ceil_div(tiles, kCUs * c.occ);
  return double(waves) * double(c.bm * c.bn * c.occ) / c.eff;
}
}  // namespace

int32_t pick_gemm_config(int dtype, int64_t m_rows, int64_t n_cols, bool lds_ok) {
  if (dtype == CNHWC_F32) {
    if (n_cols <= 32) return kCfgF32_N32;
    if (n_cols <= 64) return kCfgF32_N64;
    // least padding waste over {128, 96, 64}; ties go to the wider tile
    const int64_t cand[3] = {128, 96, 64};
    const int32_t ids[3] = {kCfgF32_N128, kCfgF32_N96, kCfgF32_N64};
    int best = 0;
    int64_t best_waste = ceil_div(n_cols, cand[0]) * cand[0] - n_cols;
    for (int i = 1; i < 3; ++i) {
      const int64_t waste = ceil_div(n_cols, cand[i]) * cand[i] - n_cols;
      if (waste < best_waste) { best = i; best_waste = waste; }
    }
    return ids[best];
  }
  // Half precision: estimated time = (waves of workgroups over the CUs) x
  // (cost of one wave).  A wave of slots costs BM*BN*occupancy/efficiency:
  // `occ` workgroups share a CU, `eff` is the measured relative throughput of
  // the tile shape on MI355X (128x128 at two workgroups per CU is the fastest
  // on every large conv of the sweep; the 256-wide tiles need one CU each and
  // lose about 20%; 128x64 is for problems too small to fill the chip).
  // The tiles with direct loads into LDS ran, on the large convs of the
  // sweep, 1.32-1.47x (256x256, one workgroup per CU) and 1.13-1.40x (256x128,
  // two per CU) the 128x128 rate; the 256x128 tile wastes less when O is not
  // a multiple of 256.
  int32_t best = kCfgH_128x128;
  double best_t = 1e300;
  for (const HalfCand& c : kHalfCands) {
    if ((c.id == kCfgH_256x256 || c.id == kCfgH_256x128L) && !lds_ok) continue;
    const double t = half_cand_time(c, m_rows, n_cols);
    if (t < best_t) { best_t = t; best = c.id; }
  }
  return best;
}

double gemm_config_time(int dtype, int32_t cfg, int64_t m_rows, int64_t n_cols) {
  if (dtype == CNHWC_F32) return 1e300;
  for (const HalfCand& c : kHalfCands)
    if (c.id == cfg) return half_cand_time(c, m_rows, n_cols);
  return 1e300;
}

bool plan_equal(const cnhwc_plan_t& a, const cnhwc_plan_t& b) {
  return a.algo == b.algo && a.inner_algo == b.inner_algo && a.out_d == b.out_d &&
         a.out_h == b.out_h && a.out_w == b.out_w && a.tile_batch == b.tile_batch &&
         a.n_tiles == b.n_tiles && a.tiles_per_image == b.tiles_per_image &&
         a.unfold_rows == b.unfold_rows && a.n_chunks == b.n_chunks &&
         a.own_bytes == b.own_bytes && a.budget_bytes == b.budget_bytes &&
         a.scratch_per_element == b.scratch_per_element &&
         a.workspace_bytes == b.workspace_bytes && a.kernel_config == b.kernel_config &&
         a.split_k == b.split_k &&
         a.opts.ws_limit_bytes == b.opts.ws_limit_bytes &&
         a.opts.force_algo == b.opts.force_algo &&
         a.opts.force_inner_algo == b.opts.force_inner_algo &&
         a.opts.force_tile_batch == b.opts.force_tile_batch &&
         a.opts.force_unfold_rows == b.opts.force_unfold_rows &&
         a.opts.force_gemm_config == b.opts.force_gemm_config &&
         a.opts.force_split_k == b.opts.force_split_k;
}

cnhwc_status_t select_impl(const cnhwc_conv_desc_t* desc, const cnhwc_select_opts_t* opts,
                           cnhwc_plan_t* plan) {
  if (!desc || !opts || !plan) return CNHWC_ERR_INVALID_ARGUMENT;
  if (opts->ws_limit_bytes == 0 || opts->force_tile_batch < 0 || opts->force_unfold_rows < 0 ||
      opts->force_gemm_config < 0 || opts->force_split_k < 0)
    return CNHWC_ERR_INVALID_ARGUMENT;
  if (opts->force_algo < CNHWC_ALGO_AUTO || opts->force_algo > CNHWC_ALGO_WINOGRAD_HALF ||
      opts->force_inner_algo < CNHWC_ALGO_AUTO || opts->force_inner_algo > CNHWC_ALGO_UNFOLD_GEMM)
    return CNHWC_ERR_INVALID_ARGUMENT;
  int64_t out[3];
  cnhwc_status_t st = check_desc(*desc, out);
  if (st != CNHWC_OK) return st;
  cnhwc_plan_t p;
  std::memset(&p, 0, sizeof(p));
  if (desc->nd == 2) {
    if (opts->force_inner_algo != CNHWC_ALGO_AUTO) return CNHWC_ERR_INVALID_ARGUMENT;
    st = select_2d(*desc, out, *opts, opts->force_algo, &p);
  } else {
    st = select_3d(*desc, out, *opts, &p);
  }
  if (st != CNHWC_OK) return st;
  p.opts = *opts;
  *plan = p;
  return CNHWC_OK;
}

}  // namespace cnhwc

extern "C" {

int cnhwc_abi_version(void) { return CNHWC_ABI_VERSION; }

const char* cnhwc_status_string(cnhwc_status_t s) {
  switch (s) {
    case CNHWC_OK: return "ok";
    case CNHWC_ERR_INVALID_ARGUMENT: return "invalid argument";
    case CNHWC_ERR_UNSUPPORTED: return "unsupported convolution";
    case CNHWC_ERR_NOT_APPLICABLE: return "forced algorithm not applicable";
    case CNHWC_ERR_BUDGET: return "forced Winograd does not fit the byte budget";
    case CNHWC_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case CNHWC_ERR_PLAN_MISMATCH: return "plan does not match the descriptor";
    case CNHWC_ERR_HIP: return "HIP launch error";
    case CNHWC_ERR_INTERNAL: return "internal error";
  }
  return "unknown status";
}

cnhwc_status_t cnhwc_conv_select(const cnhwc_conv_desc_t* desc, const cnhwc_select_opts_t* opts,
                                 cnhwc_plan_t* plan) {
  return cnhwc::select_impl(desc, opts, plan);
}

cnhwc_status_t cnhwc_winograd_tile_rule(uint64_t ws_limit, uint64_t own_bytes,
                                        uint64_t scratch_per_element, int64_t n,
                                        int64_t rows_per_element, int64_t force_tile,
                                        int64_t* tile_batch, uint64_t* budget_bytes,
                                        int32_t* fallback) {
  if (!tile_batch || !budget_bytes || !fallback || n < 1 || rows_per_element < 1 ||
      scratch_per_element == 0 || force_tile < 0)
    return CNHWC_ERR_INVALID_ARGUMENT;
  cnhwc::tile_rule(ws_limit, own_bytes, scratch_per_element, n, rows_per_element, force_tile,
                   tile_batch, budget_bytes, fallback);
  return CNHWC_OK;
}

}  // extern "C"
