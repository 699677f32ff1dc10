// Internal declarations shared by the planner (select.cpp), the launch
// sequencing (api.cpp) and the gfx950 kernels (*.hip).
#pragma once
#include <cstdint>
#include <cstddef>

#include "cnhwc.h"
#include "wino_f63_api.hpp"

namespace cnhwc {

inline uint64_t dtype_size(int dt) { return dt == CNHWC_F32 ? 4u : 2u; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline uint64_t align_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

// Winograd F(4x4,3x3) for fp16/bf16 (winograd_h.hip): 6x6 input tiles at
// stride 4, 36 tile positions, fp16 transformed operands with power-of-two
// scales, fp32 GEMM results.
constexpr int kWinoHM = 4;
constexpr int kWinoHP = 36;
// Channel stride of its fp16 rows: C rounded up to 32, one K chunk of the
// 256-row GEMM tiles, so a 3D tap's K range starts on a chunk.
inline int64_t wino_h_cs(int64_t c) { return (c + 31) / 32 * 32; }
// Channels per thread of its input transform (4 when C % 4 == 0, 2 when C is
// even): the transform runs cs / vec threads per tile row.
inline int64_t wino_h_vec(int64_t c) { return c % 4 == 0 ? 4 : (c % 2 == 0 ? 2 : 1); }
// Partial maxima per tensor (one per block of the max-|element| pass).
constexpr int32_t kWinoHSlots = 1024;
inline int32_t wino_h_absmax_blocks(int64_t n) {
  const int64_t b = (n / 8 + 1023) / 1024;  // about four 16-byte vectors per thread
  return int32_t(b < 1 ? 1 : (b > kWinoHSlots ? kWinoHSlots : b));
}
// Workspace head: the partial maxima of x and w, then 4 floats of scales.
constexpr uint64_t kWinoHScaleOff = 2ull * kWinoHSlots * 4;
constexpr uint64_t kWinoHHeadBytes = (kWinoHScaleOff + 16 + 255) / 256 * 256;

// ------------------------------------------------------------------ GEMM

// GEMM tile configurations.  Each id fixes the tile shape, the MFMA form and
// the K order, so the bits of an output row depend on (config, K, data) only,
// never on the number of rows or on which launch the row is in.
enum GemmConfig : int32_t {
  kCfgNone = 0,
  // fp32 operands, v_mfma_f32_32x32x2f32, BM=128, BK=32
  kCfgF32_N32 = 1,
  kCfgF32_N64 = 2,
  kCfgF32_N96 = 3,
  kCfgF32_N128 = 4,
  // fp16/bf16 operands, v_mfma_f32_32x32x16_{f16,bf16}, BK=64; BM x BN
  kCfgH_128x64 = 10,
  kCfgH_128x128 = 11,
  kCfgH_256x128 = 12,
  kCfgH_128x256 = 13,
  // direct global -> LDS operand loads (gemm_lds.hip): 256 x 256 at one
  // workgroup per CU, 256 x 128 at two
  kCfgH_256x256 = 14,
  kCfgH_256x128L = 15,
  // 3x3 stride-1 implicit GEMM with the input patch of a 256-pixel block
  // staged in LDS once per 64-channel chunk (gemm_patch.hip): 256 x 256 tiles
  kCfgH_Patch = 16,
  // Winograd tile-position GEMMs: persistent fp32 kernel with U_p resident in LDS
  kCfgWinoResident = 20,
};

// Pick the tile configuration.  fp32: from the output-channel count only (the
// Winograd GEMM's configuration must not depend on the batch or its tiling).
// fp16/bf16: from the GEMM shape (rows M of the whole conv, columns N), by a
// simple occupancy model over the 256 compute units; lds_ok admits the
// 256x256 direct-to-LDS tile.
int32_t pick_gemm_config(int dtype, int64_t m_rows, int64_t n_cols, bool lds_ok);
// The occupancy model's time estimate for one half-precision configuration
// (1e300 for fp32 and for configurations outside the model).
double gemm_config_time(int dtype, int32_t cfg, int64_t m_rows, int64_t n_cols);


// A-operand source.
enum AMode : int32_t {
  kADense = 0,      // A[m][k] = a[m*lda + k]      (lda, K multiples of 16 B)
  kAImplicit = 1,   // A[m][k] gathered from an NHWC image, k = (kh*KW + kw)*C + c
};

struct GemmParams {
  int32_t dtype;         // element type of A, B and the output
  int32_t a_mode;
  int32_t epi;
  int32_t config;
  int64_t M, N, K;       // C[M x N] = A[M x K] * B[N x K]^T
  const void* a;
  int64_t lda;           // dense A row stride (elements)
  // implicit-A geometry (input image [n][h][w][c])
  int64_t h, w, c, oh, ow, kh, kw;
  int32_t sh, sw, ph, pw, dh, dw;
  // native 3D implicit A (input [n][d][h][w][c], k = ((kd*KH + kh)*KW + kw)*C + c);
  // all zero for 2D
  int64_t d, od, kd;
  int32_t sd, pd, dd;
  const void* b;
  int64_t ldb;           // B row stride (elements)
  void* out;             // output rows, row stride ldc (elements of dtype)
  int64_t ldc;
  float* acc;            // fp32 accumulator rows (row stride ldc) for kEpiAcc*
  // batched GEMM (Winograd tile positions): element offsets per batch index
  int64_t batch;
  int64_t stride_a, stride_b, stride_out;
  // split K (batch == 1 only): split s covers k in [s*kchunk, min(K, (s+1)*kchunk))
  // and stores its fp32 partial sums to part + s*M*ldc; a second kernel adds
  // the splits in order 0, 1, ... and applies the epilogue.
  int32_t ksplit;        // 0 or 1: no split
  int64_t kchunk;        // multiple of the configuration's K chunk
  float* part;
  // segmented dense A (256-row tiles only; a_seg_len = 0: none): element
  // (m, k) sits at a[m*lda + k + (k / a_seg_len) * a_seg_jump].  The Winograd
  // depth taps: segment kd reads the rows kd * dd frames further on.
  int64_t a_seg_len;     // multiple of the 32-element K chunk
  int64_t a_seg_jump;
  // K-chunk-major dense operands (256-row tiles, dense A only; 0: row-major).
  // With lda = 32, the 32-element K chunk q of row m sits at
  // a[q * a_kstep + m * 32 + k % 32] (plus the segment jumps), and likewise
  // for B with ldb = 32 and b_kstep: a chunk of 16 consecutive rows is then
  // 1 KB of whole 128-byte lines instead of half of each of 16 lines.
  int64_t a_kstep;
  int64_t b_kstep;
};

int gemm_launch(const GemmParams& p, void* stream);  // returns hipError_t

// Sum of the ksplit partial slices (fixed order) with the epilogue of p.
int splitk_reduce_launch(const GemmParams& p, void* stream);  // returns hipError_t

// Most K splits of one GEMM (each adds an fp32 M x N slice to the workspace).
constexpr int64_t kMaxSplitK = 16;

// K elements per MFMA chunk of a tile configuration (split-K granularity).
inline int64_t gemm_config_bk(int32_t config) {
  return config >= kCfgH_128x64 && config != kCfgH_256x256 && config != kCfgH_256x128L ? 64 : 32;
}

// fp16/bf16 implicit GEMM of a 3x3, stride-1, dilation-1 conv (2D, or 3D with
// any depth geometry) with C % 64 == 0, from input patches staged in LDS
// (kCfgH_Patch).  Row tiles are BH x BW pixel blocks of one output image or
// frame, BH * BW = 256, BW from patch_block_w (the least padded of 8, 16, 32).
inline int64_t patch_block_w(int64_t oh, int64_t ow) {
  int64_t best = 16, best_area = -1;
  const int64_t cand[3] = {16, 32, 8};
  for (int64_t bw : cand) {
    const int64_t bh = 256 / bw;
    const int64_t area = ((oh + bh - 1) / bh) * bh * ((ow + bw - 1) / bw) * bw;
    if (best_area < 0 || area < best_area) { best = bw; best_area = area; }
  }
  return best;
}
inline int64_t patch_row_tiles(int64_t frames, int64_t oh, int64_t ow) {
  const int64_t bw = patch_block_w(oh, ow), bh = 256 / bw;
  return frames * ((oh + bh - 1) / bh) * ((ow + bw - 1) / bw);
}
bool gemm_patch_ok(const GemmParams& p);
int gemm_patch_launch(const GemmParams& p, void* stream);  // returns hipError_t

// fp16/bf16 256 x 256 tile GEMM with direct global -> LDS operand loads.
// Applicable for dense A (lda, ldb, K multiples of 8) and for implicit A with
// C a multiple of 32.
bool gemm_lds_ok(const GemmParams& p);
int gemm_lds_launch(const GemmParams& p, void* stream);  // returns hipError_t



// Half-precision Winograd F(4x4,3x3) (fp16/bf16 x and w).
// partial[t][b] = largest |element| bits of block b of tensor t (0: x of nx
// elements, 1: w of nw).
int wino_h_absmax_launch(int dtype, const void* x, int64_t nx, const void* w, int64_t nw,
                         uint32_t* partial, void* stream);
// U[p][k / 32][o][k % 32] = fp16(G (sw g) G^T)_p for k = kd*cs + c (K-chunk-major),
// g = w[o][kd][kh][kw][c] (KD = kd planes);
// the scales come from the partial maxima, and scales = {sx, sw, a, b} with
// a b = 1/(sx sw) is stored for the transforms that follow.  wm[k*o + oc]:
// bit kh*3 + kw set iff some channel of tap (kh, kw) of slice (oc, k) is nonzero.
int wino_h_filter_launch(int dtype, const void* w, int64_t o, int64_t kd, int64_t c, int64_t cs,
                         const uint32_t* partial, int64_t nx, int64_t nw, float* scales, uint16_t* u,
                         uint32_t* wm, void* stream);
// V[p][r][c] = fp16(sx (B^T d B)_p) over nb elements of dp frames each (frame
// f reads input frame f - pd, zero outside [0, d)); plane stride `plane`.
// tm[r][wino_mask_parts(cs / wino_h_vec(c))]: the parts of tile r's
// nonzero-pixel mask.
int wino_h_input_launch(int dtype, const void* x, int64_t nb, int64_t d, int64_t dp, int32_t pd,
                        int64_t h, int64_t w, int64_t c, int64_t cs, int32_t ph, int32_t pw,
                        int64_t th, int64_t tw, const float* scales, uint16_t* v, int64_t plane,
                        uint64_t* tm, void* stream);
// y = (A^T M A) / (sx sw) per tile and output channel for nimg output images
// (or frames: od per element, whose taps read dp-frame input rows at depth
// dilation dd over kd taps), cropped to [oh, ow].  Outputs with no nonzero
// pixel under a nonzero tap (tm, wm above) take 0.
int wino_h_output_launch(int dtype, const float* m, int64_t plane, int64_t nimg, int64_t oh,
                         int64_t ow, int64_t o, int64_t th, int64_t tw, const float* scales,
                         void* y, const uint64_t* tm, int64_t c, int64_t cs, const uint32_t* wm,
                         int64_t od, int64_t dp, int64_t kd, int64_t dd, void* stream);

// ------------------------------------------------------------- Unfold

// buf[r][k] for output rows m0..m0+rows-1 (k = (kh*KW + kw)*C + c, zero outside
// the image and for k >= K), row stride kp elements.
int unfold_launch(int dtype, const void* x, int64_t h, int64_t w, int64_t c, int64_t oh,
                  int64_t ow, int64_t kh, int64_t kw, int32_t sh, int32_t sw, int32_t ph,
                  int32_t pw, int32_t dh, int32_t dw, int64_t m0, int64_t rows, int64_t kp,
                  void* buf, void* stream);

// Unfold row stride: K rounded up to 16 bytes worth of elements.
inline int64_t unfold_kp(int64_t k, int dtype) {
  const int64_t v = 16 / (int64_t)dtype_size(dtype);
  return (k + v - 1) / v * v;
}

// ------------------------------------------------------------ planner

// Winograd workspace layout for a 2D conv and a tile size.
// Tap masks (uint32 per output channel) follow U; the tile masks
// (wino_mask_parts(cs) uint64 per tile row) follow M.
struct WinoLayout {
  int64_t tiles_h, tiles_w, t, cs, mask_parts;
  uint64_t u_bytes, wm_bytes, v_plane, m_plane;  // plane strides in elements
  uint64_t off_u, off_wm, off_v, off_m, off_tm, total;
};
WinoLayout wino_layout(const cnhwc_conv_desc_t& d2, int64_t oh, int64_t ow, int64_t tile_batch);

// Half-precision Winograd workspace layout (2D: od = 1, depth pad 0; 3D: one
// batch element per tile).  Frames per element dp = D + 2 pd; the GEMM K is
// ku = KD * cs.
// Tap masks (uint32 per (kd, o)) follow U; the tile masks
// (wino_mask_parts(cs / wino_h_vec(c)) uint64 per input tile row) follow M.
struct WinoHLayout {
  int64_t tiles_h, tiles_w, t, cs, dp, ku, mask_parts;
  uint64_t u_bytes, wm_bytes, v_plane, m_plane;  // plane strides in elements
  uint64_t off_u, off_wm, off_v, off_m, off_tm, total;
};
WinoHLayout wino_h_layout(const cnhwc_conv_desc_t& d, int64_t od, int64_t oh, int64_t ow,
                          int64_t tile_batch);

cnhwc_status_t select_impl(const cnhwc_conv_desc_t* desc, const cnhwc_select_opts_t* opts,
                           cnhwc_plan_t* plan);
bool plan_equal(const cnhwc_plan_t& a, const cnhwc_plan_t& b);
cnhwc_conv_desc_t frame_desc(const cnhwc_conv_desc_t& d3, int64_t od);  // 3D -> per-tap 2D

}  // namespace cnhwc
