// Declarations of the fp32-intermediate Winograd F(6x6,3x3) kernels
// (winograd.hip: filter, input and output transforms; wino_gemm.hip: the
// resident tile-position GEMM) and the constants they share with the rest of
// the library.  internal.hpp includes this header; those two kernel sources
// include only this one.
#pragma once
#include <cstdint>

#include "cnhwc.h"

namespace cnhwc {

// Winograd F(6x6,3x3): 8x8 input tiles at stride 6, 64 tile positions.
constexpr int kWinoM = 6;
constexpr int kWinoT = 8;
constexpr int kWinoP = 64;

// Channel stride of the transformed input/filter rows: C rounded up to a
// multiple of 8 so every row is 32-byte aligned (pad channels are zero).
inline int64_t wino_cs(int64_t c) { return (c + 7) / 8 * 8; }

// Epilogue: how a GEMM / output-transform result r is written.
enum EpiMode : int32_t {
  kEpiStore = 0,     // y = round(r)
  kEpiAccFirst = 1,  // acc = r                (fp32)
  kEpiAccMid = 2,    // acc = acc + r          (fp32)
  kEpiAccLast = 3,   // y = round(acc + r)
};

// Zero-window masks (both Winograd forms; wino_mask.hpp holds the device
// side).  The input transform writes each tile's nonzero-pixel mask in parts:
// when the g threads of one tile row fill whole wavefronts (g % 64 == 0) each
// wavefront writes one part, else each workgroup of 256 threads holding some
// of them.  Parts per row (the row stride of the mask array, in uint64):
inline int64_t wino_mask_parts(int64_t g) { return g % 64 == 0 ? g / 64 : (g - 1) / 256 + 2; }

// U[p][o][c] = (G g G^T)_p, g = w[o*ldo + (kh*3 + kw)*C + c]; zero for c >= C.
// wm[o]: bit kh*3 + kw set iff some channel of tap (kh, kw) of filter o is nonzero.
int wino_filter_launch(int dtype, const void* w, int64_t ldo, int64_t o, int64_t c,
                       int64_t cs, float* u, uint32_t* wm, void* stream);

// V[p][r][c] = (B^T d B)_p for tile r of nb images [nb][h][w][c] (8x8 tiles at
// stride 6 starting at (-ph, -pw), zero outside); plane stride `plane`.
// tm[r][wino_mask_parts(cs)]: the parts of tile r's nonzero-pixel mask.
int wino_input_launch(int dtype, const void* x, int64_t nb, int64_t h, int64_t w, int64_t c,
                      int64_t cs, int32_t ph, int32_t pw, int64_t tiles_h, int64_t tiles_w,
                      float* v, int64_t plane, uint64_t* tm, void* stream);

// Y = A^T M A per tile and output channel, cropped to [oh, ow]; epilogue mode.
// Outputs with no nonzero pixel under a nonzero tap (tm, wm above) take 0.
int wino_output_launch(int dtype, const float* m, int64_t plane, int64_t nb, int64_t oh,
                       int64_t ow, int64_t o, int64_t tiles_h, int64_t tiles_w, void* y,
                       float* acc, int32_t epi, const uint64_t* tm, int64_t cs,
                       const uint32_t* wm, void* stream);

// Persistent Winograd GEMM (all 64 positions): M_p[rows][o] = V_p[rows][cs] * U_p[o][cs]^T.
// Applicable when U_p fits in LDS (cs <= 192, o <= 96).
bool wino_gemm_resident_ok(int64_t cs, int64_t o);
int wino_gemm_resident_launch(const float* v, const float* u, float* m, int64_t rows, int64_t o,
                              int64_t cs, int64_t v_plane, int64_t m_plane, void* stream);

}  // namespace cnhwc
