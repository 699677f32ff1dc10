// Reference oracle for channels-last convolution forward -- TEST INFRASTRUCTURE ONLY.
//
// Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
// load or run this code.  The product path (the HIP library) never calls it and
// the two share no source.
//
// What it computes (the plain definition, no fast algorithm):
//   cross-correlation over NDHWC input and O,KD,KH,KW,C weights with zero padding,
//
//   y[n,od,oh,ow,o] = sum_{kd,kh,kw,c} X(n, od*sd - pd + kd*dd,
//                                          oh*sh - ph + kh*dh,
//                                          ow*sw - pw + kw*dw, c) * w[o,kd,kh,kw,c]
//
//   where X(...) is the input value inside the image and 0 outside.  2D is the
//   special case D = KD = 1, sd = dd = 1, pd = 0.  It also returns
//   den[...] = the same sum over |X| * |w|, the scale the acceptance test uses.
//
// The pages this follows: MLX PR "Bound winograd conv2d working set by tiling the
// batch" (conv2d on NHWC, checked against a CPU convolution in its Testing and
// review sections), MLX PR "Use the explicit gemm for wide convs on neural
// accelerators" (Verified: CPU reference over filter/stride/padding/dilation
// grids) and MLX PR "Decompose small kernel-depth 3D convs into 2D convs"
// (Change: frames [OD,H,W,C], weight depth slice [O,KH,KW,C]; Results: CPU
// reference).  None of the pages writes the formula down; the one above is the
// textbook definition of the correlation that deep-learning convolutions compute.
//
// Arithmetic: inputs arrive as float32 holding the exact values the GPU sees
// (fp16/bf16 values widen exactly); every product and sum is in fp64.  No output
// rounding.  Threads: std::thread over output pixels.
#include <cstdint>
#include <cmath>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

struct Geo {
  int64_t n, d, h, w, c, o, kd, kh, kw;
  int64_t sd, sh, sw, pd, ph, pw, dd, dh, dw;
  int64_t od, oh, ow;
};

// Output extent of one spatial dim: floor((in + 2p - dil*(k-1) - 1)/s) + 1.
int64_t out_extent(int64_t in, int64_t k, int64_t s, int64_t p, int64_t dil) {
  const int64_t span = in + 2 * p - dil * (k - 1) - 1;
  if (span < 0) return 0;
  return span / s + 1;
}

// One output pixel m (flattened n,od,oh,ow), all O channels.
void one_pixel(const Geo& g, const float* x, const float* w, int64_t m,
               double* yrow, double* drow) {
  int64_t t = m;
  const int64_t ow = t % g.ow; t /= g.ow;
  const int64_t oh = t % g.oh; t /= g.oh;
  const int64_t od = t % g.od; t /= g.od;
  const int64_t n = t;
  for (int64_t o = 0; o < g.o; ++o) {
    double acc = 0.0, den = 0.0;
    for (int64_t a = 0; a < g.kd; ++a) {
      const int64_t id = od * g.sd - g.pd + a * g.dd;
      if (id < 0 || id >= g.d) continue;
      for (int64_t b = 0; b < g.kh; ++b) {
        const int64_t ih = oh * g.sh - g.ph + b * g.dh;
        if (ih < 0 || ih >= g.h) continue;
        for (int64_t e = 0; e < g.kw; ++e) {
          const int64_t iw = ow * g.sw - g.pw + e * g.dw;
          if (iw < 0 || iw >= g.w) continue;
          const float* xp = x + (((n * g.d + id) * g.h + ih) * g.w + iw) * g.c;
          const float* wp = w + (((o * g.kd + a) * g.kh + b) * g.kw + e) * g.c;
          for (int64_t c = 0; c < g.c; ++c) {
            const double xv = (double)xp[c], wv = (double)wp[c];
            acc += xv * wv;
            den += std::fabs(xv) * std::fabs(wv);
          }
        }
      }
    }
    yrow[o] = acc;
    if (drow) drow[o] = den;
  }
}

}  // namespace

extern "C" {

// Output extents; returns 0 on success, -1 if any extent is < 1 or an argument is invalid.
int oracle_out_shape(const int64_t* in3, const int64_t* k3, const int64_t* s3,
                     const int64_t* p3, const int64_t* d3, int64_t* out3) {
  for (int i = 0; i < 3; ++i) {
    if (in3[i] < 1 || k3[i] < 1 || s3[i] < 1 || p3[i] < 0 || d3[i] < 1) return -1;
    out3[i] = out_extent(in3[i], k3[i], s3[i], p3[i], d3[i]);
    if (out3[i] < 1) return -1;
  }
  return 0;
}

// Direct convolution.  dims = {n, d, h, w, c, o, kd, kh, kw};
// s3/p3/d3 = {depth, height, width} stride / padding / dilation.
// rows: flattened output-pixel indices to compute (NULL -> all, in order);
// y, den: [n_rows][o] fp64 (den may be NULL).  threads <= 0 -> hardware count.
// Returns 0, or -1 for an invalid geometry or a row index out of range.
int oracle_conv_fwd(const float* x, const float* w, const int64_t* dims,
                    const int64_t* s3, const int64_t* p3, const int64_t* d3,
                    const int64_t* rows, int64_t n_rows, double* y, double* den,
                    int threads) {
  Geo g{dims[0], dims[1], dims[2], dims[3], dims[4], dims[5], dims[6], dims[7], dims[8],
        s3[0], s3[1], s3[2], p3[0], p3[1], p3[2], d3[0], d3[1], d3[2], 0, 0, 0};
  for (int i = 0; i < 9; ++i) if (dims[i] < 1) return -1;
  const int64_t in3[3] = {g.d, g.h, g.w}, k3[3] = {g.kd, g.kh, g.kw};
  int64_t o3[3];
  if (oracle_out_shape(in3, k3, s3, p3, d3, o3) != 0) return -1;
  g.od = o3[0]; g.oh = o3[1]; g.ow = o3[2];
  const int64_t total = g.n * g.od * g.oh * g.ow;
  const int64_t count = rows ? n_rows : total;
  if (rows)
    for (int64_t i = 0; i < count; ++i)
      if (rows[i] < 0 || rows[i] >= total) return -1;
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  threads = (int)std::min<int64_t>(threads, std::max<int64_t>(1, count));
  auto work = [&](int64_t lo, int64_t hi) {
    for (int64_t i = lo; i < hi; ++i) {
      const int64_t m = rows ? rows[i] : i;
      one_pixel(g, x, w, m, y + i * g.o, den ? den + i * g.o : nullptr);
    }
  };
  std::vector<std::thread> pool;
  const int64_t per = (count + threads - 1) / threads;
  for (int t = 0; t < threads; ++t) {
    const int64_t lo = t * per, hi = std::min(count, lo + per);
    if (lo >= hi) break;
    pool.emplace_back(work, lo, hi);
  }
  for (auto& th : pool) th.join();
  return 0;
}

}  // extern "C"
