// Host sanitizer driver for the oracle (oracle/oracle.cpp), built with g++ and
// AddressSanitizer / UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py:
// small 2D and 3D convolutions over every geometry knob, full and with row
// subsets, and invalid arguments that must be rejected.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

extern "C" int oracle_out_shape(const int64_t* in3, const int64_t* k3, const int64_t* s3,
                                const int64_t* p3, const int64_t* d3, int64_t* out3);
extern "C" int oracle_conv_fwd(const float* x, const float* w, const int64_t* dims, const int64_t* s3,
                               const int64_t* p3, const int64_t* d3, const int64_t* rows, int64_t n_rows,
                               double* y, double* den, int threads);

int main() {
  std::mt19937_64 g(7);
  std::uniform_real_distribution<float> u(-1.0f, 1.0f);
  int runs = 0;
  for (int it = 0; it < 300; ++it) {
    const bool three = it % 3 == 0;
    int64_t dims[9] = {int64_t(1 + g() % 2), three ? int64_t(1 + g() % 5) : 1, int64_t(1 + g() % 9),
                       int64_t(1 + g() % 9), int64_t(1 + g() % 5), int64_t(1 + g() % 4),
                       three ? int64_t(1 + g() % 3) : 1, int64_t(1 + g() % 4), int64_t(1 + g() % 4)};
    int64_t s3[3] = {three ? int64_t(1 + g() % 2) : 1, int64_t(1 + g() % 3), int64_t(1 + g() % 3)};
    int64_t p3[3] = {three ? int64_t(g() % 2) : 0, int64_t(g() % 3), int64_t(g() % 3)};
    int64_t d3[3] = {three ? int64_t(1 + g() % 2) : 1, int64_t(1 + g() % 2), int64_t(1 + g() % 2)};
    const int64_t in3[3] = {dims[1], dims[2], dims[3]}, k3[3] = {dims[6], dims[7], dims[8]};
    int64_t o3[3];
    if (oracle_out_shape(in3, k3, s3, p3, d3, o3) != 0) {
      std::vector<float> x(1), w(1);
      std::vector<double> y(dims[5]);
      if (oracle_conv_fwd(x.data(), w.data(), dims, s3, p3, d3, nullptr, 0, y.data(), nullptr, 2) != -1) {
        std::printf("invalid geometry accepted at %d\n", it);
        return 1;
      }
      continue;
    }
    const int64_t nx = dims[0] * dims[1] * dims[2] * dims[3] * dims[4];
    const int64_t nw = dims[5] * dims[6] * dims[7] * dims[8] * dims[4];
    const int64_t total = dims[0] * o3[0] * o3[1] * o3[2];
    std::vector<float> x(nx), w(nw);
    for (auto& v : x) v = u(g);
    for (auto& v : w) v = u(g);
    std::vector<double> y(total * dims[5]), den(total * dims[5]);
    if (oracle_conv_fwd(x.data(), w.data(), dims, s3, p3, d3, nullptr, 0, y.data(), den.data(),
                        int(1 + g() % 3)) != 0) {
      std::printf("valid conv rejected at %d\n", it);
      return 1;
    }
    std::vector<int64_t> rows;
    for (int64_t r = total - 1; r >= 0; r -= 1 + int64_t(g() % 3)) rows.push_back(r);
    std::vector<double> ys(rows.size() * dims[5]);
    if (oracle_conv_fwd(x.data(), w.data(), dims, s3, p3, d3, rows.data(), int64_t(rows.size()), ys.data(),
                        nullptr, 2) != 0) {
      std::printf("row subset rejected at %d\n", it);
      return 1;
    }
    for (size_t i = 0; i < rows.size(); ++i)
      for (int64_t o = 0; o < dims[5]; ++o)
        if (ys[i * dims[5] + o] != y[rows[i] * dims[5] + o]) {
          std::printf("row subset differs at %d\n", it);
          return 1;
        }
    const int64_t bad[1] = {total};
    if (oracle_conv_fwd(x.data(), w.data(), dims, s3, p3, d3, bad, 1, ys.data(), nullptr, 1) != -1) {
      std::printf("out-of-range row accepted at %d\n", it);
      return 1;
    }
    ++runs;
  }
  std::printf("oracle ok: %d convolutions\n", runs);
  return 0;
}
