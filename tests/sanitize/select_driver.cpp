// Host sanitizer driver for the planner (select.cpp), built with g++ and
// AddressSanitizer / UndefinedBehaviorSanitizer by tests/test_host_sanitizers.py.
// It feeds the C entry points a seeded mix of valid, extreme and invalid
// descriptors and options and checks the plans it gets back for basic
// consistency; the sanitizers check every access and every integer operation.
#include <cstdint>
#include <cstdio>
#include <random>

#include "cnhwc.h"

namespace cnhwc {
// The resident Winograd GEMM's applicability is defined next to that kernel;
// this host-only build has no GPU code, so it uses the same limits here
// (K = Cs a multiple of 32 and at most 192, O at most 96).
bool wino_gemm_resident_ok(int64_t cs, int64_t o) { return cs % 32 == 0 && cs <= 192 && o <= 96; }
}  // namespace cnhwc

namespace {

template <class T, size_t N>
T pick(std::mt19937_64& g, const T (&v)[N]) {
  return v[g() % N];
}

int check_plan(const cnhwc_conv_desc_t& d, const cnhwc_plan_t& p) {
  if (p.algo < 1 || p.algo > CNHWC_ALGO_WINOGRAD_HALF) return 1;
  if (p.out_d < 1 || p.out_h < 1 || p.out_w < 1) return 2;
  if (p.algo == CNHWC_ALGO_WINOGRAD || p.algo == CNHWC_ALGO_WINOGRAD_HALF ||
      (p.algo == CNHWC_ALGO_SMALL_KD && p.inner_algo == CNHWC_ALGO_WINOGRAD)) {
    const int64_t n = d.nd == 3 && p.algo == CNHWC_ALGO_SMALL_KD ? p.out_d : d.n;
    if (p.tile_batch < 1 || p.tile_batch > n) return 3;
    if (p.n_tiles != (n + p.tile_batch - 1) / p.tile_batch) return 4;
  }
  if (p.split_k < 1) return 5;  // a forced split may go up to the number of K chunks
  return 0;
}

}  // namespace

// The 32-bit span bound of the gathers, on both sides: in + 2 * pad == 2^30
// plans, 2^30 + 1 does not (UNSUPPORTED), on each axis, and likewise C.
int check_span_bound() {
  const int64_t span = int64_t(1) << 30;
  for (int axis = 0; axis < 3; ++axis) {
    for (int over = 0; over < 2; ++over) {
      cnhwc_conv_desc_t d{};
      d.nd = axis == 0 ? 3 : 2;
      d.dtype = CNHWC_F16;
      d.n = d.d = d.h = d.w = d.c = d.o = d.kd = d.kh = d.kw = 1;
      for (int i = 0; i < 3; ++i) { d.stride[i] = 1; d.dil[i] = 1; }
      d.groups = 1;
      int64_t* in = axis == 0 ? &d.d : (axis == 1 ? &d.h : &d.w);
      int64_t* k = axis == 0 ? &d.kd : (axis == 1 ? &d.kh : &d.kw);
      *in = span - 2 + over;
      *k = 3;
      d.pad[axis] = 1;
      cnhwc_select_opts_t o{};
      o.ws_limit_bytes = 288000000000ull;
      o.force_algo = CNHWC_ALGO_IMPLICIT_GEMM;
      cnhwc_plan_t p{};
      const cnhwc_status_t st = cnhwc_conv_select(&d, &o, &p);
      if (st != (over ? CNHWC_ERR_UNSUPPORTED : CNHWC_OK)) return 1 + axis;
    }
  }
  for (int over = 0; over < 2; ++over) {
    cnhwc_conv_desc_t d{};
    d.nd = 2;
    d.dtype = CNHWC_BF16;
    d.n = d.d = d.h = d.w = d.o = d.kd = d.kh = d.kw = 1;
    d.c = span + over;
    for (int i = 0; i < 3; ++i) { d.stride[i] = 1; d.dil[i] = 1; }
    d.groups = 1;
    cnhwc_select_opts_t o{};
    o.ws_limit_bytes = 288000000000ull;
    cnhwc_plan_t p{};
    if (cnhwc_conv_select(&d, &o, &p) != (over ? CNHWC_ERR_UNSUPPORTED : CNHWC_OK)) return 4;
  }
  return 0;
}

int main() {
  if (const int bad = check_span_bound()) {
    std::printf("span bound check %d failed\n", bad);
    return 1;
  }
  std::mt19937_64 g(20261203);
  const int64_t dims[] = {1, 2, 3, 7, 8, 16, 31, 64, 192, 512, 4096, int64_t(1) << 20, int64_t(1) << 31,
                          0, -1, (int64_t(1) << 31) + 1};
  const int64_t small_dims[] = {1, 2, 3, 5, 7, 9, 0, -3};
  const int32_t geo[] = {0, 1, 1, 1, 2, 3, -1, 1 << 20, (1 << 20) + 1};
  const uint64_t limits[] = {0, 1, 1ull << 20, 512ull << 20, 40200000000ull, 288000000000ull,
                             UINT64_MAX};
  const int32_t algos[] = {-1, 0, 1, 2, 3, 4, 5, 6};
  const int32_t cfgs[] = {-1, 0, 1, 3, 4, 10, 11, 13, 14, 15, 20, 99};
  const int64_t tiles[] = {-1, 0, 1, 3, 7, 1 << 30};
  int64_t ok = 0, errors = 0;
  const int64_t good_dims[] = {1, 2, 3, 7, 8, 16, 31, 64, 120, 192, 256, 512, 1024};
  const int64_t good_k[] = {1, 3, 3, 3, 5, 7};
  for (int it = 0; it < 200000; ++it) {
    cnhwc_conv_desc_t d{};
    if (it % 2 == 0) {  // a well-formed descriptor with forced options of every kind
      d.nd = int32_t(2 + g() % 2);
      d.dtype = int32_t(g() % 3);
      d.n = 1 + int64_t(g() % 48);
      d.h = 1 + int64_t(g() % 260);
      d.w = 1 + int64_t(g() % 260);
      d.c = pick(g, good_dims);
      d.o = pick(g, good_dims);
      d.kh = pick(g, good_k);
      d.kw = g() % 4 ? d.kh : pick(g, good_k);
      d.d = d.nd == 3 ? 1 + int64_t(g() % 48) : 1;
      d.kd = d.nd == 3 ? pick(g, good_k) : 1;
      for (int i = 0; i < 3; ++i) {
        d.stride[i] = 1 + int32_t(g() % 4 == 0);
        d.pad[i] = int32_t(g() % 3);
        d.dil[i] = 1 + int32_t(g() % 6 == 0);
      }
      if (d.nd == 2) { d.stride[0] = 1; d.pad[0] = 0; d.dil[0] = 1; }
      d.groups = 1;
      cnhwc_select_opts_t o{};
      o.ws_limit_bytes = g() % 3 ? 288000000000ull : pick(g, limits);
      o.force_algo = g() % 2 ? 0 : int32_t(g() % 6);
      o.force_inner_algo = g() % 8 == 0 ? int32_t(g() % 4) : 0;
      o.force_tile_batch = g() % 4 == 0 ? int64_t(1 + g() % 9) : 0;
      o.force_unfold_rows = g() % 4 == 0 ? int64_t(1 + g() % 5000) : 0;
      o.force_gemm_config = g() % 6 == 0 ? pick(g, cfgs) : 0;
      o.force_split_k = g() % 6 == 0 ? int32_t(g() % 20) : 0;
      cnhwc_plan_t p{};
      const cnhwc_status_t st = cnhwc_conv_select(&d, &o, &p);
      if (st == CNHWC_OK) {
        ++ok;
        const int bad = check_plan(d, p);
        if (bad) {
          std::printf("inconsistent plan (check %d) at iteration %d\n", bad, it);
          return 1;
        }
      } else {
        ++errors;
      }
      continue;
    }
    d.nd = (g() % 8 == 0) ? int32_t(g() % 5) : int32_t(2 + g() % 2);
    d.dtype = int32_t(g() % 4);
    d.n = pick(g, dims) % 65 == 0 ? 1 : pick(g, small_dims) * (g() % 3 == 0 ? 1 : 8);
    if (g() % 16 == 0) d.n = pick(g, dims);
    d.h = g() % 4 == 0 ? pick(g, dims) : int64_t(1 + g() % 300);
    d.w = g() % 4 == 0 ? pick(g, dims) : int64_t(1 + g() % 300);
    d.c = g() % 4 == 0 ? pick(g, dims) : int64_t(1 + g() % 1100);
    d.o = g() % 4 == 0 ? pick(g, dims) : int64_t(1 + g() % 1100);
    d.kh = pick(g, small_dims);
    d.kw = g() % 2 ? d.kh : pick(g, small_dims);
    if (d.nd == 3) {
      d.d = g() % 4 == 0 ? pick(g, dims) : int64_t(1 + g() % 64);
      d.kd = pick(g, small_dims);
    } else {
      d.d = g() % 16 == 0 ? 2 : 1;
      d.kd = 1;
    }
    for (int i = 0; i < 3; ++i) {
      d.stride[i] = g() % 3 ? 1 : pick(g, geo);
      d.pad[i] = g() % 3 ? int32_t(g() % 3) : pick(g, geo);
      d.dil[i] = g() % 3 ? 1 : pick(g, geo);
    }
    if (d.nd == 2) {
      if (g() % 8) { d.stride[0] = 1; d.pad[0] = 0; d.dil[0] = 1; }
    }
    d.groups = g() % 16 == 0 ? int32_t(g() % 3) : 1;
    cnhwc_select_opts_t o{};
    o.ws_limit_bytes = pick(g, limits);
    o.force_algo = pick(g, algos);
    o.force_inner_algo = g() % 4 == 0 ? pick(g, algos) : 0;
    o.force_tile_batch = g() % 4 == 0 ? pick(g, tiles) : 0;
    o.force_unfold_rows = g() % 4 == 0 ? pick(g, tiles) : 0;
    o.force_gemm_config = g() % 4 == 0 ? pick(g, cfgs) : 0;
    o.force_split_k = g() % 4 == 0 ? int32_t(int64_t(g() % 70) - 2) : 0;
    cnhwc_plan_t p{};
    const cnhwc_status_t st = cnhwc_conv_select(&d, &o, &p);
    if (st == CNHWC_OK) {
      ++ok;
      const int bad = check_plan(d, p);
      if (bad) {
        std::printf("inconsistent plan (check %d) at iteration %d\n", bad, it);
        return 1;
      }
      cnhwc_plan_t q{};
      if (cnhwc_conv_select(&d, &o, &q) != CNHWC_OK || q.workspace_bytes != p.workspace_bytes ||
          q.algo != p.algo || q.tile_batch != p.tile_batch || q.kernel_config != p.kernel_config) {
        std::printf("plan not deterministic at iteration %d\n", it);
        return 1;
      }
    } else {
      ++errors;
    }
    (void)cnhwc_status_string(st);
    int64_t tb;
    uint64_t budget;
    int32_t fb;
    (void)cnhwc_winograd_tile_rule(pick(g, limits), pick(g, limits) >> (g() % 64), g() % 1000 == 0 ? 0 : g(),
                                   pick(g, dims), pick(g, dims), pick(g, tiles), &tb, &budget, &fb);
  }
  (void)cnhwc_conv_select(nullptr, nullptr, nullptr);
  (void)cnhwc_status_string(cnhwc_status_t(12345));
  std::printf("select ok: %lld plans, %lld rejected\n", (long long)ok, (long long)errors);
  return 0;
}
