// Drives every host entry point of libasp on small inputs, valid and
// invalid, so that a build with AddressSanitizer and UndefinedBehaviorSanitizer
// checks the packers' memory accesses and arithmetic.  Exit status 0 when
// every call returned the expected status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "asp.h"

static int failures = 0;
static void expect(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "unexpected result: %s (%s)\n", what, asp_last_error());
    ++failures;
  }
}

int main() {
  std::mt19937 gen(7);
  std::normal_distribution<float> nd(0.0f, 1.0f);
  for (int64_t K : {128, 384}) {
    for (int32_t r : {0, 1, 17, 64}) {
      const int64_t N = 24;
      std::vector<float> w(N * K), s(K), v(K * (r > 0 ? r : 1));
      for (auto& a : w) a = nd(gen);
      for (auto& a : s) a = 0.5f + std::fabs(nd(gen));
      for (auto& a : v) a = nd(gen) / 16.0f;
      size_t cb = 0, sb = 0, wb = 0, pb = 0;
      expect(asp_packed_sizes(N, K, r, &cb, &sb, &wb) == ASP_OK, "packed sizes");
      std::vector<uint8_t> codes(cb), scales(sb);
      std::vector<uint16_t> wv(wb / 2 + 1);
      std::vector<float> pre(N * K);
      expect(asp_pack_weight(N, K, r, w.data(), s.data(), r ? v.data() : nullptr, codes.data(),
                             scales.data(), r ? wv.data() : nullptr, pre.data(), 3) == ASP_OK,
             "pack weight");
      expect(asp_pack_weight_shared(N, K, r, w.data(), s.data(), r ? v.data() : nullptr,
                                    codes.data(), scales.data(), r ? wv.data() : nullptr,
                                    nullptr, 2) == ASP_OK,
             "pack shared weight");
      expect(asp_prep_pack_bytes(K, r, &pb) == ASP_OK, "prep bytes");
      std::vector<uint8_t> prep(pb);
      expect(asp_pack_prep(K, r, s.data(), r ? v.data() : nullptr, prep.data()) == ASP_OK,
             "pack prep");
      expect(asp_quantize_nvfp4_host(w.data(), N, K, codes.data(), scales.data()) == ASP_OK,
             "host quantiser");
      // the SVDQuant-style packer (rank at most 64, K a multiple of 128)
      std::vector<float> g(K * K);
      expect(asp_svdq_gram(N, K, w.data(), s.data(), g.data()) == ASP_OK, "svdq gram");
      size_t c2 = 0, s2 = 0, l2 = 0, p2 = 0;
      expect(asp_svdq_packed_sizes(N, K, r, &c2, &s2, &l2, &p2) == ASP_OK, "svdq sizes");
      std::vector<uint8_t> c2v(c2), p2v(p2);
      std::vector<uint16_t> s2v(s2 / 2), l2v(l2 / 2 + 1);
      expect(asp_svdq_pack_weight(N, K, r, w.data(), s.data(), r ? v.data() : nullptr,
                                  c2v.data(), s2v.data(), r ? l2v.data() : nullptr,
                                  p2v.data()) == ASP_OK,
             "svdq pack");
    }
  }
  // invalid arguments are rejected before any buffer is touched
  size_t a = 0, b = 0, c = 0;
  expect(asp_packed_sizes(8, 100, 0, &a, &b, &c) == ASP_ERR_SHAPE, "K not a multiple of 128");
  expect(asp_packed_sizes(8, 128, 65, &a, &b, &c) == ASP_ERR_SHAPE, "rank above 64");
  expect(asp_pack_weight(8, 128, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                         1) == ASP_ERR_ARG,
         "null weight");
  std::vector<float> w(8 * 128, 1.0f), s(128, 1.0f);
  s[3] = 0.0f;
  std::vector<uint8_t> codes(8 * 64), scales(8 * 8);
  expect(asp_pack_weight(8, 128, 0, w.data(), s.data(), nullptr, codes.data(), scales.data(),
                         nullptr, nullptr, 1) == ASP_ERR_ARG,
         "zero smoothing entry");
  expect(asp_quantize_nvfp4_host(w.data(), 8, 100, codes.data(), scales.data()) != ASP_OK,
         "quantiser: cols not a multiple of 16");
  std::printf("%s\n", failures ? "FAILED" : "host entry points ok");
  return failures ? 1 : 0;
}
