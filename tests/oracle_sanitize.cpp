// Memory and undefined-behaviour check of the C++ oracle: every exported function on small seeded
// inputs, built with AddressSanitizer and UBSan (single-threaded: no OpenMP) by
// test_oracle_sanitized.py. Exits nonzero on a broken invariant; the sanitizers abort on any report.
#include "../oracle/oracle.cpp"

#include <stdio.h>
#include <stdlib.h>

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double urand() {  // xorshift64*, uniform in [0, 1)
  st ^= st >> 12; st ^= st << 25; st ^= st >> 27;
  return (double)((st * 2685821657736338717ull) >> 11) * (1.0 / 9007199254740992.0);
}
static float nrand() { return (float)((urand() + urand() + urand() + urand() - 2.0) * 1.7); }

#define CHECK(c) do { if (!(c)) { fprintf(stderr, "failed: %s (line %d)\n", #c, __LINE__); return 1; } } while (0)

int main() {
  // codecs: every code decodes, encode(decode(c)) == c for the canonical codes
  for (int c = 0; c < 16; c++) {
    const double v = orc_e2m1_decode((uint8_t)c);
    if (c != 8) CHECK(orc_e2m1_encode((float)v) == c);
  }
  for (int c = 0; c < 127; c++) CHECK(orc_e4m3_encode((float)orc_e4m3_decode((uint8_t)c)) == c);
  CHECK(orc_e4m3_encode(1e30f) == 0x7E);
  // quantizer: one row per 32-block scale, zero rows give zero codes
  const int R = 5, C = 96;
  std::vector<float> x(R * C);
  for (auto& v : x) v = nrand();
  for (int c = 0; c < C; c++) x[3 * C + c] = 0.0f;
  const float g = orc_global_scale(orc_amax(x.data(), (int64_t)x.size()));
  std::vector<uint8_t> q(R * C / 2), s(R * C / 32);
  CHECK(orc_quantize_rows(x.data(), R, C, C, &g, nullptr, q.data(), s.data()) == 0);
  for (int c = 0; c < C / 2; c++) CHECK(q[3 * C / 2 + c] == 0);
  std::vector<double> dq(R * C);
  orc_dequant_codes(q.data(), s.data(), R, C, dq.data());
  // weights: prune, compress (pack inside), unpack round trip
  const int E = 3, N = 32, K = 64;
  std::vector<float> w(E * N * K), pr(E * N * K);
  for (auto& v : w) v = nrand() * 0.02f;
  orc_prune_paired48(w.data(), (int64_t)E * N, K, pr.data());
  std::vector<uint8_t> pk(E * N * K / 4), mk(E * N * K / 16), sc(E * N * K / 32);
  std::vector<float> gs(E);
  CHECK(orc_compress_weights(w.data(), E, N, K, pk.data(), mk.data(), sc.data(), gs.data()) == 0);
  for (size_t i = 0; i < mk.size(); i++) {
    const int lo = __builtin_popcount(mk[i] & 15), hi = __builtin_popcount(mk[i] >> 4);
    CHECK(lo == 2 && hi == 2);
  }
  std::vector<uint8_t> dense(E * N * K / 2), pk2(pk.size()), mk2(mk.size());
  CHECK(orc_unpack_pair_bitmask(pk.data(), mk.data(), (int64_t)E * N, K, dense.data()) == 0);
  CHECK(orc_pack_pair_bitmask(dense.data(), (int64_t)E * N, K, pk2.data(), mk2.data()) == 0);
  CHECK(memcmp(pk.data(), pk2.data(), pk.size()) == 0 && memcmp(mk.data(), mk2.data(), mk.size()) == 0);
  // routing, dispatch quantization, grouped GEMM (all rows and a row list), SwiGLU, combine
  const int T = 7, k = 2;
  std::vector<int32_t> ids(T * k);
  for (int t = 0; t < T; t++) {
    ids[2 * t] = (int32_t)(urand() * E);
    ids[2 * t + 1] = (ids[2 * t] + 1 + (int32_t)(urand() * (E - 1))) % E;
  }
  std::vector<int32_t> cnt(E), off(E + 1), sorted(T * k), pos(T * k);
  CHECK(orc_route(ids.data(), T, k, E, cnt.data(), off.data(), sorted.data(), pos.data()) == 0);
  CHECK(off[E] == T * k);
  std::vector<float> xa(T * K);
  for (auto& v : xa) v = nrand();
  std::vector<float> ga(E, orc_global_scale(orc_amax(xa.data(), (int64_t)xa.size())));
  std::vector<uint8_t> qa(T * k * K / 2), sa(T * k * K / 32);
  CHECK(orc_dispatch_quantize(xa.data(), T, K, sorted.data(), k, off.data(), E, ga.data(), qa.data(), sa.data()) == 0);
  std::vector<double> y((size_t)T * k * N), y2((size_t)T * k * N);
  CHECK(orc_grouped_gemm(pk.data(), mk.data(), sc.data(), gs.data(), E, N, K, qa.data(), sa.data(), ga.data(),
                         off.data(), nullptr, 0, y.data()) == 0);
  std::vector<int64_t> rl = {0, 3, (int64_t)T * k - 1};
  CHECK(orc_grouped_gemm(pk.data(), mk.data(), sc.data(), gs.data(), E, N, K, qa.data(), sa.data(), ga.data(),
                         off.data(), rl.data(), (int64_t)rl.size(), y2.data()) == 0);
  std::vector<double> h((size_t)T * k * N / 2);
  orc_swiglu(y.data(), (int64_t)T * k, N / 2, h.data());
  std::vector<float> tw(T * k, 0.5f);
  std::vector<double> out((size_t)T * N);
  orc_combine(y.data(), N, pos.data(), tw.data(), T, k, out.data());
  printf("oracle sanitizer run ok\n");
  return 0;
}
