// Driver for the sanitizer build of the C++ reference loops.
//
// test_oracle_sanitizers.py compiles this file together with
// oracle/moe_oracle_ref.cpp under AddressSanitizer and UndefinedBehavior-
// Sanitizer and runs it: every entry point is called on tiny inputs,
// including the degenerate ones (no tokens, no rows, indices outside
// [0, E), rejected group configurations), so that an out-of-bounds access,
// a null pointer handed to a library routine or a signed overflow in the
// loops stops the run.  The checks below are invariants that hold whatever
// the arithmetic: distinct in-range indices, gates that sum to one, a
// permutation that lists every valid pair once.  Exit status 0 = all held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

extern "C" {
void oracle_set_threads(int32_t n);
int32_t oracle_threads(void);
void oracle_decode_bf16(const uint16_t* src, int64_t n, double* dst);
void oracle_decode_e4m3(const uint8_t* src, int64_t n, double* dst);
void oracle_router_logits(const double* x, const double* w_r, const float* router_bias, int64_t S, int32_t d,
                          int32_t E, float* logits);
int32_t oracle_route(const float* logits, const float* select_bias, int64_t S, int32_t E, int32_t K,
                     int32_t n_groups, int32_t topk_groups, int32_t renormalize, double temperature,
                     int32_t* topk_idx, double* topk_gate);
void oracle_permute(const int32_t* topk_idx, int64_t S, int32_t K, int32_t E, int32_t tile_m, int32_t* counts,
                    int32_t* offsets, int32_t* perm, int32_t* inv_perm);
void oracle_dense_ffn(const double* x, int64_t n, int32_t d, int32_t d_ff, const double* w1, const double* b1,
                      const double* w2, const double* b2, double* out);
int32_t oracle_layer_forward(const double* x, const double* w_r, const float* router_bias,
                             const float* select_bias, const double* W1, const double* b1, const double* W2,
                             const double* b2, int64_t S, int32_t d, int32_t d_ff, int32_t E, int32_t K,
                             int32_t n_groups, int32_t topk_groups, int32_t renormalize, double temperature,
                             const float* logits_in, double* y, int32_t* topk_idx_out, double* topk_gate_out);
}

namespace {

int failures = 0;

void check(bool ok, const char* what) {
  if (!ok) {
    std::fprintf(stderr, "FAILED: %s\n", what);
    ++failures;
  }
}

// splitmix64: a fixed, seeded stream of test values.
struct Rng {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
  }
  double uniform() { return (double)(next() >> 11) * (1.0 / 9007199254740992.0); }  // [0, 1)
  double sym() { return 2.0 * uniform() - 1.0; }
};

std::vector<double> randd(Rng& r, size_t n, double scale) {
  std::vector<double> v(n);
  for (auto& a : v) a = scale * r.sym();
  return v;
}

std::vector<float> randf(Rng& r, size_t n, double scale) {
  std::vector<float> v(n);
  for (auto& a : v) a = (float)(scale * r.sym());
  return v;
}

void test_decoders() {
  std::vector<uint16_t> b(65536);
  for (int i = 0; i < 65536; ++i) b[i] = (uint16_t)i;
  std::vector<double> out(65536);
  oracle_decode_bf16(b.data(), 65536, out.data());
  int bad = 0;
  for (int i = 0; i < 65536; ++i) {
    const uint32_t w = (uint32_t)i << 16;
    float f;
    std::memcpy(&f, &w, 4);
    if (!(std::isnan(f) ? std::isnan(out[i]) : out[i] == (double)f)) ++bad;
  }
  check(bad == 0, "bf16 decode is the upper half of a binary32 word");
  std::vector<uint8_t> c(256);
  for (int i = 0; i < 256; ++i) c[i] = (uint8_t)i;
  std::vector<double> e(256);
  oracle_decode_e4m3(c.data(), 256, e.data());
  int nans = 0;
  for (int i = 0; i < 256; ++i) nans += std::isnan(e[i]) ? 1 : 0;
  check(nans == 2 && std::isnan(e[0x7f]) && std::isnan(e[0xff]), "e4m3: exactly two NaN codes");
  check(e[0x7e] == 448.0 && e[0xfe] == -448.0, "e4m3: largest finite is 448");
  check(e[0x01] == std::ldexp(1.0, -9) && e[0x08] == std::ldexp(1.0, -6), "e4m3: subnormal and normal ends");
  for (int i = 1; i < 0x7f; ++i) check(e[i] > e[i - 1], "e4m3: positive codes increase");
  oracle_decode_bf16(b.data(), 0, out.data());
  oracle_decode_e4m3(c.data(), 0, e.data());
}

void test_router_logits(Rng& r) {
  const int64_t S = 5;
  const int32_t d = 7, E = 8;
  auto x = randd(r, S * d, 1.0), w = randd(r, (size_t)E * d, 0.5);
  auto bias = randf(r, E, 0.1);
  std::vector<float> l0(S * E), l1(S * E);
  oracle_router_logits(x.data(), w.data(), nullptr, S, d, E, l0.data());
  oracle_router_logits(x.data(), w.data(), bias.data(), S, d, E, l1.data());
  for (int64_t i = 0; i < S * E; ++i) check(std::isfinite(l0[i]) && std::isfinite(l1[i]), "finite scores");
  oracle_router_logits(x.data(), w.data(), nullptr, 0, d, E, l0.data());
}

// Indices distinct and in [0, E); with groups, inside at most topk_groups
// groups; gates positive and summing to one over the K chosen (renormalised)
// or to at most one (full-softmax probabilities).
void check_route(const std::vector<int32_t>& idx, const std::vector<double>& gate, int64_t S, int32_t E,
                 int32_t K, int32_t G, int32_t topk_groups, int32_t renorm) {
  const int32_t m = E / G;
  for (int64_t t = 0; t < S; ++t) {
    std::vector<char> seen(E, 0), grp(G, 0);
    double sum = 0.0;
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = idx[t * K + k];
      check(e >= 0 && e < E, "route: index in range");
      if (e < 0 || e >= E) continue;
      check(!seen[e], "route: indices distinct");
      seen[e] = 1;
      grp[e / m] = 1;
      check(gate[t * K + k] > 0.0, "route: gates positive");
      sum += gate[t * K + k];
    }
    int ng = 0;
    for (int32_t g = 0; g < G; ++g) ng += grp[g];
    check(ng <= topk_groups, "route: experts from the kept groups only");
    if (renorm)
      check(std::fabs(sum - 1.0) < 1e-12, "route: renormalised gates sum to one");
    else
      check(sum <= 1.0 + 1e-12, "route: softmax gates sum to at most one");
  }
}

void test_route(Rng& r) {
  struct Cfg {
    int32_t E, K, G, TG, renorm;
    double temp;
  };
  const Cfg cfgs[] = {{8, 2, 1, 1, 1, 1.0}, {8, 8, 1, 1, 0, 0.5}, {1, 1, 1, 1, 1, 1.0},
                      {16, 3, 4, 2, 1, 1.0}, {16, 8, 4, 2, 0, 2.0}, {32, 4, 8, 8, 1, 1.0},
                      {64, 8, 8, 4, 1, 0.7}};
  const int64_t S = 9;
  for (const Cfg& c : cfgs) {
    auto l = randf(r, S * c.E, 3.0);
    auto sb = randf(r, c.E, 0.5);
    std::vector<int32_t> idx(S * c.K);
    std::vector<double> gate(S * c.K);
    for (int with_bias = 0; with_bias < 2; ++with_bias) {
      const int32_t rc = oracle_route(l.data(), with_bias ? sb.data() : nullptr, S, c.E, c.K, c.G, c.TG, c.renorm,
                                      c.temp, idx.data(), gate.data());
      check(rc == 0, "route: valid configuration accepted");
      check_route(idx, gate, S, c.E, c.K, c.G, c.TG, c.renorm);
    }
  }
  // ties: equal keys go to the lower index
  std::vector<float> flat(3 * 8, 0.25f);
  std::vector<int32_t> idx(3 * 4);
  std::vector<double> gate(3 * 4);
  check(oracle_route(flat.data(), nullptr, 3, 8, 4, 1, 1, 1, 1.0, idx.data(), gate.data()) == 0, "route: ties");
  for (int t = 0; t < 3; ++t)
    for (int k = 0; k < 4; ++k) check(idx[t * 4 + k] == k && gate[t * 4 + k] == 0.25, "route: ties by index");
  // rejected configurations never write outside the outputs
  const Cfg bad[] = {{8, 0, 1, 1, 1, 1.0},  {8, 9, 1, 1, 1, 1.0},  {12, 2, 4, 2, 1, 1.0},
                     {16, 2, 4, 0, 1, 1.0}, {16, 2, 4, 5, 1, 1.0}, {16, 9, 4, 2, 1, 1.0},
                     {10, 2, 3, 1, 1, 1.0}};
  for (const Cfg& c : bad) {
    auto l = randf(r, 2 * c.E, 1.0);
    std::vector<int32_t> i2(2 * 16, 7);
    std::vector<double> g2(2 * 16, 7.0);
    check(oracle_route(l.data(), nullptr, 2, c.E, c.K, c.G, c.TG, c.renorm, c.temp, i2.data(), g2.data()) == -1,
          "route: invalid configuration rejected");
  }
  auto l = randf(r, 8, 1.0);
  check(oracle_route(l.data(), nullptr, 0, 8, 2, 1, 1, 1, 1.0, idx.data(), gate.data()) == 0, "route: no tokens");
}

void test_permute(Rng& r) {
  const int32_t E = 6;
  for (int32_t tile_m : {1, 4, 16}) {
    for (int64_t S : {0, 1, 7, 33}) {
      const int32_t K = 3;
      std::vector<int32_t> idx(S * K);
      for (auto& e : idx) e = (int32_t)(r.next() % (E + 2)) - 1;  // includes -1 and E: dropped
      std::vector<int32_t> counts(E), offsets(E + 1), perm(S * K + 1), inv(S * K + 1);
      oracle_permute(idx.data(), S, K, E, tile_m, counts.data(), offsets.data(), perm.data(), inv.data());
      int64_t valid = 0;
      for (int64_t p = 0; p < S * K; ++p) valid += (idx[p] >= 0 && idx[p] < E) ? 1 : 0;
      int64_t total = 0;
      for (int32_t e = 0; e < E; ++e) {
        total += counts[e];
        check(offsets[e] % tile_m == 0, "permute: offsets aligned to the tile");
        check(offsets[e + 1] - offsets[e] >= counts[e], "permute: room for the expert's rows");
      }
      check(total == valid, "permute: counts cover the valid pairs");
      std::vector<char> hit(S * K, 0);
      for (int64_t i = 0; i < valid; ++i) {
        const int32_t p = perm[i];
        check(p >= 0 && p < S * K && !hit[p], "permute: perm lists each valid pair once");
        if (p >= 0 && p < S * K) hit[p] = 1;
      }
      for (int64_t p = 0; p < S * K; ++p) {
        const int32_t e = idx[p];
        if (e < 0 || e >= E)
          check(inv[p] == -1, "permute: dropped pair has no row");
        else
          check(inv[p] >= offsets[e] && inv[p] < offsets[e] + counts[e], "permute: row inside its expert");
      }
    }
  }
}

void test_dense_ffn(Rng& r) {
  const int32_t d = 5, d_ff = 11;
  auto x = randd(r, 3 * d, 1.0), w1 = randd(r, (size_t)d_ff * d, 0.5), b1 = randd(r, d_ff, 0.1);
  auto w2 = randd(r, (size_t)d * d_ff, 0.5), b2 = randd(r, d, 0.1);
  std::vector<double> out(3 * d);
  oracle_dense_ffn(x.data(), 3, d, d_ff, w1.data(), b1.data(), w2.data(), b2.data(), out.data());
  for (double v : out) check(std::isfinite(v), "ffn: finite outputs");
  oracle_dense_ffn(x.data(), 0, d, d_ff, w1.data(), b1.data(), w2.data(), b2.data(), out.data());
}

void test_layer(Rng& r) {
  struct Cfg {
    int64_t S;
    int32_t d, d_ff, E, K, G, TG, renorm;
  };
  const Cfg cfgs[] = {{6, 8, 12, 4, 2, 1, 1, 1}, {5, 6, 10, 16, 3, 4, 2, 0}, {0, 8, 12, 4, 2, 1, 1, 1},
                      {3, 4, 6, 1, 1, 1, 1, 1}};
  for (const Cfg& c : cfgs) {
    auto x = randd(r, c.S * c.d, 1.0), wr = randd(r, (size_t)c.E * c.d, 0.5);
    auto W1 = randd(r, (size_t)c.E * c.d_ff * c.d, 0.3), b1 = randd(r, (size_t)c.E * c.d_ff, 0.1);
    auto W2 = randd(r, (size_t)c.E * c.d * c.d_ff, 0.3), b2 = randd(r, (size_t)c.E * c.d, 0.1);
    auto rb = randf(r, c.E, 0.1), sb = randf(r, c.E, 0.1);
    std::vector<double> y(c.S * c.d + 1), y2(c.S * c.d + 1), gate(c.S * c.K + 1);
    std::vector<int32_t> idx(c.S * c.K + 1);
    check(oracle_layer_forward(x.data(), wr.data(), rb.data(), sb.data(), W1.data(), b1.data(), W2.data(),
                               b2.data(), c.S, c.d, c.d_ff, c.E, c.K, c.G, c.TG, c.renorm, 1.0, nullptr, y.data(),
                               idx.data(), gate.data()) == 0,
          "layer: accepted");
    check_route(idx, gate, c.S, c.E, c.K, c.G, c.TG, c.renorm);
    // the same layer from precomputed scores, no optional outputs
    std::vector<float> lg(c.S * c.E + 1);
    oracle_router_logits(x.data(), wr.data(), rb.data(), c.S, c.d, c.E, lg.data());
    check(oracle_layer_forward(x.data(), wr.data(), nullptr, sb.data(), W1.data(), b1.data(), W2.data(), b2.data(),
                               c.S, c.d, c.d_ff, c.E, c.K, c.G, c.TG, c.renorm, 1.0, lg.data(), y2.data(), nullptr,
                               nullptr) == 0,
          "layer: accepted with scores given");
    for (int64_t i = 0; i < c.S * c.d; ++i) check(y[i] == y2[i], "layer: given scores give the same output");
  }
  // a rejected group configuration
  std::vector<double> z(64, 0.0);
  std::vector<double> y(8);
  check(oracle_layer_forward(z.data(), z.data(), nullptr, nullptr, z.data(), z.data(), z.data(), z.data(), 1, 2, 2,
                             6, 2, 4, 2, 1, 1.0, nullptr, y.data(), nullptr, nullptr) == -1,
        "layer: invalid groups rejected");
}

}  // namespace

#ifdef PLANT_SHORT_OFFSETS
// A caller's mistake the sanitizer must catch: offsets sized E, not E + 1.
void planted_short_offsets() {
  const int32_t E = 4, K = 2;
  std::vector<int32_t> idx = {0, 1, 2, 3}, counts(E), perm(4), inv(4);
  int32_t* offsets = new int32_t[E];
  oracle_permute(idx.data(), 2, K, E, 1, counts.data(), offsets, perm.data(), inv.data());
  delete[] offsets;
}
#endif

int main() {
#ifdef PLANT_SHORT_OFFSETS
  planted_short_offsets();
#endif
  oracle_set_threads(2);
  check(oracle_threads() == 2, "threads set");
  Rng r{12345};
  test_decoders();
  test_router_logits(r);
  test_route(r);
  test_permute(r);
  test_dense_ffn(r);
  test_layer(r);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("all checks held\n");
  return 0;
}
