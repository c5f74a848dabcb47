// Plain C++ reference loops of the single-GPU MoE-layer forward, over host
// memory in double precision.
//
// TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
// cpu_baseline leg load this library.  It shares no code with the HIP path
// (nor with the numpy oracle next to it, which it is checked against).
//
// Sources (page title, section):
//  [P1] "MoE 推理工程深层实战" (ybb.press), section 2.3: selection-only bias and
//       the node(group)-limited Top-K.
//  [P2] "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), sections 11.1.1
//       (router-weighted sum of experts, softmax router, TopK), 11.1.2 (expert
//       FFN GeLU(x W1 + b1) W2 + b2; B x L x K forwards grouped per expert),
//       11.2.1 (regrouping per expert and back), 11.3.3 (gate temperature).
//  [P3] "MoE 混合专家推理" (plumephp.com), one MoE forward and the worked example.
//
// Readings (where the pages are silent): equal keys choose the lower expert
// index and equal group scores the lower group index; a group's score is the
// float32 sum of its biased scores in the pairwise-halving order
// v[j] += v[j + w], w = m/2 ... 1; gates come from the unbiased scores,
// renormalised over the K chosen (renormalize = 1) or as full-softmax
// probabilities (renormalize = 0); GeLU is x * Phi(x) with erf; the experts'
// rows keep token order.
#include <omp.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>

namespace {

// bfloat16 = the upper half of an IEEE binary32 word.
double bf16_value(uint16_t b) {
  uint32_t w = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &w, 4);
  return (double)f;
}

// OCP E4M3FN: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
// exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity.
double e4m3_value(uint8_t c) {
  const int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  const double mag = e == 0 ? std::ldexp(m / 8.0, -6) : std::ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

double gelu(double a) { return 0.5 * a * (1.0 + std::erf(a / std::sqrt(2.0))); }

}  // namespace

extern "C" {

// Threads the loops below use (OpenMP): set, and query.
void oracle_set_threads(int32_t n) { omp_set_num_threads(n > 0 ? n : 1); }
int32_t oracle_threads(void) { return omp_get_max_threads(); }

void oracle_decode_bf16(const uint16_t* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = bf16_value(src[i]);
}

void oracle_decode_e4m3(const uint8_t* src, int64_t n, double* dst) {
  for (int64_t i = 0; i < n; ++i) dst[i] = e4m3_value(src[i]);
}

// [P2] 11.1.2: scores s = x W_r (+ bias), summed in double with i ascending
// and rounded once to float.  x [S][d], w_r [E][d] (linear-layer layout).
void oracle_router_logits(const double* x, const double* w_r, const float* router_bias, int64_t S, int32_t d,
                          int32_t E, float* logits) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < S; ++t) {
    for (int32_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int32_t i = 0; i < d; ++i) acc += x[t * d + i] * w_r[(int64_t)e * d + i];
      if (router_bias != nullptr) acc += (double)router_bias[e];
      logits[t * E + e] = (float)acc;
    }
  }
}

// Selection and gates for each token ([P2] 11.1.1 TopK and softmax; [P1]
// 2.3 bias and group limit; [P2] 11.3.3 temperature).  Returns 0, or -1 for
// an invalid group configuration.
int32_t oracle_route(const float* logits, const float* select_bias, int64_t S, int32_t E, int32_t K,
                     int32_t n_groups, int32_t topk_groups, int32_t renormalize, double temperature,
                     int32_t* topk_idx, double* topk_gate) {
  const int32_t G = n_groups > 1 ? n_groups : 1;
  const int32_t m = E / G;
  if (K < 1 || K > E || m * G != E)
    return -1;
  if (G > 1 && ((m & (m - 1)) != 0 || topk_groups < 1 || topk_groups > G || K > topk_groups * m)) return -1;
  const float NEG = -std::numeric_limits<float>::infinity();
  std::vector<float> key(E), v(m), gs(G);
  std::vector<char> used(E), keep(G);
  for (int64_t t = 0; t < S; ++t) {
    const float* l = logits + t * E;
    for (int32_t e = 0; e < E; ++e) key[e] = select_bias ? l[e] + select_bias[e] : l[e];
    if (G > 1) {
      for (int32_t g = 0; g < G; ++g) {
        for (int32_t j = 0; j < m; ++j) v[j] = key[g * m + j];
        for (int32_t w = m / 2; w >= 1; w /= 2)
          for (int32_t j = 0; j < w; ++j) v[j] = v[j] + v[j + w];
        gs[g] = v[0];
        keep[g] = 0;
      }
      for (int32_t r = 0; r < topk_groups; ++r) {
        int32_t best = -1;
        for (int32_t g = 0; g < G; ++g)
          if (!keep[g] && (best < 0 || gs[g] > gs[best])) best = g;
        keep[best] = 1;
      }
      for (int32_t e = 0; e < E; ++e)
        if (!keep[e / m]) key[e] = NEG;
    }
    for (int32_t e = 0; e < E; ++e) used[e] = 0;
    for (int32_t k = 0; k < K; ++k) {
      int32_t best = -1;
      for (int32_t e = 0; e < E; ++e)
        if (!used[e] && (best < 0 || key[e] > key[best])) best = e;
      used[best] = 1;
      topk_idx[t * K + k] = best;
    }
    // gates from the unbiased scores, divided by the temperature
    if (renormalize) {
      double mx = -std::numeric_limits<double>::infinity();
      for (int32_t k = 0; k < K; ++k) mx = std::fmax(mx, (double)l[topk_idx[t * K + k]] / temperature);
      double z = 0.0;
      for (int32_t k = 0; k < K; ++k) z += std::exp((double)l[topk_idx[t * K + k]] / temperature - mx);
      for (int32_t k = 0; k < K; ++k)
        topk_gate[t * K + k] = std::exp((double)l[topk_idx[t * K + k]] / temperature - mx) / z;
    } else {
      double mx = -std::numeric_limits<double>::infinity();
      for (int32_t e = 0; e < E; ++e) mx = std::fmax(mx, (double)l[e] / temperature);
      double z = 0.0;
      for (int32_t e = 0; e < E; ++e) z += std::exp((double)l[e] / temperature - mx);
      for (int32_t k = 0; k < K; ++k)
        topk_gate[t * K + k] = std::exp((double)l[topk_idx[t * K + k]] / temperature - mx) / z;
    }
  }
  return 0;
}

// [P2] 11.2.1: group the (token, slot) pairs p = t*K + k by expert, token
// order inside an expert.  counts[e]; offsets[e] = sum over e' < e of counts
// rounded up to tile_m (offsets[E] = the total); perm lists the pair ids
// expert by expert (dense, no padding); inv_perm[p] = the padded row of pair
// p, -1 for a pair whose index is outside [0, E).
void oracle_permute(const int32_t* topk_idx, int64_t S, int32_t K, int32_t E, int32_t tile_m, int32_t* counts,
                    int32_t* offsets, int32_t* perm, int32_t* inv_perm) {
  const int64_t P = S * K;
  for (int32_t e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t p = 0; p < P; ++p)
    if (topk_idx[p] >= 0 && topk_idx[p] < E) ++counts[topk_idx[p]];
  int64_t off = 0, dense = 0;
  std::vector<int64_t> dstart(E), fill(E, 0);
  for (int32_t e = 0; e < E; ++e) {
    offsets[e] = (int32_t)off;
    dstart[e] = dense;
    off += (counts[e] + tile_m - 1) / tile_m * tile_m;
    dense += counts[e];
  }
  offsets[E] = (int32_t)off;
  for (int64_t p = 0; p < P; ++p) {
    const int32_t e = topk_idx[p];
    if (e < 0 || e >= E) {
      inv_perm[p] = -1;
      continue;
    }
    perm[dstart[e] + fill[e]] = (int32_t)p;
    inv_perm[p] = (int32_t)(offsets[e] + fill[e]);
    ++fill[e];
  }
}

// [P2] 11.1.2: out = GeLU(x W1 + b1) W2 + b2 for n rows.  w1 [d_ff][d],
// w2 [d][d_ff] (linear-layer layout); sums in double, index ascending.
void oracle_dense_ffn(const double* x, int64_t n, int32_t d, int32_t d_ff, const double* w1, const double* b1,
                      const double* w2, const double* b2, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < n; ++r) {
    std::vector<double> h(d_ff);
    for (int32_t j = 0; j < d_ff; ++j) {
      double a = 0.0;
      for (int32_t i = 0; i < d; ++i) a += x[r * d + i] * w1[(int64_t)j * d + i];
      h[j] = gelu(a + b1[j]);
    }
    for (int32_t c = 0; c < d; ++c) {
      double o = 0.0;
      for (int32_t j = 0; j < d_ff; ++j) o += h[j] * w2[(int64_t)c * d_ff + j];
      out[r * d + c] = o + b2[c];
    }
  }
}

// The whole layer ([P2] 11.1.1-11.1.2; [P3] one MoE forward): scores (or
// logits_in), selection, gates, each routed pair through its expert, the
// gate-weighted sum over the slots in slot order.  Decoded inputs: x [S][d],
// w_r [E][d], W1 [E][d_ff][d], b1 [E][d_ff], W2 [E][d][d_ff], b2 [E][d]
// (fp8 weights already times their channel scales).  Optional outputs:
// topk_idx_out [S][K], topk_gate_out [S][K].  Returns 0 or -1.
int32_t oracle_layer_forward(const double* x, const double* w_r, const float* router_bias,
                             const float* select_bias, const double* W1, const double* b1, const double* W2,
                             const double* b2, int64_t S, int32_t d, int32_t d_ff, int32_t E, int32_t K,
                             int32_t n_groups, int32_t topk_groups, int32_t renormalize, double temperature,
                             const float* logits_in, double* y, int32_t* topk_idx_out, double* topk_gate_out) {
  std::vector<float> logits;
  const float* lg = logits_in;
  if (lg == nullptr) {
    logits.resize((size_t)S * E);
    oracle_router_logits(x, w_r, router_bias, S, d, E, logits.data());
    lg = logits.data();
  }
  std::vector<int32_t> idx((size_t)S * K);
  std::vector<double> gate((size_t)S * K);
  if (oracle_route(lg, select_bias, S, E, K, n_groups, topk_groups, renormalize, temperature, idx.data(),
                   gate.data()) != 0)
    return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t t = 0; t < S; ++t) {
    std::vector<double> o(d);
    for (int32_t c = 0; c < d; ++c) y[t * d + c] = 0.0;
    for (int32_t k = 0; k < K; ++k) {
      const int32_t e = idx[t * K + k];
      oracle_dense_ffn(x + t * d, 1, d, d_ff, W1 + (int64_t)e * d_ff * d, b1 + (int64_t)e * d_ff,
                       W2 + (int64_t)e * d * d_ff, b2 + (int64_t)e * d, o.data());
      for (int32_t c = 0; c < d; ++c) y[t * d + c] += gate[t * K + k] * o[c];
    }
  }
  // (no tokens: the vectors own no storage and there is nothing to copy)
  if (topk_idx_out && !idx.empty()) std::memcpy(topk_idx_out, idx.data(), idx.size() * sizeof(int32_t));
  if (topk_gate_out && !gate.empty()) std::memcpy(topk_gate_out, gate.data(), gate.size() * sizeof(double));
  return 0;
}

}  // extern "C"
