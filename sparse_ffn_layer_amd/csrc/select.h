// Per-token selection keys and slot gates, shared by the router and the
// capacity-limited dispatch so that both rank experts and weigh slots with
// bit-identical arithmetic.  One wavefront holds one token: expert e lives in
// lane (e % 64), register (e / 64) of a per-lane array of R registers.
//
// Chapter "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), sections 11.1.1-11.1.2
// (softmax router, TopK) and 11.3.3 (gate temperature); "MoE 推理工程深层实战"
// (ybb.press), section 2.3 (selection-only bias, group-limited choice).
#pragma once

#include "common.h"

namespace sfl {

// key[r] = lg[r] + select_bias[e] (one float32 add; lg[r] alone when sbias is
// NULL).  With n_groups > 1 the experts outside the token's topk_groups best
// groups get key -inf.  A group's score is the float32 sum of its m = E /
// n_groups keys in the pairwise-halving order v[j] += v[j + w], w = m/2 ... 1;
// equal scores choose the lower group index.
template <int R>
__device__ __forceinline__ void selection_keys(const float (&lg)[R], int E,
                                               const float* __restrict__ sbias, int n_groups,
                                               int topk_groups, float (&key)[R]) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * 64 + lane;
    key[r] = lg[r];
    if (sbias != nullptr && e < E) key[r] = lg[r] + sbias[e];
  }
  if (n_groups <= 1) return;

  const int m = E / n_groups;  // power of two
  float v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = key[r];
  for (int w = m >> 1; w >= 1; w >>= 1) {
    if (w >= 64) {  // partner lives in register r + w/64 of the same lane
      const int dr = w >> 6, per = m >> 6;
#pragma unroll
      for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int s = 1; s < R; ++s) {
          if (s == dr && r + s < R && (r % per) < dr) v[r] = v[r] + v[r + s];
        }
      }
    } else {  // partner is lane + w of the same register
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float o = __shfl_down(v[r], w, 64);
        v[r] = v[r] + o;
      }
    }
  }
  // group heads hold the scores; pick topk_groups groups
  uint64_t chosen = 0;
  for (int gk = 0; gk < topk_groups; ++gk) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = r * 64 + lane;
      const int g = e / m;
      if (e < E && (e % m) == 0 && !((chosen >> g) & 1ull)) {
        if (v[r] > bv || (v[r] == bv && g < bi)) { bv = v[r]; bi = g; }
      }
    }
    wave_argmax(bv, bi);
    chosen |= 1ull << bi;
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * 64 + lane;
    if (e < E && !((chosen >> (e / m)) & 1ull)) key[r] = -INFINITY;
  }
}

// Gate of the slot this lane holds (kept: the lane holds a slot with an
// expert; my_l: that expert's unbiased logit).  renorm = 1: softmax of
// logit / tau over the kept slots; renorm = 0: the expert's probability under
// the full softmax of logit / tau over all E experts.  0 for lanes that hold
// no kept slot.  inv_tau = 1 / tau (section 11.3.3's soft-routing
// temperature); at tau = 1 the product is exact.  Every lane must call it.
template <int R>
__device__ __forceinline__ float slot_gate(const float (&lg)[R], int E, int renorm, float inv_tau,
                                           bool kept, float my_l) {
  const int lane = lane_id();
  if (renorm) {
    const float mx = wave_max(kept ? my_l : -INFINITY);
    const float ex = kept ? expf((my_l - mx) * inv_tau) : 0.f;
    const float z = wave_sum(ex);
    return kept ? ex / z : 0.f;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int r = 0; r < R; ++r) mx = fmaxf(mx, lg[r]);
  mx = wave_max(mx);
  float z = 0.f;
#pragma unroll
  for (int r = 0; r < R; ++r) z += (r * 64 + lane < E) ? expf((lg[r] - mx) * inv_tau) : 0.f;
  z = wave_sum(z);
  return kept ? expf((my_l - mx) * inv_tau) / z : 0.f;
}

}  // namespace sfl
