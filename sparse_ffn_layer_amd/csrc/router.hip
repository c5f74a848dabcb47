// Router: scores, (group-limited) Top-K selection and gates; one wavefront
// selects for each token (its scores summed by one wave, or by four for a
// small batch).
//
// Chapter "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), sections
// 11.1.1-11.1.2: router scores are x W_r, a softmax over the experts gives the
// routing distribution, TopK keeps the K largest scores.  Section 11.4.1 notes
// that fusing softmax, Top-K and the weighting into one kernel cuts
// batch-size-1 latency; here scores, selection and gates share one launch
// (the weighting itself has to wait for the experts, in the combine kernel).
// "MoE 推理工程深层实战" (ybb.press), section 2.3: the selection-only bias and
// the node(group)-limited two-stage choice.
//
// Register layout: expert e lives in lane (e % 64), slot (e / 64) of a
// per-lane array, so a token's E scores sit in registers and every reduction
// is a wave shuffle.  Ties: equal keys choose the lower expert index, equal
// group scores the lower group index.  Group scores are float32 sums taken in
// the pairwise-halving order v[j] += v[j + w], w = m/2 ... 1, over the
// group's experts in index order.
#include "common.h"
#include "select.h"

#include <climits>

namespace sfl {

constexpr int ROUTER_WAVES = 4;  // waves of a router block
// Large batches with a small router matrix: blocks of 16 waves (one token
// each) stage W_r in LDS once instead of every wave reading all of it through
// its L1 (64 KB per token at the Mixtral shape).
constexpr int ROUTER_LDS_WAVES = 16;
constexpr int ROUTER_LDS_BYTES = 64 * 1024;
constexpr int ROUTER_LDS_SPANS = 8;   // the row's 16-byte-per-lane spans held in registers

// Select K experts from this token's logits and write indices and gates.
// lg[r]: unbiased logit of expert r*64 + lane (-inf where that is >= E).
template <int R>
__device__ __forceinline__ void select_and_gate(const float (&lg)[R], int E, int K,
                                                const float* __restrict__ sbias, int n_groups,
                                                int topk_groups, int renorm, float inv_tau, int64_t t,
                                                int32_t* __restrict__ idx_out,
                                                float* __restrict__ gate_out) {
  const int lane = lane_id();
  float key[R];
  selection_keys<R>(lg, E, sbias, n_groups, topk_groups, key);

  // K rounds of wave arg-max; lane k keeps slot k's expert and logit
  int my_e = 0;
  float my_l = -INFINITY;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int e = r * 64 + lane;
      if (e < E && (key[r] > bv || (key[r] == bv && e < bi))) { bv = key[r]; bi = e; }
    }
    wave_argmax(bv, bi);
    float l_sel = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if ((bi >> 6) == r) {
        l_sel = lg[r];
        if ((bi & 63) == lane) key[r] = -INFINITY;  // taken
      }
    }
    l_sel = __shfl(l_sel, bi & 63, 64);
    if (lane == k) { my_e = bi; my_l = l_sel; }
  }

  const float g = slot_gate<R>(lg, E, renorm, inv_tau, lane < K, my_l);
  if (lane < K) {
    idx_out[t * K + lane] = my_e;
    gate_out[t * K + lane] = g;
  }
}

// Scores x . W_r (+ router_bias) on the vector ALUs, then selection.  WPT
// waves per token (ROUTER_WAVES / WPT tokens per block): wave w of a token
// sums the spans w, w + WPT, ... of the row (a span is one 16-byte load per
// lane) for every expert, EC experts per pass; the partial sums meet in LDS
// and are added in wave order, so the scores do not depend on scheduling;
// the token's first wave then selects.  Splitting a row over several waves
// shortens the chain of dependent loads each wave waits on, which is what a
// small batch pays for; a large batch has waves enough to hide it (WPT = 1).
// WR_LDS (WPT = 1, E d sizeof(T) <= ROUTER_LDS_BYTES, d <= ROUTER_LDS_SPANS
// spans): the block first copies W_r to LDS and the waves read it there;
// every lane sums the same products in the same order as when it reads W_r
// from memory, so the scores are the same bits.
template <typename T, int EC, int R, int WPT, int WAVES = ROUTER_WAVES, bool WR_LDS = false>
__global__ void __launch_bounds__(64 * WAVES)
router_fused_kernel(int64_t S, int d, int E, int K, const T* __restrict__ x,
                    const T* __restrict__ Wr, const float* __restrict__ rbias,
                    const float* __restrict__ sbias, int n_groups, int topk_groups, int renorm,
                    float inv_tau, float* __restrict__ logits_out, int32_t* __restrict__ idx,
                    float* __restrict__ gate) {
  static_assert(WAVES % WPT == 0, "whole tokens per block");
  static_assert(!WR_LDS || WPT == 1, "W_r in LDS: one wave per token");
  __shared__ float part[WAVES][64 * R];
  __shared__ uint4 wr_s[WR_LDS ? ROUTER_LDS_BYTES / 16 : 1];
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = wave % WPT;  // this wave's share of the token's row
  const int64_t t = (int64_t)blockIdx.x * (WAVES / WPT) + wave / WPT;
  const bool live = t < S;     // every wave still reaches the barrier
  constexpr int VEC = 16 / sizeof(T);  // elements per 16-byte load
  constexpr int SPAN = 64 * VEC;
  const T* xr = x + (live ? t : 0) * d;
  // WR_LDS: the lane's chunks of the token's row are loaded first, all at
  // once (d <= ROUTER_LDS_SPANS spans, checked by the host), and stay in
  // registers while W_r is copied
  uint4 xrow[WR_LDS ? ROUTER_LDS_SPANS : 1];
  if constexpr (WR_LDS) {
#pragma unroll
    for (int k = 0; k < ROUTER_LDS_SPANS; ++k) {
      const int i0 = k * SPAN + lane * VEC;
      xrow[k] = (live && i0 < d) ? *reinterpret_cast<const uint4*>(xr + i0) : make_uint4(0, 0, 0, 0);
    }
    const int chunks = E * d / VEC;  // the host checked E d sizeof(T) <= ROUTER_LDS_BYTES
    for (int c = threadIdx.x; c < chunks; c += 64 * WAVES) wr_s[c] = reinterpret_cast<const uint4*>(Wr)[c];
    __syncthreads();
  }

  for (int e0 = 0; e0 < E && live; e0 += EC) {
    float acc[EC];
#pragma unroll
    for (int j = 0; j < EC; ++j) acc[j] = 0.f;
    if constexpr (WR_LDS) {
      // spans in the same order as the loop below (WPT = 1)
#pragma unroll
      for (int k = 0; k < ROUTER_LDS_SPANS; ++k) {
        if (k * SPAN >= d) break;
        const int i0 = k * SPAN + lane * VEC;
        if (i0 >= d) continue;
        float xv[VEC];
        if constexpr (sizeof(T) == 2) {
          const uint32_t w[4] = {xrow[k].x, xrow[k].y, xrow[k].z, xrow[k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) { xv[2 * q] = bf16_bits_to_f32(w[q] & 0xffff); xv[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16); }
        } else {
          xv[0] = __uint_as_float(xrow[k].x); xv[1] = __uint_as_float(xrow[k].y);
          xv[2] = __uint_as_float(xrow[k].z); xv[3] = __uint_as_float(xrow[k].w);
        }
#pragma unroll
        for (int j = 0; j < EC; ++j) {
          if (e0 + j < E) {
            const uint4 raw = wr_s[((e0 + j) * d + i0) / VEC];
            float s = acc[j];
            if constexpr (sizeof(T) == 2) {
              const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                s = fmaf(xv[2 * q], bf16_bits_to_f32(w[q] & 0xffff), s);
                s = fmaf(xv[2 * q + 1], bf16_bits_to_f32(w[q] >> 16), s);
              }
            } else {
              s = fmaf(xv[0], __uint_as_float(raw.x), s); s = fmaf(xv[1], __uint_as_float(raw.y), s);
              s = fmaf(xv[2], __uint_as_float(raw.z), s); s = fmaf(xv[3], __uint_as_float(raw.w), s);
            }
            acc[j] = s;
          }
        }
      }
    } else
#pragma unroll 2
    for (int s0 = sub * SPAN; s0 < d; s0 += WPT * SPAN) {
      const int i0 = s0 + lane * VEC;
      if (i0 >= d) continue;
      float xv[VEC];
      if constexpr (sizeof(T) == 2) {
        const uint4 raw = *reinterpret_cast<const uint4*>(xr + i0);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { xv[2 * q] = bf16_bits_to_f32(w[q] & 0xffff); xv[2 * q + 1] = bf16_bits_to_f32(w[q] >> 16); }
      } else {
        const float4 raw = *reinterpret_cast<const float4*>(xr + i0);
        xv[0] = raw.x; xv[1] = raw.y; xv[2] = raw.z; xv[3] = raw.w;
      }
#pragma unroll
      for (int j = 0; j < EC; ++j) {
        if (e0 + j < E) {
          const T* wr = Wr + (int64_t)(e0 + j) * d + i0;
          float s = acc[j];
          if constexpr (sizeof(T) == 2) {
            const uint4 raw = *reinterpret_cast<const uint4*>(wr);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              s = fmaf(xv[2 * q], bf16_bits_to_f32(w[q] & 0xffff), s);
              s = fmaf(xv[2 * q + 1], bf16_bits_to_f32(w[q] >> 16), s);
            }
          } else {
            const float4 raw = *reinterpret_cast<const float4*>(wr);
            s = fmaf(xv[0], raw.x, s); s = fmaf(xv[1], raw.y, s);
            s = fmaf(xv[2], raw.z, s); s = fmaf(xv[3], raw.w, s);
          }
          acc[j] = s;
        }
      }
    }
#pragma unroll
    for (int j = 0; j < EC; ++j) {
      const float tot = wave_sum(acc[j]);
      if (lane == 0 && e0 + j < E) part[wave][e0 + j] = tot;
    }
  }
  __syncthreads();
  if (sub != 0 || !live) return;
  float lg[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * 64 + lane;
    lg[r] = -INFINITY;
    if (e < E) {
      float l = part[wave][e];
#pragma unroll
      for (int w = 1; w < WPT; ++w) l += part[wave + w][e];
      lg[r] = rbias != nullptr ? l + rbias[e] : l;
    }
  }
  if (logits_out != nullptr) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r * 64 + lane < E) logits_out[t * E + r * 64 + lane] = lg[r];
  }
  select_and_gate<R>(lg, E, K, sbias, n_groups, topk_groups, renorm, inv_tau, t, idx, gate);
}

// Selection from precomputed float32 scores [S][E].
template <int R>
__global__ void __launch_bounds__(64 * ROUTER_WAVES)
route_logits_kernel(int64_t S, int E, int K, const float* __restrict__ logits,
                    const float* __restrict__ sbias, int n_groups, int topk_groups, int renorm,
                    float inv_tau, float* __restrict__ logits_copy, int32_t* __restrict__ idx,
                    float* __restrict__ gate) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * ROUTER_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= S) return;
  float lg[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * 64 + lane;
    lg[r] = e < E ? logits[t * E + e] : -INFINITY;
    if (logits_copy != nullptr && e < E) logits_copy[t * E + e] = lg[r];
  }
  select_and_gate<R>(lg, E, K, sbias, n_groups, topk_groups, renorm, inv_tau, t, idx, gate);
}

// ------------------------------------------------------------------ statistics
// Load statistics of one routing, one workgroup of 16 waves.  Counts: thread
// e reads expert e's count; sums in a fixed tree order.  Aux loss: wave w
// takes tokens w, w + 16, ... in order and accumulates softmax(logits / tau)
// per expert in its registers; the 16 partial sums are added in wave order.
// Every sum has a fixed order, so the result is deterministic.
constexpr int STATS_WAVES = 16;
template <int R>
__global__ void __launch_bounds__(64 * STATS_WAVES)
load_stats_kernel(int64_t S, int E, int K, const int32_t* __restrict__ counts,
                  const float* __restrict__ logits, const int32_t* __restrict__ dropped, float alpha,
                  float inv_tau, float* __restrict__ stats) {
  __shared__ float red[64 * STATS_WAVES];
  __shared__ int ired[64 * STATS_WAVES];
  __shared__ float pexp[STATS_WAVES][R * 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // ---- counts: sum, max, min, empty (exact integers), then sum of squares
  int c = tid < E ? counts[tid] : 0;
  auto tree_i = [&](int v, int op) -> int {  // op 0: sum, 1: max, 2: min
    ired[tid] = v;
    __syncthreads();
    for (int w = 64 * STATS_WAVES / 2; w >= 1; w >>= 1) {
      if (tid < w) {
        const int o = ired[tid + w];
        ired[tid] = op == 0 ? ired[tid] + o : op == 1 ? max(ired[tid], o) : min(ired[tid], o);
      }
      __syncthreads();
    }
    const int r = ired[0];
    __syncthreads();
    return r;
  };
  auto tree_f = [&](float v) -> float {
    red[tid] = v;
    __syncthreads();
    for (int w = 64 * STATS_WAVES / 2; w >= 1; w >>= 1) {
      if (tid < w) red[tid] += red[tid + w];
      __syncthreads();
    }
    const float r = red[0];
    __syncthreads();
    return r;
  };
  const int total = tree_i(c, 0);
  const int cmax = tree_i(tid < E ? c : INT_MIN, 1);
  const int cmin = tree_i(tid < E ? c : INT_MAX, 2);
  const int empty = tree_i(tid < E && c == 0 ? 1 : 0, 0);
  const float mean = (float)total / (float)E;
  const float dev = tid < E ? (float)c - mean : 0.f;
  const float var = tree_f(dev * dev) / (float)E;

  // ---- aux loss: P_i = mean over tokens of softmax(logits[t] / tau)[i]
  float aux = 0.f;
  if (logits != nullptr && total > 0 && S > 0) {
    float p[R];
#pragma unroll
    for (int r = 0; r < R; ++r) p[r] = 0.f;
    for (int64_t t = wave; t < S; t += STATS_WAVES) {
      float l[R];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = r * 64 + lane;
        l[r] = e < E ? logits[t * E + e] : -INFINITY;
        mx = fmaxf(mx, l[r]);
      }
      mx = wave_max(mx);
      float z = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        l[r] = (r * 64 + lane < E) ? expf((l[r] - mx) * inv_tau) : 0.f;
        z += l[r];
      }
      z = wave_sum(z);
      const float iz = 1.f / z;
#pragma unroll
      for (int r = 0; r < R; ++r) p[r] += l[r] * iz;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) pexp[wave][r * 64 + lane] = p[r];
    __syncthreads();
    float term = 0.f;
    if (tid < E) {
      float P = 0.f;
      for (int w = 0; w < STATS_WAVES; ++w) P += pexp[w][tid];  // wave order
      P /= (float)S;
      term = ((float)c / (float)total) * P;
    }
    aux = alpha * tree_f(term);
  }
  if (tid == 0) {
    const int64_t pairs = S * (int64_t)K;
    const int drop = dropped != nullptr ? dropped[0] : 0;
    stats[0] = mean;
    stats[1] = sqrtf(var);
    stats[2] = mean > 0.f ? (float)cmax / mean : 0.f;
    stats[3] = pairs > 0 ? (float)drop / (float)pairs : 0.f;
    stats[4] = aux;
    stats[5] = (float)cmax;
    stats[6] = (float)cmin;
    stats[7] = (float)empty;
  }
}

hipError_t launch_load_stats(const Problem& p, const int32_t* counts, const float* logits,
                             const int32_t* dropped, float alpha, float* stats, hipStream_t st) {
  const int R = (p.E + 63) / 64;
  const dim3 grid(1), block(64 * STATS_WAVES);
#define SFL_STATS(RR) \
  load_stats_kernel<RR><<<grid, block, 0, st>>>(p.S, p.E, p.K, counts, logits, dropped, alpha, p.inv_tau, stats)
  switch (R) {
    case 1: SFL_STATS(1); break;
    case 2: SFL_STATS(2); break;
    case 3: case 4: SFL_STATS(4); break;
    default: SFL_STATS(8); break;
  }
#undef SFL_STATS
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
template <typename T, int EC>
static hipError_t launch_fused_T(const Problem& p, const void* x, const void* Wr, const float* rb,
                                 const float* sb, float* lo, int32_t* idx, float* gate,
                                 hipStream_t st) {
  const int R = (p.E + 63) / 64;
  // a row per wave once the batch alone fills the chip with waves
  const bool split = p.S < 2048;
  // ... and then W_r in LDS when it fits
  const bool wr_lds = !split && (int64_t)p.E * p.d * (int64_t)sizeof(T) <= ROUTER_LDS_BYTES &&
                      p.d <= ROUTER_LDS_SPANS * 64 * (16 / (int)sizeof(T));
  const dim3 grid((unsigned)(split ? p.S : ceil_div(p.S, ROUTER_WAVES))), block(64 * ROUTER_WAVES);
  const dim3 grid_lds((unsigned)ceil_div(p.S, ROUTER_LDS_WAVES)), block_lds(64 * ROUTER_LDS_WAVES);
#define SFL_FUSED(RR)                                                                              \
  do {                                                                                             \
    if (wr_lds)                                                                                    \
      router_fused_kernel<T, EC, RR, 1, ROUTER_LDS_WAVES, true><<<grid_lds, block_lds, 0, st>>>(   \
          p.S, p.d, p.E, p.K, (const T*)x, (const T*)Wr, rb, sb, p.n_groups, p.topk_groups,        \
          p.renormalize, p.inv_tau, lo, idx, gate);                                                \
    else if (split)                                                                                \
      router_fused_kernel<T, EC, RR, ROUTER_WAVES><<<grid, block, 0, st>>>(                        \
          p.S, p.d, p.E, p.K, (const T*)x, (const T*)Wr, rb, sb, p.n_groups, p.topk_groups,        \
          p.renormalize, p.inv_tau, lo, idx, gate);                                                \
    else                                                                                           \
      router_fused_kernel<T, EC, RR, 1><<<grid, block, 0, st>>>(                                   \
          p.S, p.d, p.E, p.K, (const T*)x, (const T*)Wr, rb, sb, p.n_groups, p.topk_groups,        \
          p.renormalize, p.inv_tau, lo, idx, gate);                                                \
  } while (0)
  switch (R) {
    case 1: SFL_FUSED(1); break;
    case 2: SFL_FUSED(2); break;
    case 3: case 4: SFL_FUSED(4); break;
    default: SFL_FUSED(8); break;
  }
#undef SFL_FUSED
  return hipGetLastError();
}

hipError_t launch_router_fused(const Problem& p, const void* x, const void* Wr, const float* rb,
                               const float* sb, float* logits_out, int32_t* idx, float* gate,
                               hipStream_t st) {
  if (p.act == DT_BF16) {
    if (p.E <= 8) return launch_fused_T<uint16_t, 8>(p, x, Wr, rb, sb, logits_out, idx, gate, st);
    return launch_fused_T<uint16_t, 32>(p, x, Wr, rb, sb, logits_out, idx, gate, st);
  }
  if (p.E <= 8) return launch_fused_T<float, 8>(p, x, Wr, rb, sb, logits_out, idx, gate, st);
  return launch_fused_T<float, 32>(p, x, Wr, rb, sb, logits_out, idx, gate, st);
}

hipError_t launch_route_logits(const Problem& p, const float* logits, const float* sb,
                               float* logits_copy, int32_t* idx, float* gate, hipStream_t st) {
  const int R = (p.E + 63) / 64;
  const dim3 grid((unsigned)ceil_div(p.S, ROUTER_WAVES)), block(64 * ROUTER_WAVES);
#define SFL_ROUTE(RR)                                                                         \
  route_logits_kernel<RR><<<grid, block, 0, st>>>(p.S, p.E, p.K, logits, sb, p.n_groups,     \
                                                  p.topk_groups, p.renormalize, p.inv_tau,   \
                                                  logits_copy, idx, gate)
  switch (R) {
    case 1: SFL_ROUTE(1); break;
    case 2: SFL_ROUTE(2); break;
    case 3: case 4: SFL_ROUTE(4); break;
    default: SFL_ROUTE(8); break;
  }
#undef SFL_ROUTE
  return hipGetLastError();
}

}  // namespace sfl
