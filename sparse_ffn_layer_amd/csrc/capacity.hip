// Capacity-limited dispatch: at most `cap` (token, slot) pairs per expert;
// the excess is rerouted to the next-best expert, or dropped.
//
// Chapter "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), section 11.3.3,
// expert dropping: the excess of an overloaded expert moves to its next-best
// expert.  "MoE 推理工程深层实战" (ybb.press), section 1.2 (token drop rate)
// and section 2.2 (tokens past a receive buffer's capacity are dropped or
// deferred).  The pages leave the rule open; this file implements rounds:
//   accept:  every pending pair proposes its current expert; the expert takes
//            proposals in (token, slot) order while it has room;
//   reroute: a rejected pair moves to the best expert of its token's
//            selection ranking (the router's keys: logit + select_bias, kept
//            groups only; key descending, lower index on ties) that has room
//            and that the token does not hold in another accepted or pending
//            slot; a token's rejected slots are taken in slot order; with no
//            such expert the pair is dropped (index -1).
// A round with a rejection fills at least one more expert, so at most E + 1
// rounds run.
//
// One workgroup of 16 waves runs every round (the rounds are sequential and
// usually few).  The state lives in topk_idx itself (the current expert of
// each pair, -1 once dropped), the LDS (run[e]: pairs expert e has been
// offered, so e is full once run[e] >= cap) and one list of pair ids in
// the workspace:
//   accept:  the pending pairs are taken 1024 at a time in list order; wave
//            ballots over the expert id bits give each pair its rank among
//            equal experts in the wave, per-wave LDS counts carry it across
//            waves, run[e] across chunks.  Rejected pairs are compacted, in
//            order, to the front of the list (a pair is written at or before
//            the slot it was read from, after the chunk has been read).
//   reroute: one wave per token.  Rejected pairs of one token are adjacent in
//            the list; the wave recomputes the token's keys with the
//            router's arithmetic and runs one arg-max per rejected slot.
// Gates are then recomputed for every token over its kept slots, one wave
// per token, with the router's arithmetic (so a token that kept all its
// slots keeps bit-identical gates).
#include "common.h"
#include "select.h"

#include <climits>

namespace sfl {

constexpr int CAP_WAVES = 16;
constexpr int CAP_THREADS = 64 * CAP_WAVES;
constexpr int CAP_MAX_E = 512;
constexpr int CAP_GATE_WAVES = 4;

template <int R>
__global__ void __launch_bounds__(CAP_THREADS)
capacity_dispatch_kernel(int pairs, int E, int K, int ebits, int cap, const float* __restrict__ logits,
                         const float* __restrict__ sbias, int n_groups, int topk_groups,
                         int32_t* __restrict__ idx, int32_t* __restrict__ list,
                         int32_t* __restrict__ dropped_out) {
  __shared__ int run[CAP_MAX_E];
  __shared__ int wc[CAP_WAVES][CAP_MAX_E + 1];
  __shared__ int wrej[CAP_WAVES];
  __shared__ int ndrop;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = threadIdx.x; e < E; e += CAP_THREADS) {
    run[e] = 0;
#pragma unroll
    for (int w = 0; w < CAP_WAVES; ++w) wc[w][e] = 0;
  }
  if (threadIdx.x == 0) ndrop = 0;
  __syncthreads();

  // One acceptance pass over n entries (the pairs 0..n-1 themselves in the
  // first round, list[0..n) afterwards).  Returns the number of rejected
  // pairs, now at list[0..nrej) in order.
  auto accept = [&](bool first, int n) -> int {
    int nrej = 0;
    for (int q0 = 0; q0 < n; q0 += CAP_THREADS) {
      const int i = q0 + (int)threadIdx.x;
      int pr = -1, e = E;  // E: sentinel for no pending pair
      bool bad = false;
      if (i < n) {
        pr = first ? i : list[i];
        const int v = idx[pr];
        if (v >= 0 && v < E) e = v;
        else if (first) bad = true;  // routed to no expert: a dropped pair
      }
      if (bad) idx[pr] = -1;
      const uint64_t bb = __ballot(bad);
      if (lane == 0 && bb) atomicAdd(&ndrop, __popcll(bb));
      const bool valid = e < E;
      uint64_t peers = ~0ull;
      for (int bit = 0; bit < ebits; ++bit) {
        const bool set = (e >> bit) & 1;
        const uint64_t bal = __ballot(set);
        peers &= set ? bal : ~bal;
      }
      const int rank_w = __popcll(peers & lt);
      const bool leader = (peers & lt) == 0;
      if (valid && leader) wc[wave][e] = __popcll(peers);
      __syncthreads();
      bool rej = false;
      if (valid) {
        int pos = run[e] + rank_w;
        for (int w = 0; w < wave; ++w) pos += wc[w][e];
        rej = pos >= cap;
      }
      const uint64_t rb = __ballot(rej);
      if (lane == 0) wrej[wave] = __popcll(rb);
      __syncthreads();
      int base = nrej, tot = 0;
      for (int w = 0; w < CAP_WAVES; ++w) {
        const int c = wrej[w];
        if (w < wave) base += c;
        tot += c;
      }
      if (rej) list[base + __popcll(rb & lt)] = pr;
      if (valid && leader) {
        atomicAdd(&run[e], __popcll(peers));
        wc[wave][e] = 0;
      }
      nrej += tot;
      __syncthreads();
    }
    return nrej;
  };

  // Reroute the rejected pairs list[0..n); one wave per token.
  auto reroute = [&](int n) {
    for (int c = wave; c * 64 < n; c += CAP_WAVES) {
      const int i = c * 64 + lane;
      const int ti = i < n ? list[i] / K : -1;
      const bool start = i < n && (i == 0 || list[i - 1] / K != ti);
      uint64_t sm = __ballot(start);
      while (sm) {
        const int b = __builtin_ctzll(sm);
        sm &= sm - 1;
        const int s = c * 64 + b;
        const int t = __shfl(ti, b, 64);
        // this token's rejected slots: list[s .. s + len), len <= K <= 64
        const int j = s + lane;
        const int pj = (lane < K && j < n) ? list[j] : -1;
        const bool inrun = pj >= 0 && pj / K == t;
        const int len = __popcll(__ballot(inrun));
        const int kj = inrun ? pj - t * K : 0;
        uint64_t umask = 0;  // slots still waiting to be rerouted
        for (int l = 0; l < len; ++l) umask |= 1ull << __shfl(kj, l, 64);
        const int64_t row = (int64_t)t * K;
        int cur = lane < K ? idx[row + lane] : -1;  // lane l: slot l's expert
        float lg[R], key[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int e = r * 64 + lane;
          lg[r] = e < E ? logits[(int64_t)t * E + e] : -INFINITY;
        }
        selection_keys<R>(lg, E, sbias, n_groups, topk_groups, key);
        for (int l = 0; l < len; ++l) {
          const int k = __shfl(kj, l, 64);
          // experts held by the token's other accepted or pending slots
          const int h = (lane < K && lane != k && !((umask >> lane) & 1ull)) ? cur : -1;
          bool ok[R];
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int e = r * 64 + lane;
            ok[r] = e < E && key[r] != -INFINITY && run[e] < cap;
          }
          for (int m = 0; m < K; ++m) {
            const int hm = __shfl(h, m, 64);
#pragma unroll
            for (int r = 0; r < R; ++r)
              if (r * 64 + lane == hm) ok[r] = false;
          }
          float bv = -INFINITY;
          int bi = INT_MAX;
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const int e = r * 64 + lane;
            if (ok[r] && (key[r] > bv || (key[r] == bv && e < bi))) { bv = key[r]; bi = e; }
          }
          wave_argmax(bv, bi);
          const int ne = bi < E ? bi : -1;
          if (lane == k) cur = ne;
          umask &= ~(1ull << k);
          if (lane == 0) {
            idx[row + k] = ne;
            if (ne < 0) atomicAdd(&ndrop, 1);
          }
        }
      }
    }
  };

  int nrej = accept(true, pairs);
  for (int round = 0; nrej > 0 && round <= E; ++round) {
    reroute(nrej);
    __syncthreads();
    nrej = accept(false, nrej);
  }
  // Unreachable by the round bound above; kept so that every pair ends in a
  // defined state whatever the input.
  for (int i = threadIdx.x; i < nrej; i += CAP_THREADS) {
    idx[list[i]] = -1;
    atomicAdd(&ndrop, 1);
  }
  __syncthreads();
  if (threadIdx.x == 0 && dropped_out != nullptr) dropped_out[0] = ndrop;
}

// Gates over each token's kept slots, one wave per token.
template <int R>
__global__ void __launch_bounds__(64 * CAP_GATE_WAVES)
capacity_gates_kernel(int64_t S, int E, int K, int renorm, float inv_tau,
                      const float* __restrict__ logits, const int32_t* __restrict__ idx,
                      float* __restrict__ gate) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * CAP_GATE_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (t >= S) return;
  float lg[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = r * 64 + lane;
    lg[r] = e < E ? logits[t * E + e] : -INFINITY;
  }
  const int my_e = lane < K ? idx[t * K + lane] : -1;
  const bool kept = my_e >= 0 && my_e < E;
  const float my_l = kept ? logits[t * E + my_e] : 0.f;
  const float g = slot_gate<R>(lg, E, renorm, inv_tau, kept, my_l);
  if (lane < K) gate[t * K + lane] = g;
}

// ------------------------------------------------------------------ launchers
size_t capacity_scratch_ints(int64_t pairs) { return (size_t)pairs; }

hipError_t launch_capacity(const Problem& p, int cap, const float* logits, const float* sb,
                           int32_t* idx, float* gate, int32_t* dropped, int32_t* scratch,
                           hipStream_t st) {
  const int pairs = (int)(p.S * p.K);
  const int c = cap > 0 ? cap : INT_MAX;  // 0: no limit
  int ebits = 0;
  while ((1 << ebits) <= p.E) ++ebits;  // enough bits for 0..E (E is the sentinel)
  const int R = (p.E + 63) / 64;
  const dim3 gg((unsigned)ceil_div(p.S, CAP_GATE_WAVES)), gb(64 * CAP_GATE_WAVES);
#define SFL_CAP(RR)                                                                              \
  capacity_dispatch_kernel<RR><<<1, CAP_THREADS, 0, st>>>(pairs, p.E, p.K, ebits, c, logits, sb,  \
                                                          p.n_groups, p.topk_groups, idx, scratch, \
                                                          dropped);                               \
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;                              \
  capacity_gates_kernel<RR><<<gg, gb, 0, st>>>(p.S, p.E, p.K, p.renormalize, p.inv_tau, logits,   \
                                               idx, gate)
  switch (R) {
    case 1: SFL_CAP(1); break;
    case 2: SFL_CAP(2); break;
    case 3: case 4: SFL_CAP(4); break;
    default: SFL_CAP(8); break;
  }
#undef SFL_CAP
  return hipGetLastError();
}

}  // namespace sfl
