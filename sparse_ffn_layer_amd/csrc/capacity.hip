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
// rounds run; skewed routings need a handful.
//
// State: topk_idx itself (the current expert of each pair, -1 once dropped),
// run[e] (pairs expert e has been offered, so e is full once run[e] >= cap),
// the drop count, and one list of pair ids.  Kernels, in stream order:
//   first:  one workgroup accepts all pairs; the rejected ones are compacted,
//           in order, into the list.
//   round (a few launches): every wave of a wide grid reroutes the token runs
//           that start in its share of the list (one wave per token, the
//           router's arithmetic for the keys); the last workgroup to finish
//           (counted with a device-scope atomic after a release fence) then
//           runs the next acceptance over the rerouted pairs.  A launch with
//           nothing left to reroute exits at once.
//   finish: one workgroup runs whatever rounds remain (normally none).
//   gates:  one wave per token recomputes the gates over its kept slots with
//           the router's arithmetic (so a token that kept all its slots keeps
//           bit-identical gates).
// Acceptance: the pending pairs are taken 1024 at a time in list order; wave
// ballots over the expert id bits give each pair its rank among equal experts
// in the wave, per-wave LDS counts carry it across waves, run[e] across
// chunks.  A rejected pair is written at or before the list slot it was read
// from, after its chunk has been read, so the compaction can run in place.
#include "common.h"
#include "select.h"

#include <climits>

namespace sfl {

constexpr int CAP_WAVES = 16;
constexpr int CAP_THREADS = 64 * CAP_WAVES;
constexpr int CAP_MAX_E = 512;
constexpr int CAP_GATE_WAVES = 4;

// Workspace after the pair list: [CAP_ST_N] state ints, then run[E].
enum { CAP_ST_NREJ = 0, CAP_ST_NDROP = 1, CAP_ST_DONE = 2, CAP_ST_N = 4 };
constexpr int CAP_ROUND_BLOCKS = 64;  // workgroups of a rerouting launch
constexpr int CAP_FAST_ROUNDS = 6;    // rerouting launches before the finisher

struct CapLds {
  int run[CAP_MAX_E];
  int wc[CAP_WAVES][CAP_MAX_E + 1];
  int wrej[CAP_WAVES];
  int ndrop;
  int flag;
};

// One acceptance pass over n entries (the pairs 0..n-1 themselves when
// `first`, list[0..n) otherwise) by a whole 1024-thread workgroup.  Returns
// the number of rejected pairs, now at list[0..nrej) in order.  Entries whose
// pair has index -1 (dropped while rerouting) are skipped; in the first pass
// indices outside [0, E) become -1 and count into L.ndrop.
__device__ int accept_pass(bool first, int n, int E, int ebits, int cap, int32_t* __restrict__ idx,
                           int32_t* __restrict__ list, CapLds& L) {
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int nrej = 0;
  // entries of the next chunk are loaded one chunk ahead; the compaction only
  // writes list slots of the current and earlier chunks
  int pr_next = -1, v_next = -1;
  if ((int)threadIdx.x < n) {
    pr_next = first ? (int)threadIdx.x : list[threadIdx.x];
    v_next = idx[pr_next];
  }
  for (int q0 = 0; q0 < n; q0 += CAP_THREADS) {
    const int pr = pr_next, v = v_next;
    const int inext = q0 + CAP_THREADS + (int)threadIdx.x;
    pr_next = -1;
    v_next = -1;
    if (inext < n) {
      pr_next = first ? inext : list[inext];
      v_next = idx[pr_next];
    }
    int e = E;  // E: sentinel for no pending pair
    bool bad = false;
    if (pr >= 0) {
      if (v >= 0 && v < E) e = v;
      else if (first) bad = true;  // routed to no expert: a dropped pair
    }
    if (bad) idx[pr] = -1;
    const uint64_t bb = __ballot(bad);
    if (lane == 0 && bb) atomicAdd(&L.ndrop, __popcll(bb));
    const bool valid = e < E;
    uint64_t peers = ~0ull;
    for (int bit = 0; bit < ebits; ++bit) {
      const bool set = (e >> bit) & 1;
      const uint64_t bal = __ballot(set);
      peers &= set ? bal : ~bal;
    }
    const int rank_w = __popcll(peers & lt);
    const bool leader = (peers & lt) == 0;
    if (valid && leader) L.wc[wave][e] = __popcll(peers);
    __syncthreads();
    bool rej = false;
    if (valid) {
      int pos = L.run[e] + rank_w;
      for (int w = 0; w < wave; ++w) pos += L.wc[w][e];
      rej = pos >= cap;
    }
    const uint64_t rb = __ballot(rej);
    if (lane == 0) L.wrej[wave] = __popcll(rb);
    __syncthreads();
    int base = nrej, tot = 0;
    for (int w = 0; w < CAP_WAVES; ++w) {
      const int c = L.wrej[w];
      if (w < wave) base += c;
      tot += c;
    }
    if (rej) list[base + __popcll(rb & lt)] = pr;
    if (valid && leader) {
      atomicAdd(&L.run[e], __popcll(peers));
      L.wc[wave][e] = 0;
    }
    nrej += tot;
    __syncthreads();
  }
  return nrej;
}

// Reroute the rejected pairs list[0..n): wave gw of nw handles the token runs
// that start in list[gw*per .. (gw+1)*per), per = ceil(n / nw).  run[] is
// read only; ndrop may live in LDS or global memory.
template <int R>
__device__ void reroute_pass(int n, int gw, int nw, int E, int K, int cap,
                             const float* __restrict__ logits, const float* __restrict__ sbias,
                             int n_groups, int topk_groups, int32_t* __restrict__ idx,
                             const int32_t* __restrict__ list, const int* run, int* ndrop) {
  const int lane = lane_id();
  const int per = (n + nw - 1) / nw;
  const int lo = gw * per;
  const int hi = lo + per < n ? lo + per : n;
  for (int b0 = lo; b0 < hi; b0 += 64) {
    const int i = b0 + lane;
    const int ti = i < hi ? list[i] / K : -1;
    const bool start = i < hi && (i == 0 || list[i - 1] / K != ti);
    uint64_t sm = __ballot(start);
    while (sm) {
      const int b = __builtin_ctzll(sm);
      sm &= sm - 1;
      const int s = b0 + b;
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
      // experts that are not eligible or have no room drop out of the ranking
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int e = r * 64 + lane;
        if (!(e < E && run[e] < cap)) key[r] = -INFINITY;
      }
      for (int l = 0; l < len; ++l) {
        const int k = __shfl(kj, l, 64);
        // experts held by the token's other accepted or pending slots
        const int h = (lane < K && lane != k && !((umask >> lane) & 1ull)) ? cur : -1;
        bool ok[R];
#pragma unroll
        for (int r = 0; r < R; ++r) ok[r] = key[r] != -INFINITY;
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
          if (ne < 0) atomicAdd(ndrop, 1);
        }
      }
    }
  }
}

// First acceptance over all pairs; initialises the state.
__global__ void __launch_bounds__(CAP_THREADS)
capacity_first_kernel(int pairs, int E, int ebits, int cap, int32_t* __restrict__ idx,
                      int32_t* __restrict__ list, int32_t* __restrict__ st) {
  __shared__ CapLds L;
  for (int e = threadIdx.x; e < E; e += CAP_THREADS) {
    L.run[e] = 0;
#pragma unroll
    for (int w = 0; w < CAP_WAVES; ++w) L.wc[w][e] = 0;
  }
  if (threadIdx.x == 0) L.ndrop = 0;
  __syncthreads();
  const int nrej = accept_pass(true, pairs, E, ebits, cap, idx, list, L);
  int* run = st + CAP_ST_N;
  for (int e = threadIdx.x; e < E; e += CAP_THREADS) run[e] = L.run[e];
  if (threadIdx.x == 0) {
    st[CAP_ST_NREJ] = nrej;
    st[CAP_ST_NDROP] = L.ndrop;
    st[CAP_ST_DONE] = 0;
  }
}

// One round: reroute across the grid, then the last workgroup to finish
// accepts the rerouted pairs.
template <int R>
__global__ void __launch_bounds__(CAP_THREADS)
capacity_round_kernel(int E, int K, int ebits, int cap, const float* __restrict__ logits,
                      const float* __restrict__ sbias, int n_groups, int topk_groups,
                      int32_t* __restrict__ idx, int32_t* __restrict__ list, int32_t* __restrict__ st) {
  __shared__ CapLds L;
  const int n = st[CAP_ST_NREJ];
  if (n == 0) return;
  int* run = st + CAP_ST_N;
  const int nw = gridDim.x * CAP_WAVES;
  const int gw = blockIdx.x * CAP_WAVES + (threadIdx.x >> 6);
  reroute_pass<R>(n, gw, nw, E, K, cap, logits, sbias, n_groups, topk_groups, idx, list, run,
                  st + CAP_ST_NDROP);
  __threadfence();  // release this workgroup's index writes before it is counted
  __syncthreads();
  if (threadIdx.x == 0) L.flag = atomicAdd(&st[CAP_ST_DONE], 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!L.flag) return;
  __threadfence();  // acquire every workgroup's writes
  for (int e = threadIdx.x; e < E; e += CAP_THREADS) {
    L.run[e] = run[e];
#pragma unroll
    for (int w = 0; w < CAP_WAVES; ++w) L.wc[w][e] = 0;
  }
  if (threadIdx.x == 0) L.ndrop = 0;
  __syncthreads();
  const int nrej = accept_pass(false, n, E, ebits, cap, idx, list, L);
  for (int e = threadIdx.x; e < E; e += CAP_THREADS) run[e] = L.run[e];
  if (threadIdx.x == 0) {
    st[CAP_ST_NREJ] = nrej;
    st[CAP_ST_DONE] = 0;
  }
}

// Whatever rounds remain, in one workgroup; writes the drop count.
template <int R>
__global__ void __launch_bounds__(CAP_THREADS)
capacity_finish_kernel(int E, int K, int ebits, int cap, const float* __restrict__ logits,
                       const float* __restrict__ sbias, int n_groups, int topk_groups,
                       int32_t* __restrict__ idx, int32_t* __restrict__ list, int32_t* __restrict__ st,
                       int32_t* __restrict__ dropped_out) {
  __shared__ CapLds L;
  int nrej = st[CAP_ST_NREJ];
  if (nrej > 0) {
    const int* grun = st + CAP_ST_N;
    for (int e = threadIdx.x; e < E; e += CAP_THREADS) {
      L.run[e] = grun[e];
#pragma unroll
      for (int w = 0; w < CAP_WAVES; ++w) L.wc[w][e] = 0;
    }
    if (threadIdx.x == 0) L.ndrop = st[CAP_ST_NDROP];
    __syncthreads();
    for (int round = 0; nrej > 0 && round <= E; ++round) {
      reroute_pass<R>(nrej, threadIdx.x >> 6, CAP_WAVES, E, K, cap, logits, sbias, n_groups, topk_groups,
                      idx, list, L.run, &L.ndrop);
      __syncthreads();
      nrej = accept_pass(false, nrej, E, ebits, cap, idx, list, L);
    }
    // Unreachable by the round bound above; kept so that every pair ends in
    // a defined state whatever the input.
    for (int i = threadIdx.x; i < nrej; i += CAP_THREADS) {
      idx[list[i]] = -1;
      atomicAdd(&L.ndrop, 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      st[CAP_ST_NDROP] = L.ndrop;
      st[CAP_ST_NREJ] = 0;
    }
  }
  if (threadIdx.x == 0 && dropped_out != nullptr) dropped_out[0] = st[CAP_ST_NDROP];
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
size_t capacity_scratch_ints(int64_t pairs, int E) { return (size_t)pairs + CAP_ST_N + (size_t)E; }

hipError_t launch_capacity(const Problem& p, int cap, const float* logits, const float* sb,
                           int32_t* idx, float* gate, int32_t* dropped, int32_t* scratch,
                           hipStream_t st) {
  const int pairs = (int)(p.S * p.K);
  const int c = cap > 0 ? cap : INT_MAX;  // 0: no limit
  int ebits = 0;
  while ((1 << ebits) <= p.E) ++ebits;  // enough bits for 0..E (E is the sentinel)
  int32_t* list = scratch;
  int32_t* state = scratch + pairs;
  capacity_first_kernel<<<1, CAP_THREADS, 0, st>>>(pairs, p.E, ebits, c, idx, list, state);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const int R = (p.E + 63) / 64;
  const dim3 gg((unsigned)ceil_div(p.S, CAP_GATE_WAVES)), gb(64 * CAP_GATE_WAVES);
#define SFL_CAP(RR)                                                                                  \
  for (int f = 0; f < CAP_FAST_ROUNDS; ++f) {                                                        \
    capacity_round_kernel<RR><<<CAP_ROUND_BLOCKS, CAP_THREADS, 0, st>>>(                             \
        p.E, p.K, ebits, c, logits, sb, p.n_groups, p.topk_groups, idx, list, state);               \
    if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;                               \
  }                                                                                                  \
  capacity_finish_kernel<RR><<<1, CAP_THREADS, 0, st>>>(p.E, p.K, ebits, c, logits, sb, p.n_groups,  \
                                                        p.topk_groups, idx, list, state, dropped);   \
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;                                 \
  capacity_gates_kernel<RR><<<gg, gb, 0, st>>>(p.S, p.E, p.K, p.renormalize, p.inv_tau, logits,       \
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
