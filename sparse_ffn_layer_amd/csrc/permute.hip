// Dispatch: regroup (token, slot) pairs into expert-contiguous, tile-padded
// row groups and gather the token rows.
//
// Chapter "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), section 11.2.1:
// after routing, the tokens of one expert must be gathered together before
// the expert runs, and the outputs are put back in token order afterwards;
// section 11.1.2: the S x K expert forwards are grouped per expert.
// "MoE 推理工程深层实战" (ybb.press), section 2.2: sizing receive buffers from
// the data costs a host synchronisation; here every size is computed on the
// device and the host launches fixed grids.
//
// Pairs p = t*K + k keep token order inside an expert (stable), so the
// grouping is unique and bit-reproducible:
//   1. count:   each block histograms its contiguous chunk of pairs in LDS.
//   2. scan:    one block turns the [E][blocks] histogram into per-block
//               starting ranks, and the per-expert totals into dense and
//               tile-padded offsets.
//   3. scatter: each block ranks its pairs in order (wave ballots give the
//               rank among equal experts inside a wave, LDS counters carry
//               the rank across waves and rounds) and writes perm/inv_perm.
//   4. gather:  x_perm[inv_perm[p]] = x[p / K], one wave per row; or, for a
//               product that reads the token rows of x itself, the row ->
//               token map row_tok[inv_perm[p]] = p / K written in step 3.
// When all pairs fit one block, steps 1-3 run as one single-block kernel.
#include "common.h"

namespace sfl {

constexpr int PERM_THREADS = 256;
constexpr int PERM_MAX_E = 512;
constexpr int SCAN_THREADS = 1024;
constexpr int SCAN_LDS_INTS = 15360;  // histogram entries staged in LDS by the scan (<= 64 KiB in all)

// Number of count/scatter blocks for S*K pairs: ~1024 pairs per block, and
// E * blocks small enough for the scan to stage in LDS.
int permute_blocks(int64_t pairs, int E) {
  int64_t nb = ceil_div(pairs, 1024);
  int64_t cap = SCAN_LDS_INTS / E;
  if (nb > cap) nb = cap;
  return nb < 1 ? 1 : (int)nb;
}

__global__ void __launch_bounds__(PERM_THREADS)
permute_count_kernel(const int32_t* __restrict__ idx, int64_t pairs, int E, int64_t chunk,
                     int32_t* __restrict__ hist) {
  __shared__ int cnt[PERM_MAX_E];
  const int nb = gridDim.x, b = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) cnt[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)b * chunk;
  const int64_t p1 = p0 + chunk < pairs ? p0 + chunk : pairs;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += PERM_THREADS) {
    const unsigned e = (unsigned)idx[p];
    if (e < (unsigned)E) atomicAdd(&cnt[e], 1);  // ids outside [0, E) are ignored
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) hist[(int64_t)e * nb + b] = cnt[e];
}

// Single block.  hist[e][b] (counts) becomes the number of expert-e pairs in
// blocks before b.  counts[e], dense[e] (exclusive scan of counts) and
// offsets[e] (exclusive scan of counts rounded up to tile_m) are written for
// e in [0, E], with the totals in entry E.
__global__ void __launch_bounds__(SCAN_THREADS)
permute_scan_kernel(int E, int nb, int tile_m, int32_t* __restrict__ hist,
                    int32_t* __restrict__ counts, int32_t* __restrict__ dense,
                    int32_t* __restrict__ offsets) {
  extern __shared__ int lds[];  // E * nb histogram entries, then 2 * E scan space
  int* h = lds;
  int* tot = lds + E * nb;
  const int n = E * nb;
  for (int i = threadIdx.x; i < n; i += SCAN_THREADS) h[i] = hist[i];
  __syncthreads();
  // per-expert exclusive scan over blocks, one wave per expert at a time
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int e = wave; e < E; e += SCAN_THREADS / 64) {
    int carry = 0;
    for (int b0 = 0; b0 < nb; b0 += 64) {
      const int b = b0 + lane;
      const int v = b < nb ? h[e * nb + b] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      if (b < nb) h[e * nb + b] = carry + incl - v;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) tot[e] = carry;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += SCAN_THREADS) hist[i] = h[i];
  // scan over experts (E <= 512): wave 0 in chunks of 64
  if (wave == 0) {
    int cd = 0, cp = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? tot[e] : 0;
      const int cpad = (c + tile_m - 1) / tile_m * tile_m;
      int id = c, ip = cpad;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(id, o, 64), w = __shfl_up(ip, o, 64);
        if (lane >= o) { id += u; ip += w; }
      }
      if (e < E) {
        counts[e] = c;
        dense[e] = cd + id - c;
        offsets[e] = cp + ip - cpad;
      }
      cd += __shfl(id, 63, 64);
      cp += __shfl(ip, 63, 64);
    }
    if (lane == 0) { dense[E] = cd; offsets[E] = cp; }
  }
}

__global__ void __launch_bounds__(PERM_THREADS)
permute_scatter_kernel(const int32_t* __restrict__ idx, int64_t pairs, int E, int ebits,
                       int64_t chunk, const int32_t* __restrict__ base,
                       const int32_t* __restrict__ dense, const int32_t* __restrict__ offsets,
                       int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, int K,
                       int32_t* __restrict__ row_tok) {
  __shared__ int run[PERM_MAX_E];
  __shared__ int wc[PERM_THREADS / 64][PERM_MAX_E + 1];
  const int nb = gridDim.x, b = blockIdx.x;
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) {
    run[e] = base[(int64_t)e * nb + b];
#pragma unroll
    for (int w = 0; w < PERM_THREADS / 64; ++w) wc[w][e] = 0;
  }
  __syncthreads();
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int64_t p0 = (int64_t)b * chunk;
  const int64_t p1 = p0 + chunk < pairs ? p0 + chunk : pairs;
  for (int64_t q0 = p0; q0 < p1; q0 += PERM_THREADS) {
    const int64_t p = q0 + threadIdx.x;
    int e = p < p1 ? idx[p] : E;
    if (e < 0 || e > E) e = E;          // E: sentinel for lanes past the end and bad ids
    const bool valid = e < E;
    if (p < p1 && !valid) inv_perm[p] = -1;
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
    if (valid) {
      int pos = run[e] + rank_w;
      for (int w = 0; w < wave; ++w) pos += wc[w][e];
      perm[dense[e] + pos] = (int32_t)p;
      inv_perm[p] = offsets[e] + pos;
      if (row_tok != nullptr) row_tok[offsets[e] + pos] = (int32_t)(p / K);
    }
    __syncthreads();
    if (valid && leader) {
      atomicAdd(&run[e], __popcll(peers));
      wc[wave][e] = 0;
    }
    __syncthreads();
  }
}

// All pairs in one block (a small batch): count, scan and scatter in one
// workgroup -- the steps above without their cross-block parts -- so a
// decode step pays one launch instead of three.
__global__ void __launch_bounds__(PERM_THREADS)
permute_single_kernel(const int32_t* __restrict__ idx, int64_t pairs, int E, int ebits, int tile_m,
                      int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                      int32_t* __restrict__ perm, int32_t* __restrict__ inv_perm, int K,
                      int32_t* __restrict__ row_tok) {
  __shared__ int run[PERM_MAX_E];
  __shared__ int dns[PERM_MAX_E];
  __shared__ int ofs[PERM_MAX_E];
  __shared__ int wc[PERM_THREADS / 64][PERM_MAX_E + 1];
  const int lane = lane_id(), wave = threadIdx.x >> 6;
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) {
    run[e] = 0;
#pragma unroll
    for (int w = 0; w < PERM_THREADS / 64; ++w) wc[w][e] = 0;
  }
  __syncthreads();
  // 1. histogram (ids outside [0, E) are ignored)
  for (int64_t p = threadIdx.x; p < pairs; p += PERM_THREADS) {
    const unsigned e = (unsigned)idx[p];
    if (e < (unsigned)E) atomicAdd(&run[e], 1);
  }
  __syncthreads();
  // 2. dense and tile-padded exclusive scans over the experts (wave 0)
  if (wave == 0) {
    int cd = 0, cp = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + lane;
      const int c = e < E ? run[e] : 0;
      const int cpad = (c + tile_m - 1) / tile_m * tile_m;
      int id = c, ip = cpad;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(id, o, 64), w = __shfl_up(ip, o, 64);
        if (lane >= o) { id += u; ip += w; }
      }
      if (e < E) {
        counts[e] = c;
        dns[e] = cd + id - c;
        ofs[e] = cp + ip - cpad;
        offsets[e] = cp + ip - cpad;
      }
      cd += __shfl(id, 63, 64);
      cp += __shfl(ip, 63, 64);
    }
    if (lane == 0) offsets[E] = cp;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += PERM_THREADS) run[e] = 0;
  __syncthreads();
  // 3. stable ranks in pair order (as permute_scatter_kernel with one block)
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t q0 = 0; q0 < pairs; q0 += PERM_THREADS) {
    const int64_t p = q0 + threadIdx.x;
    int e = p < pairs ? idx[p] : E;
    if (e < 0 || e > E) e = E;  // E: sentinel for lanes past the end and bad ids
    const bool valid = e < E;
    if (p < pairs && !valid) inv_perm[p] = -1;
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
    if (valid) {
      int pos = run[e] + rank_w;
      for (int w = 0; w < wave; ++w) pos += wc[w][e];
      perm[dns[e] + pos] = (int32_t)p;
      inv_perm[p] = ofs[e] + pos;
      if (row_tok != nullptr) row_tok[ofs[e] + pos] = (int32_t)(p / K);
    }
    __syncthreads();
    if (valid && leader) {
      atomicAdd(&run[e], __popcll(peers));
      wc[wave][e] = 0;
    }
    __syncthreads();
  }
}

// x_perm[inv_perm[p]] = x[p / K]; one wave per pair, 16-byte copies.
__global__ void __launch_bounds__(PERM_THREADS)
gather_rows_kernel(const uint4* __restrict__ x, int64_t pairs, int K, int row_vecs,
                   const int32_t* __restrict__ inv_perm, uint4* __restrict__ x_perm) {
  const int64_t p = (int64_t)blockIdx.x * (PERM_THREADS / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (p >= pairs) return;
  const int64_t t = p / K;
  const int64_t row = inv_perm[p];
  if (row < 0) return;  // pair with an out-of-range expert id
  const uint4* src = x + t * row_vecs;
  uint4* dst = x_perm + row * row_vecs;
  for (int i = lane_id(); i < row_vecs; i += 64) dst[i] = src[i];
}

// ------------------------------------------------------------------ launchers
size_t permute_scratch_ints(int64_t pairs, int E) {
  return (size_t)E * permute_blocks(pairs, E) + (size_t)E + 1;
}

// row_tok (nullable): also write, for every row of the expert groups, the
// token it holds (row_tok[inv_perm[p]] = p / K), so that a product can read
// the token rows of x in place of a gathered x_perm.
hipError_t launch_permute(const Problem& p, int tile_m, const int32_t* idx, const void* x,
                          int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* inv_perm,
                          void* x_perm, int32_t* scratch, hipStream_t st, int32_t* row_tok) {
  const int64_t pairs = p.S * p.K;
  const int nb = permute_blocks(pairs, p.E);
  const int64_t chunk = ceil_div(pairs, nb);
  int32_t* hist = scratch;
  int32_t* dense = scratch + (size_t)p.E * nb;
  int ebits = 0;
  while ((1 << ebits) <= p.E) ++ebits;  // enough bits for 0..E (E is the sentinel)

  hipError_t err;
  if (nb == 1) {
    permute_single_kernel<<<1, PERM_THREADS, 0, st>>>(idx, pairs, p.E, ebits, tile_m, counts, offsets, perm,
                                                      inv_perm, p.K, row_tok);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else {
    permute_count_kernel<<<nb, PERM_THREADS, 0, st>>>(idx, pairs, p.E, chunk, hist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const size_t lds = ((size_t)p.E * nb + 2 * (size_t)p.E) * sizeof(int);
    permute_scan_kernel<<<1, SCAN_THREADS, lds, st>>>(p.E, nb, tile_m, hist, counts, dense, offsets);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    permute_scatter_kernel<<<nb, PERM_THREADS, 0, st>>>(idx, pairs, p.E, ebits, chunk, hist, dense,
                                                       offsets, perm, inv_perm, p.K, row_tok);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (x_perm != nullptr) {
    const int esz = p.act == DT_F32 ? 4 : 2;
    const int row_vecs = p.d * esz / 16;
    const unsigned g = (unsigned)ceil_div(pairs, PERM_THREADS / 64);
    gather_rows_kernel<<<g, PERM_THREADS, 0, st>>>((const uint4*)x, pairs, p.K, row_vecs, inv_perm,
                                                  (uint4*)x_perm);
    err = hipGetLastError();
  }
  return err;
}

}  // namespace sfl
