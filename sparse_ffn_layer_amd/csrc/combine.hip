// Combine: gate-weighted sum of each token's K expert outputs, back in token
// order.
//
// Chapter "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), section 11.1.1:
// the layer output is the router-weighted sum of the chosen experts' outputs;
// section 11.2.1: expert outputs are put back in the tokens' original order.
// "MoE 混合专家推理" (plumephp.com), one MoE forward: the chosen experts'
// results are weighted by their scores and added.
//
// One block per token: each lane owns 16-byte column chunks of the token's
// row, reads its K rows of y_perm (through inv_perm) in slot order and
// accumulates in float32 with no atomics, so the result does not depend on
// scheduling or on how the row is split over lanes.  DeepSeek shape
// (d = 7168, K = 8, 470 MB of y_perm): 0.114 -> 0.099 ms with non-temporal
// loads and a block size that divides the row.
#include "common.h"

namespace sfl {

template <int NT, bool BF16, bool NTL>
__global__ void __launch_bounds__(NT)
combine_kernel(int64_t S, int K, int row_vecs, const uint4* __restrict__ y_perm,
               const int32_t* __restrict__ inv_perm, const float* __restrict__ gate,
               uint4* __restrict__ y) {
  const int64_t t = blockIdx.x;
  if (t >= S) return;
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  for (int i = threadIdx.x; i < row_vecs; i += NT) {
    float acc[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int64_t row = inv_perm[t * K + k];
      if (row < 0) continue;  // pair dropped by the dispatch
      const float g = gate[t * K + k];
      // every row of y_perm is read once: non-temporal loads when it does
      // not fit the last-level cache anyway (NTL)
      const uint4* src = y_perm + row * row_vecs + i;
      uint4 v;
      if constexpr (NTL) v = __builtin_bit_cast(uint4, __builtin_nontemporal_load((const i32x4_t*)src));
      else v = *src;
      if constexpr (BF16) {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] = fmaf(g, bf16_bits_to_f32(w[q] & 0xffff), acc[2 * q]);
          acc[2 * q + 1] = fmaf(g, bf16_bits_to_f32(w[q] >> 16), acc[2 * q + 1]);
        }
      } else {
        acc[0] = fmaf(g, __uint_as_float(v.x), acc[0]);
        acc[1] = fmaf(g, __uint_as_float(v.y), acc[1]);
        acc[2] = fmaf(g, __uint_as_float(v.z), acc[2]);
        acc[3] = fmaf(g, __uint_as_float(v.w), acc[3]);
      }
    }
    uint4 o;
    if constexpr (BF16) {
      o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                     __float_as_uint(acc[3]));
    }
    y[t * row_vecs + i] = o;
  }
}

template <int NT>
static void launch_nt(bool bf, bool ntl, const Problem& p, int row_vecs, const void* y_perm,
                      const int32_t* inv_perm, const float* gate, void* y, hipStream_t st) {
  const unsigned grid = (unsigned)p.S;  // one block per token
  const uint4* src = (const uint4*)y_perm;
  uint4* dst = (uint4*)y;
  if (bf && ntl) combine_kernel<NT, true, true><<<grid, NT, 0, st>>>(p.S, p.K, row_vecs, src, inv_perm, gate, dst);
  else if (bf) combine_kernel<NT, true, false><<<grid, NT, 0, st>>>(p.S, p.K, row_vecs, src, inv_perm, gate, dst);
  else if (ntl) combine_kernel<NT, false, true><<<grid, NT, 0, st>>>(p.S, p.K, row_vecs, src, inv_perm, gate, dst);
  else combine_kernel<NT, false, false><<<grid, NT, 0, st>>>(p.S, p.K, row_vecs, src, inv_perm, gate, dst);
}

hipError_t launch_combine(const Problem& p, const void* y_perm, const int32_t* inv_perm,
                          const float* gate, void* y, hipStream_t st) {
  const bool bf = p.act == DT_BF16;
  const int row_vecs = p.d * (bf ? 2 : 4) / 16;
  // y_perm larger than the 256 MB last-level cache: its rows come from HBM
  // whatever the load, and non-temporal loads keep them from evicting the
  // rest (smaller ones are still in that cache after the down product, and
  // plain loads are faster there)
  const bool ntl = (int64_t)p.S * p.K * row_vecs * 16 > ((int64_t)256 << 20);
  // threads per block: 256, or a multiple of 64 that divides the row's
  // 16-byte chunks when 256 does not, so that no lane idles in the last pass
  // (DeepSeek shape, d = 7168: 896 chunks, 448 threads)
  if (row_vecs % 256 == 0) launch_nt<256>(bf, ntl, p, row_vecs, y_perm, inv_perm, gate, y, st);
  else if (row_vecs % 448 == 0) launch_nt<448>(bf, ntl, p, row_vecs, y_perm, inv_perm, gate, y, st);
  else if (row_vecs % 384 == 0) launch_nt<384>(bf, ntl, p, row_vecs, y_perm, inv_perm, gate, y, st);
  else if (row_vecs % 320 == 0) launch_nt<320>(bf, ntl, p, row_vecs, y_perm, inv_perm, gate, y, st);
  else launch_nt<256>(bf, ntl, p, row_vecs, y_perm, inv_perm, gate, y, st);
  return hipGetLastError();
}

}  // namespace sfl
