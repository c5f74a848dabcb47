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
// scheduling or on how the row is split over lanes.
#include "common.h"

namespace sfl {

constexpr int COMBINE_WAVES = 4;

template <bool BF16>
__global__ void __launch_bounds__(64 * COMBINE_WAVES)
combine_kernel(int64_t S, int K, int row_vecs, const uint4* __restrict__ y_perm,
               const int32_t* __restrict__ inv_perm, const float* __restrict__ gate,
               uint4* __restrict__ y) {
  const int64_t t = blockIdx.x;
  if (t >= S) return;
  constexpr int EPV = BF16 ? 8 : 4;  // elements per 16-byte vector
  for (int i = threadIdx.x; i < row_vecs; i += 64 * COMBINE_WAVES) {
    float acc[EPV];
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int64_t row = inv_perm[t * K + k];
      if (row < 0) continue;  // pair dropped by the dispatch
      const float g = gate[t * K + k];
      const uint4 v = y_perm[row * row_vecs + i];
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

hipError_t launch_combine(const Problem& p, const void* y_perm, const int32_t* inv_perm,
                          const float* gate, void* y, hipStream_t st) {
  const bool bf = p.act == DT_BF16;
  const int row_vecs = p.d * (bf ? 2 : 4) / 16;
  const unsigned grid = (unsigned)p.S;  // one block per token
  if (bf)
    combine_kernel<true><<<grid, 64 * COMBINE_WAVES, 0, st>>>(p.S, p.K, row_vecs, (const uint4*)y_perm,
                                                             inv_perm, gate, (uint4*)y);
  else
    combine_kernel<false><<<grid, 64 * COMBINE_WAVES, 0, st>>>(p.S, p.K, row_vecs, (const uint4*)y_perm,
                                                              inv_perm, gate, (uint4*)y);
  return hipGetLastError();
}

}  // namespace sfl
