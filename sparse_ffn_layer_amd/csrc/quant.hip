// Per-row fp8 (OCP e4m3) quantisation of bf16 activations, for the W8A8
// expert products.
//
// "MoE 推理工程深层实战" (ybb.press), section 3.3: FP8 E4M3 is the production
// format for experts, with a precision loss the page calls negligible.  Here
// both operands of each expert product are e4m3: the weights as stored, the
// activations quantised per row just before the product that reads them:
//   amax = max |v| over the row,  s = amax / 448,  r = 448 / amax,
//   code = e4m3(clamp(v * r, -448, 448))  (round to nearest even),
// and the row's value is decode(code) * s; a row of zeros gets s = 0 and
// codes 0.  Each quotient and product is one float32 operation, so the codes
// are a function of the bf16 inputs alone.
//
// One wave per row: a pass over the row for amax, a second (from cache) for
// the codes, 16 bytes of bf16 in and 8 bytes of codes out per lane and step.
#include "common.h"

namespace sfl {

constexpr int QUANT_WAVES = 4;

// Four float32 values -> four e4m3 codes, value 0 in the low byte.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Rows to quantise: pair p (of `pairs`) reads source row src_row(p) and
// writes destination row dst_row(p):
//   gather (x -> x_perm):  src = p / K (the token),  dst = inv_perm[p]
//   in place (h -> h8):    src = dst = inv_perm[p]
//   plain (rows given):    src = dst = p  (inv_perm == null)
// Pairs whose inv_perm entry is negative are skipped.  n % 8 == 0.
__global__ void __launch_bounds__(64 * QUANT_WAVES)
quantize_rows_kernel(const uint16_t* __restrict__ src, int64_t ld_src, int n, int64_t pairs, int K, bool gather,
                     const int32_t* __restrict__ inv_perm, uint8_t* __restrict__ dst, int64_t ld_dst,
                     float* __restrict__ scales) {
  const int64_t p = (int64_t)blockIdx.x * QUANT_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (p >= pairs) return;
  const int lane = lane_id();
  int64_t drow = p, srow = p;
  if (inv_perm != nullptr) {
    drow = inv_perm[p];
    if (drow < 0) return;
    srow = gather ? p / K : drow;
  }
  const uint16_t* s = src + srow * ld_src;
  float amax = 0.f;
  for (int c = lane * 8; c < n; c += 64 * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(s + c);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] & 0xffff)));
      amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] >> 16)));
    }
  }
  amax = wave_max(amax);
  const float scale = amax / 448.f;
  const float r = amax > 0.f ? 448.f / amax : 0.f;
  uint8_t* d = dst + drow * ld_dst;
  for (int c = lane * 8; c < n; c += 64 * 8) {
    const uint4 raw = *reinterpret_cast<const uint4*>(s + c);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[2 * q] = clamp448(bf16_bits_to_f32(w[q] & 0xffff) * r);
      v[2 * q + 1] = clamp448(bf16_bits_to_f32(w[q] >> 16) * r);
    }
    uint2 out;
    out.x = amax > 0.f ? e4m3x4(v[0], v[1], v[2], v[3]) : 0u;
    out.y = amax > 0.f ? e4m3x4(v[4], v[5], v[6], v[7]) : 0u;
    *reinterpret_cast<uint2*>(d + c) = out;
  }
  if (lane == 0) scales[drow] = scale;
}

hipError_t launch_quantize_rows(const uint16_t* src, int64_t ld_src, int n, int64_t pairs, int K, bool gather,
                                const int32_t* inv_perm, uint8_t* dst, int64_t ld_dst, float* scales,
                                hipStream_t st) {
  if (pairs == 0) return hipSuccess;
  const unsigned g = (unsigned)ceil_div(pairs, QUANT_WAVES);
  quantize_rows_kernel<<<g, 64 * QUANT_WAVES, 0, st>>>(src, ld_src, n, pairs, K, gather, inv_perm, dst, ld_dst,
                                                       scales);
  return hipGetLastError();
}

}  // namespace sfl
