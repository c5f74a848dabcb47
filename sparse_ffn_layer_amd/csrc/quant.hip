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
// are a function of the bf16 inputs alone.  Where 448 / amax overflows
// float32 (amax below about 1.3e-36) the row and amax are first multiplied
// by 2^64, which is exact, so such rows get the codes an unbounded exponent
// range would give.
//
// One wave per row (wave_quantize_row_e4m3 in common.h).
#include "common.h"

namespace sfl {

constexpr int QUANT_WAVES = 4;

// Rows to quantise: pair p (of `pairs`) reads source row src_row(p) and
// writes destination row dst_row(p):
//   gather (x -> x_perm):  src = p / K (the token),  dst = inv_perm[p]
//   in place (h -> h8):    src = dst = inv_perm[p]
//   plain (rows given):    src = dst = p  (inv_perm == null)
// Pairs whose inv_perm entry is negative are skipped.  n % 8 == 0.
template <int R>
__global__ void __launch_bounds__(64 * QUANT_WAVES)
quantize_rows_kernel(const uint16_t* __restrict__ src, int64_t ld_src, int n, int64_t pairs, int K, bool gather,
                     const int32_t* __restrict__ inv_perm, uint8_t* __restrict__ dst, int64_t ld_dst,
                     float* __restrict__ scales) {
  const int64_t p = (int64_t)blockIdx.x * QUANT_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (p >= pairs) return;
  int64_t drow = p, srow = p;
  if (inv_perm != nullptr) {
    drow = inv_perm[p];
    if (drow < 0) return;
    srow = gather ? p / K : drow;
  }
  wave_quantize_row_e4m3<R>(src + srow * ld_src, n, dst + drow * ld_dst, scales + drow);
}

hipError_t launch_quantize_rows(const uint16_t* src, int64_t ld_src, int n, int64_t pairs, int K, bool gather,
                                const int32_t* inv_perm, uint8_t* dst, int64_t ld_dst, float* scales,
                                hipStream_t st) {
  if (pairs == 0) return hipSuccess;
  const unsigned g = (unsigned)ceil_div(pairs, QUANT_WAVES);
  // R 16-byte chunks per lane held in registers: the smallest instance that
  // holds the whole row (rows of up to 512 R values are read once), so short
  // rows keep the registers per wave low and many waves resident
  auto kern = quantize_rows_kernel<16>;
  if (n <= 64 * 8 * 2) kern = quantize_rows_kernel<2>;
  else if (n <= 64 * 8 * 4) kern = quantize_rows_kernel<4>;
  else if (n <= 64 * 8 * 8) kern = quantize_rows_kernel<8>;
  kern<<<g, 64 * QUANT_WAVES, 0, st>>>(src, ld_src, n, pairs, K, gather, inv_perm, dst, ld_dst, scales);
  return hipGetLastError();
}

}  // namespace sfl
