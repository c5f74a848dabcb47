// Internal helpers shared by the HIP kernels of the MoE layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfl {

// ------------------------------------------------------------------ problem
struct Problem {
  int64_t S;
  int d, d_ff, E, K;
  int n_groups, topk_groups, renormalize;
  int act, w;  // moe_dtype values
  float inv_tau;  // 1 / gate temperature
  int capacity;   // per-expert limit of (token, slot) pairs, 0 = none
  int act_quant;  // 1: e4m3 activations with per-row scales in the expert products
};

enum { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline int64_t ceil_div(int64_t v, int64_t m) { return (v + m - 1) / m; }

// ------------------------------------------------------------------ types
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Round-to-nearest-even float -> bfloat16 (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

// GeLU(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt 2)), the erf form, written
// as  max(x, 0) - |x|/2 * erfc(|x| / sqrt 2)  (the same function; the small
// term is a product, so negative x loses nothing to cancellation).  erfc is
// evaluated with Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26 (|error| <= 1.5e-7 for z >= 0):
//   erfc(z) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2),
//   t = 1 / (1 + p z),
// with z = |x| / sqrt 2 folded into p and into the exponent, and the 1/2 into
// the a_i.  About 12 VALU operations (two of them transcendental) per value,
// less than half of a general-purpose erff.  |x| is capped at 2^16 in the
// small term so that x = +inf gives +inf (that term is 0 there).
__device__ __forceinline__ float gelu_erf(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.2316418882663604f, ax, 1.0f));  // p / sqrt 2
  float q = fmaf(t, 0.5307027145f, -0.7265760135f);                              // a5/2, a4/2
  q = fmaf(t, q, 0.7107068705f);                                                 // a3/2
  q = fmaf(t, q, -0.142248368f);                                                 // a2/2
  q = fmaf(t, q, 0.127414796f);                                                  // a1/2
  const float w = (fminf(ax, 65536.0f) * t) * q;
  const float e = __builtin_amdgcn_exp2f((x * x) * -0.7213475204444817f);       // exp(-x^2 / 2)
  return fmaf(-w, e, fmaxf(x, 0.0f));
}

// ------------------------------------------------------------------ waves
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
// (value desc, index asc) arg-max over the wave; every lane gets the winner.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}

// ------------------------------------------------------------------ e4m3 rows
// Four float32 values -> four OCP e4m3 codes (round to nearest even), value 0
// in the low byte.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.f), 448.f); }

// Eight bf16 values (one 16-byte chunk) times pre, then times r, clamped,
// as e4m3 codes.  pre is 1 or 2^64 (exact either way).
__device__ __forceinline__ uint2 e4m3x8_scaled(uint4 raw, float pre, float r) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = clamp448((bf16_bits_to_f32(w[q] & 0xffff) * pre) * r);
    v[2 * q + 1] = clamp448((bf16_bits_to_f32(w[q] >> 16) * pre) * r);
  }
  return make_uint2(e4m3x4(v[0], v[1], v[2], v[3]), e4m3x4(v[4], v[5], v[6], v[7]));
}
__device__ __forceinline__ float chunk_amax(uint4 raw, float amax) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] & 0xffff)));
    amax = fmaxf(amax, fabsf(bf16_bits_to_f32(w[q] >> 16)));
  }
  return amax;
}

// r = 448 / amax, or 448 / (amax 2^64) with pre = 2^64 where the first
// quotient overflows; amax = 0 gives r = 0.
__device__ __forceinline__ float row_factor(float amax, float& pre) {
  pre = 1.f;
  if (!(amax > 0.f)) return 0.f;
  const float r = 448.f / amax;
  if (!__builtin_isinf(r)) return r;
  pre = 0x1p64f;
  return 448.f / (amax * pre);
}

// One row of n bf16 values (n % 8 == 0) -> e4m3 codes and one float32 scale,
// by the whole wave:  amax = max |v|,  scale = amax / 448,  r = 448 / amax,
// code = e4m3(clamp(v * r, -448, 448)); a row of zeros gets scale 0 and
// codes 0.  Each quotient and product is one float32 operation, so the codes
// are a function of the bf16 inputs alone.  When 448 / amax overflows
// float32 (amax below about 1.3e-36) the row and amax are first multiplied
// by 2^64, exactly: r = 448 / (amax 2^64), code = e4m3(clamp((v 2^64) r)),
// the codes an unbounded exponent range would give.  Rows of up to 512 R values are
// read once, all of a lane's chunks in flight together, and held in
// registers for the second step; longer rows are read twice (the second
// time from cache).
template <int R>
__device__ __forceinline__ void wave_quantize_row_e4m3(const uint16_t* __restrict__ s, int n,
                                                       uint8_t* __restrict__ d, float* __restrict__ scale_out) {
  const int lane = lane_id();
  float amax = 0.f, scale, r, pre;
  if (n <= 64 * 8 * R) {
    uint4 raw[R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = (i * 64 + lane) * 8;
      raw[i] = c < n ? *reinterpret_cast<const uint4*>(s + c) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < R; ++i) amax = chunk_amax(raw[i], amax);
    amax = wave_max(amax);
    scale = amax / 448.f;
    r = row_factor(amax, pre);
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = (i * 64 + lane) * 8;
      if (c < n) *reinterpret_cast<uint2*>(d + c) = amax > 0.f ? e4m3x8_scaled(raw[i], pre, r) : make_uint2(0u, 0u);
    }
  } else {
    for (int c = lane * 8; c < n; c += 64 * 8) amax = chunk_amax(*reinterpret_cast<const uint4*>(s + c), amax);
    amax = wave_max(amax);
    scale = amax / 448.f;
    r = row_factor(amax, pre);
    for (int c = lane * 8; c < n; c += 64 * 8) {
      const uint4 raw = *reinterpret_cast<const uint4*>(s + c);
      *reinterpret_cast<uint2*>(d + c) = amax > 0.f ? e4m3x8_scaled(raw, pre, r) : make_uint2(0u, 0u);
    }
  }
  if (lane == 0) *scale_out = scale;
}

// ------------------------------------------------------------------ sync
// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait until at most N LDS (and scalar-memory) operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier that orders LDS traffic but does not drain global loads.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void_t;

// 16-byte global -> LDS copy through the load path (no VGPR staging).  Lane i
// of the wave writes LDS bytes [lds_base + 16 i, lds_base + 16 i + 16); the
// LDS base must be the same for every lane of the wave.
__device__ __forceinline__ void load_lds_16(const void* gptr, void* lds_base) {
  __builtin_amdgcn_global_load_lds(gptr, (lds_void_t*)lds_base, 16, 0, 0);
}

// Buffer resource for raw byte addressing (gfx9 layout): 48-bit base, stride
// 0, num_records bytes, word 3 = 32-bit data format.  The base must be
// uniform across the wave (it lives in scalar registers).
typedef int i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  i32x4_t r;
  r.x = (int)(uint32_t)a;
  r.y = (int)(uint32_t)((a >> 32) & 0xffffu);
  r.z = (int)num_records;
  r.w = 0x00020000;
  return r;
}
// 16-byte buffer load straight into LDS: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) (the LDS base is uniform); the global byte
// address is base + voffset + soffset.
__device__ void llvm_amdgcn_raw_buffer_load_lds(i32x4_t rsrc, lds_void_t* lds, int size, int voffset, int soffset,
                                                int offset, int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
// AUX = cache policy bits; 2 marks the load non-temporal ("nt": data read
// once, streamed past the caches' normal retention).
template <int AUX = 0>
__device__ __forceinline__ void buffer_load_lds_16(i32x4_t rsrc, void* lds_base, uint32_t voffset, uint32_t soffset) {
  llvm_amdgcn_raw_buffer_load_lds(rsrc, (lds_void_t*)lds_base, 16, (int)voffset, (int)soffset, 0, AUX);
}

// 16-byte global -> VGPR load through a buffer resource (range-checked:
// bytes past num_records read as zero, with no memory access).
__device__ i32x4_t llvm_amdgcn_raw_buffer_load_v4i32(i32x4_t rsrc, int voffset, int soffset, int aux)
    __asm("llvm.amdgcn.raw.buffer.load.v4i32");
__device__ __forceinline__ i32x4_t buffer_load_16(i32x4_t rsrc, uint32_t voffset, uint32_t soffset) {
  return llvm_amdgcn_raw_buffer_load_v4i32(rsrc, (int)voffset, (int)soffset, 0);
}

}  // namespace sfl
