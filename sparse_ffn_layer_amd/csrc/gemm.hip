// Grouped GEMM over expert-contiguous rows: the expert FFN and the router
// product.
//
// Chapter "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com), section 11.1.2:
// every expert is GeLU(x W1 + b1) W2 + b2 with the same shape and its own
// weights, and the S x K expert forwards are run grouped per expert; section
// 11.4.1: all experts' weights stay resident and are visited in expert order;
// "MoE 混合专家推理" (plumephp.com), activation-memory block: running a whole
// batch through one expert turns many small products into one large GEMM.
//
// out[r][n] = epilogue( sum_k A[r][k] * B_g[n][k] )  for the rows r of group g
//   A    : activations, bf16, row-major [rows][K]
//   B_g  : weights of group g in linear-layer layout [N][K] (bf16 or OCP
//          e4m3 fp8, converted exactly to bf16 on the way into the MFMAs)
//   epilogue: * scale_g[n] (fp8), + bias_g[n], optional exact GeLU, round
//
// Rows of group g occupy [offsets[g], offsets[g] + counts[g]) and every
// group starts at a multiple of the row tile, so a BM x BN tile never
// straddles two experts; its expert is found by a binary search over the
// offsets, on the device, without a host round trip.  Tiles past the last
// group, and rows past a group's count, do no loads or stores.
//
// gfx950 mapping: 16x16x32 bf16 MFMAs, tiles staged in LDS by the
// global_load_lds DMA path (no VGPR staging) in a STAGES-deep ring, XOR
// swizzled in 16-byte chunks so the fragment reads are bank-conflict free.
// The MFMA is issued as (weights x activations) so each lane ends up with
// four consecutive output channels of one row (one 8-byte store).
#include "common.h"

namespace sfl {

enum Epi { EPI_GELU = 0, EPI_BIAS = 1, EPI_F32 = 2 };

struct GemmArgs {
  const void* A;
  int64_t lda;  // elements
  const void* B;
  int64_t ldb;       // elements
  int64_t b_gstride;  // elements between consecutive groups
  const float* scale;  // [G][N] fp8 channel scales or null
  const void* bias;    // [G][N] (bf16 for EPI_GELU/EPI_BIAS, f32 for EPI_F32) or null
  void* C;
  int64_t ldc;
  const int32_t* offsets;  // [G+1] padded row offsets; null: one group of M rows
  const int32_t* counts;   // [G]
  int G;
  int64_t M;
  int N, K;
  int m_tiles, n_tiles;
};

// Find the tile's group and number of valid rows; false if it has none.
template <int BM>
__device__ __forceinline__ bool tile_group(const GemmArgs& a, int64_t row0, int& g, int& rows) {
  if (a.offsets == nullptr) {
    if (row0 >= a.M) return false;
    g = 0;
    rows = (int)(a.M - row0 < BM ? a.M - row0 : BM);
    return true;
  }
  if (row0 >= a.offsets[a.G]) return false;
  int lo = 0, hi = a.G;  // offsets[lo] <= row0 < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.offsets[mid] <= row0) lo = mid; else hi = mid;
  }
  g = lo;
  const int64_t left = a.counts[g] - (row0 - a.offsets[g]);
  rows = (int)(left < BM ? left : BM);
  return rows > 0;
}

// Two OCP e4m3 codes (low 16 bits of `w` if !HI) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool BFP8, int EPI>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_bf16_kernel(const GemmArgs a) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BSZ = BFP8 ? 1 : 2;
  constexpr int CA = BK * 2 / 16;    // 16-byte chunks per A row
  constexpr int CB = BK * BSZ / 16;  // 16-byte chunks per B row
  constexpr int A_BYTES = BM * BK * 2;
  constexpr int B_BYTES = BN * BK * BSZ;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_LOADS = BM * CA / NT;
  constexpr int B_LOADS = BN * CB / NT;
  constexpr int LOADS = A_LOADS + B_LOADS;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 16, FN = WTN / 16;
  constexpr int KS = BK / 32;  // MFMA k-steps per stage
  static_assert(BM * CA % NT == 0 && BN * CB % NT == 0, "tile loads must divide evenly");
  static_assert(FM >= 1 && FN >= 1 && WTM % 16 == 0 && WTN % 16 == 0, "wave tile");
  static_assert((CA & (CA - 1)) == 0 && (CB & (CB - 1)) == 0, "chunk counts are powers of two");
  static_assert((STAGES - 2) * LOADS < 64, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const int bid = blockIdx.x;
  const int mt = bid % a.m_tiles;
  const int nt = bid / a.m_tiles;
  const int64_t row0 = (int64_t)mt * BM;
  int g, rows;
  if (!tile_group<BM>(a, row0, g, rows)) return;
  const int n0 = nt * BN;

  // per-thread source addresses of the 16-byte chunks this thread copies
  const char* a_src[A_LOADS];
  const char* b_src[B_LOADS];
  {
    const char* A = (const char*)a.A;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const int q = i * NT + tid;
      const int r = q / CA, s = q % CA;
      const int c = s ^ (r & (CA - 1));
      const int rr = r < rows ? r : rows - 1;
      a_src[i] = A + ((row0 + rr) * a.lda) * 2 + c * 16;
    }
    const char* B = (const char*)a.B + (int64_t)g * a.b_gstride * BSZ;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
      const int q = i * NT + tid;
      const int r = q / CB, s = q % CB;
      const int c = s ^ (r & (CB - 1));
      b_src[i] = B + ((int64_t)(n0 + r) * a.ldb) * BSZ + c * 16;
    }
  }
  auto issue = [&](int kt, int slot) {
    char* sa = smem + slot * STAGE_BYTES;
    char* sb = sa + A_BYTES;
    const int64_t ka = (int64_t)kt * BK * 2, kb = (int64_t)kt * BK * BSZ;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) load_lds_16(a_src[i] + ka, sa + (i * NT + wave * 64) * 16);
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) load_lds_16(b_src[i] + kb, sb + (i * NT + wave * 64) * 16);
  };

  f32x4_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int KT = a.K / BK;
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < KT) issue(s, s);

  const int lr = lane & 15, lk = lane >> 4;
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + STAGES - 2 < KT) wait_vmcnt<(STAGES - 2) * LOADS>();
    else wait_vmcnt<0>();
    barrier_lds();
    if (kt + STAGES - 1 < KT) issue(kt + STAGES - 1, (kt + STAGES - 1) % STAGES);

    const char* sa = smem + (kt % STAGES) * STAGE_BYTES;
    const char* sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = wm * WTM + i * 16 + lr;
        const int c = ks * 4 + lk;
        af[i] = *(const bf16x8_t*)(sa + (r * CA + (c ^ (r & (CA - 1)))) * 16);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int r = wn * WTN + j * 16 + lr;
        if constexpr (BFP8) {
          const int c = ks * 2 + (lk >> 1);
          const uint2 q = *(const uint2*)(sb + (r * CB + (c ^ (r & (CB - 1)))) * 16 + (lk & 1) * 8);
          const bf16x2_t p0 = fp8x2_to_bf16x2<false>(q.x), p1 = fp8x2_to_bf16x2<true>(q.x);
          const bf16x2_t p2 = fp8x2_to_bf16x2<false>(q.y), p3 = fp8x2_to_bf16x2<true>(q.y);
          bfr[j] = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        } else {
          const int c = ks * 4 + lk;
          bfr[j] = *(const bf16x8_t*)(sb + (r * CB + (c ^ (r & (CB - 1)))) * 16);
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: lane holds out[m = lr][n = 4*lk .. 4*lk+3] of each 16x16 tile
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * WTN + j * 16 + lk * 4;
    float sc[4] = {1.f, 1.f, 1.f, 1.f}, bi[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (BFP8) {
      const float4 s4 = *(const float4*)(a.scale + (int64_t)g * a.N + n);
      sc[0] = s4.x; sc[1] = s4.y; sc[2] = s4.z; sc[3] = s4.w;
    }
    if (a.bias != nullptr) {
      if constexpr (EPI == EPI_F32) {
        const float4 b4 = *(const float4*)((const float*)a.bias + (int64_t)g * a.N + n);
        bi[0] = b4.x; bi[1] = b4.y; bi[2] = b4.z; bi[3] = b4.w;
      } else {
        const uint2 b2 = *(const uint2*)((const uint16_t*)a.bias + (int64_t)g * a.N + n);
        bi[0] = bf16_bits_to_f32(b2.x & 0xffff); bi[1] = bf16_bits_to_f32(b2.x >> 16);
        bi[2] = bf16_bits_to_f32(b2.y & 0xffff); bi[3] = bf16_bits_to_f32(b2.y >> 16);
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int m = wm * WTM + i * 16 + lr;
      if (m < rows) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float t = BFP8 ? acc[i][j][q] * sc[q] : acc[i][j][q];
          t += bi[q];
          if constexpr (EPI == EPI_GELU) t = gelu_erf(t);
          v[q] = t;
        }
        const int64_t off = (row0 + m) * a.ldc + n;
        if constexpr (EPI == EPI_F32) {
          *(float4*)((float*)a.C + off) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
          *(uint2*)((uint16_t*)a.C + off) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
  }
}

// fp32 activations and weights: vector-ALU tiles (64 x 64 outputs, 4 x 4 per
// thread), exact fp32 fused multiply-adds.
template <int EPI>
__global__ void __launch_bounds__(256) grouped_gemm_f32_kernel(const GemmArgs a) {
  constexpr int BM = 64, BN = 64, BK = 16;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  const int tid = threadIdx.x;
  const int mt = blockIdx.x % a.m_tiles, nt = blockIdx.x / a.m_tiles;
  const int64_t row0 = (int64_t)mt * BM;
  int g, rows;
  if (!tile_group<BM>(a, row0, g, rows)) return;
  const int n0 = nt * BN;
  const float* A = (const float*)a.A;
  const float* B = (const float*)a.B + (int64_t)g * a.b_gstride;
  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  const int lr = tid / 4, lq = (tid % 4) * 4;  // loader: row, k quad
  const int ar = lr < rows ? lr : rows - 1;
  for (int k0 = 0; k0 < a.K; k0 += BK) {
    const float4 av = *(const float4*)(A + (row0 + ar) * a.lda + k0 + lq);
    const float4 bv = *(const float4*)(B + (int64_t)(n0 + lr) * a.ldb + k0 + lq);
    As[lq + 0][lr] = av.x; As[lq + 1][lr] = av.y; As[lq + 2][lr] = av.z; As[lq + 3][lr] = av.w;
    Bs[lq + 0][lr] = bv.x; Bs[lq + 1][lr] = bv.y; Bs[lq + 2][lr] = bv.z; Bs[lq + 3][lr] = bv.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float x[4], w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) { x[i] = As[kk][ty * 4 + i]; w[i] = Bs[kk][tx * 4 + i]; }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(x[i], w[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int n = n0 + tx * 4;
  float bi[4] = {0.f, 0.f, 0.f, 0.f};
  if (a.bias != nullptr) {
    const float4 b4 = *(const float4*)((const float*)a.bias + (int64_t)g * a.N + n);
    bi[0] = b4.x; bi[1] = b4.y; bi[2] = b4.z; bi[3] = b4.w;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = ty * 4 + i;
    if (m < rows) {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float t = acc[i][j] + bi[j];
        if constexpr (EPI == EPI_GELU) t = gelu_erf(t);
        v[j] = t;
      }
      *(float4*)((float*)a.C + (row0 + m) * a.ldc + n) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
}

// ------------------------------------------------------------------ configs
// Tile shapes per regime; the padding granule of the expert groups equals BM.
struct TileCfg { int bm; };
// 0: prefill (many rows per expert)  1: mid  2: decode (few rows per expert)
int gemm_regime(const Problem& p) {
  if (p.act == DT_F32) return 3;
  const int64_t per_expert = p.S * p.K / p.E;
  if (per_expert >= 256) return 0;
  if (per_expert >= 48) return 1;
  return 2;
}
int gemm_tile_m(const Problem& p) {
  switch (gemm_regime(p)) {
    case 0: return 128;
    case 1: return 64;
    case 2: return 16;
    default: return 64;
  }
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool BFP8, int EPI>
static hipError_t run_bf16(GemmArgs a, int64_t rows_cap, hipStream_t st) {
  a.m_tiles = (int)ceil_div(rows_cap, BM);
  a.n_tiles = a.N / BN;
  const int64_t blocks = (int64_t)a.m_tiles * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  grouped_gemm_bf16_kernel<BM, BN, BK, WM, WN, STAGES, BFP8, EPI>
      <<<(unsigned)blocks, 64 * WM * WN, 0, st>>>(a);
  return hipGetLastError();
}

template <int EPI>
static hipError_t run_f32(GemmArgs a, int64_t rows_cap, hipStream_t st) {
  a.m_tiles = (int)ceil_div(rows_cap, 64);
  a.n_tiles = a.N / 64;
  const int64_t blocks = (int64_t)a.m_tiles * a.n_tiles;
  if (blocks == 0) return hipSuccess;
  grouped_gemm_f32_kernel<EPI><<<(unsigned)blocks, 256, 0, st>>>(a);
  return hipGetLastError();
}

// Tile shapes per regime.  BN must divide N and BK must divide K; both are
// multiples of 64, so the 128-wide variants fall back to 64 when needed.
template <bool BFP8, int EPI>
static hipError_t run_regime(int regime, const GemmArgs& a, int64_t rows_cap, hipStream_t st) {
  const bool n128 = a.N % 128 == 0, k128 = a.K % 128 == 0;
  switch (regime) {
    case 0:
      if (n128) return run_bf16<128, 128, 64, 2, 2, 3, BFP8, EPI>(a, rows_cap, st);
      return run_bf16<128, 64, 64, 2, 2, 3, BFP8, EPI>(a, rows_cap, st);
    case 1:
      if (n128) return run_bf16<64, 128, 64, 1, 4, 4, BFP8, EPI>(a, rows_cap, st);
      return run_bf16<64, 64, 64, 1, 4, 4, BFP8, EPI>(a, rows_cap, st);
    default:
      if (k128) return run_bf16<16, 64, 128, 1, 4, 5, BFP8, EPI>(a, rows_cap, st);
      return run_bf16<16, 64, 64, 1, 2, 8, BFP8, EPI>(a, rows_cap, st);  // 128 threads: A tile is 128 chunks
  }
}

static GemmArgs expert_args(const Problem& p, const int32_t* counts, const int32_t* offsets) {
  GemmArgs g{};
  g.offsets = offsets; g.counts = counts; g.G = p.E;
  return g;
}

template <int EPI>
static hipError_t run_expert_gemm(const Problem& p, const GemmArgs& g, int64_t rows_cap, hipStream_t st) {
  if (p.act == DT_F32) return run_f32<EPI>(g, rows_cap, st);
  if (p.w == DT_FP8) return run_regime<true, EPI>(gemm_regime(p), g, rows_cap, st);
  return run_regime<false, EPI>(gemm_regime(p), g, rows_cap, st);
}

// h = GeLU(x_perm W1^T + b1) over the expert groups.
hipError_t launch_expert_up(const Problem& p, int64_t rows_cap, const void* x_perm,
                            const int32_t* counts, const int32_t* offsets, const void* W1,
                            const void* b1, const float* s1, void* h, hipStream_t st) {
  GemmArgs g = expert_args(p, counts, offsets);
  g.A = x_perm; g.lda = p.d;
  g.B = W1; g.ldb = p.d; g.b_gstride = (int64_t)p.d_ff * p.d;
  g.scale = s1; g.bias = b1;
  g.C = h; g.ldc = p.d_ff;
  g.N = p.d_ff; g.K = p.d;
  return run_expert_gemm<EPI_GELU>(p, g, rows_cap, st);
}

// y_perm = h W2^T + b2 over the expert groups.
hipError_t launch_expert_down(const Problem& p, int64_t rows_cap, const void* h,
                              const int32_t* counts, const int32_t* offsets, const void* W2,
                              const void* b2, const float* s2, void* y_perm, hipStream_t st) {
  GemmArgs g = expert_args(p, counts, offsets);
  g.A = h; g.lda = p.d_ff;
  g.B = W2; g.ldb = p.d_ff; g.b_gstride = (int64_t)p.d * p.d_ff;
  g.scale = s2; g.bias = b2;
  g.C = y_perm; g.ldc = p.d;
  g.N = p.d; g.K = p.d_ff;
  return run_expert_gemm<EPI_BIAS>(p, g, rows_cap, st);
}

// Router scores x W_r^T (+ router_bias) as one bf16 MFMA GEMM (E % 64 == 0).
hipError_t launch_router_gemm(const Problem& p, const void* x, const void* Wr, const float* rbias,
                              float* logits, hipStream_t st) {
  GemmArgs a{};
  a.A = x; a.lda = p.d;
  a.B = Wr; a.ldb = p.d; a.b_gstride = 0;
  a.bias = rbias;
  a.C = logits; a.ldc = p.E;
  a.M = p.S; a.G = 1;
  a.N = p.E; a.K = p.d;
  return run_bf16<128, 64, 64, 4, 1, 3, false, EPI_F32>(a, p.S, st);
}

}  // namespace sfl
