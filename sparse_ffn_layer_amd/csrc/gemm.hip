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
//   A    : activations, bf16, row-major [rows][K]; or (W8A8) OCP e4m3
//          codes with one float32 scale per row
//   B_g  : weights of group g in linear-layer layout [N][K] (bf16 or OCP
//          e4m3 fp8; with bf16 activations the codes are converted exactly
//          to bf16 on the way into the MFMAs, with e4m3 activations both
//          operands go to the fp8 MFMAs)
//   epilogue: * scale_g[n] (fp8) * row scale (W8A8), + bias_g[n], optional
//          exact GeLU, round
//
// Rows of group g occupy [offsets[g], offsets[g] + counts[g]) and every
// group starts at a multiple of the row tile, so a BM x BN tile never
// straddles two experts; its expert is found by a binary search over the
// offsets, on the device, without a host round trip.  Rows past a group's
// count do no loads or stores.
//
// Scheduling: the kernel is persistent.  The number of row tiles in use is
// read on the device (offsets[G] / BM), so the host never waits for the
// routing.  The tile space is cut into 8 contiguous slices, one per XCD
// (workgroups are dealt to the 8 XCDs round-robin, so workgroup b runs on
// XCD b % 8), and inside a slice tiles are ordered in bands of GM row tiles
// with the row tile varying fastest: the workgroups running at the same time
// on one XCD share a few weight and activation panels through that XCD's
// L2.  The mapping is a bijection for any grid of at least 8 workgroups;
// only the locality depends on the dispatch order.
//
// gfx950 mapping: 16x16x32 bf16 MFMAs, tiles staged in LDS by the
// global_load_lds DMA path (no VGPR staging) in a STAGES-deep ring, XOR
// swizzled in 16-byte chunks so the fragment reads are bank-conflict free.
// The MFMA is issued as (weights x activations) so each lane ends up with
// four consecutive output channels of one row (one 8-byte store).  Fragments
// of the next 32-wide k step are read from LDS while the MFMAs of the
// current one run.
#include "common.h"

#include <type_traits>

namespace sfl {

enum Epi { EPI_GELU = 0, EPI_BIAS = 1, EPI_F32 = 2 };

struct GemmArgs {
  const void* A;
  int64_t lda;  // elements
  const void* B;
  int64_t ldb;       // elements
  int64_t b_gstride;  // elements between consecutive groups
  const float* scale;  // [G][N] fp8 channel scales or null
  const float* a_scale;  // [rows] scale of each e4m3 activation row (W8A8) or null
  const void* bias;    // [G][N] (bf16 for EPI_GELU/EPI_BIAS, f32 for EPI_F32) or null
  void* C;
  int64_t ldc;
  const int32_t* offsets;  // [G+1] padded row offsets; null: one group of M rows
  const int32_t* counts;   // [G]
  int G;
  int64_t M;
  int N, K;
  int m_tiles, n_tiles;  // m_tiles: upper bound (capacity / BM)
  float* partial;        // split-K partial sums of the tail tiles ([grid][BM*BN] floats) or null
  int grid;              // workgroups of the persistent launch
  // Rows read in place (nullable): row r of the product reads row a_rows[r]
  // of A, an array of a_src_rows rows (the token rows of x, for instance,
  // in place of a gathered copy); its byte size must stay below 2^32 - lda.
  // Row scales of e4m3 activations are then those of the source rows.
  const int32_t* a_rows;
  int64_t a_src_rows;
};

// Tail split of one XCD's tile range.  The tile space is cut into 8 slices
// (one per XCD) and each slice is processed in rounds by its nx workgroups.
// When the last round is partial (tail tiles < nx), each tail tile's k range
// is split into `split` slices run by otherwise idle workgroups: the item
// (tile tau, slice sig) goes to workgroup xj = tau * split + sig of that XCD,
// which writes float32 partial sums; a second kernel adds them up in slice
// order (deterministic) and runs the epilogue.
struct TailPlan {
  int64_t t_lo, t_hi, full_end;  // [t_lo, full_end): whole rounds; full_end + tau: tail tiles
  int tail, split;               // split == 0: no split
};
__device__ __forceinline__ TailPlan tail_plan(int64_t T, int xcd, int nx, bool enable) {
  TailPlan t;
  t.t_lo = T * xcd / 8;
  t.t_hi = T * (xcd + 1) / 8;
  const int64_t tx = t.t_hi - t.t_lo;
  t.full_end = t.t_lo + tx / nx * nx;
  t.tail = (int)(tx % nx);
  t.split = (enable && t.tail > 0) ? nx / t.tail : 0;
  if (t.split < 2) t.split = 0;
  if (t.split > 8) t.split = 8;
  return t;
}

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

// Row tiles in use: read on the device from the padded offsets.
template <int BM>
__device__ __forceinline__ int rows_tiles_used(const GemmArgs& a) {
  if (a.offsets == nullptr) return (int)((a.M + BM - 1) / BM);
  const int used = (a.offsets[a.G] + BM - 1) / BM;
  return used < a.m_tiles ? used : a.m_tiles;
}

// Two OCP e4m3 codes (low 16 bits of `w` if !HI) -> two bf16, exact.
template <bool HI>
__device__ __forceinline__ bf16x2_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w, 1.0f, HI);
}

// LDS slot of 16-byte chunk c in row r of a tile with NC chunks per row is
// c ^ swz<NC>(r).  The XOR term (r ^ (r >> 2)) keeps the 16-byte fragment
// reads of both MFMA shapes free of bank conflicts for 64-, 128- and
// 256-byte rows (measured on gfx950: 64 banks, ~240 B/clk per CU).
template <int NC>
__device__ __forceinline__ int swz(int r) {
  return NC > 1 ? ((r ^ (r >> 2)) & (NC - 1)) : 0;
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

// Tile L of the persistent order: bands of row tiles, the row tile varying
// fastest inside a band.  False if the tile has no valid rows.
//  GM > 0: bands of GM consecutive row tiles of the whole tile space.
//  GM < 0: expert-aligned bands: each group's row tiles split into bands of
//  at most -GM row tiles starting at its first row tile, so the row tiles of
//  one expert run side by side on one XCD and read each slice of a weight
//  panel from HBM once, the others finding it in that XCD's L2.  The bands
//  sit in the tile space exactly where their row tiles are (row tile r
//  covers positions [r n_tiles, (r + 1) n_tiles)), so tile L finds its band
//  with the same binary search over the offsets that finds its expert.
//  FR > 0 (GM < 0 only): balanced row tiles: the expert's rows, in blocks of
//  FR (the MFMA fragment), are dealt evenly over its row tiles instead of
//  filling them in order (129 rows on 128-row tiles: 96 + 33 rather than
//  128 + 1), so the tiles sharing a weight panel do the same work and stay
//  in step, and the panel read by one is still in L2 for the other.
template <int BM, int BN, int GM, int FR = 0>
__device__ __forceinline__ bool tile_coords(const GemmArgs& a, int m_used, int64_t L, int64_t& row0, int& n0,
                                            int& g, int& rows) {
  static_assert(FR == 0 || (GM < 0 && BM % FR == 0), "balanced row tiles: expert-aligned bands, whole fragments");
  if constexpr (GM < 0) {
    if (a.offsets == nullptr) return tile_coords<BM, BN, 1>(a, m_used, L, row0, n0, g, rows);
    constexpr int GB = -GM;
    const int r = (int)(L / a.n_tiles);
    const int64_t rr = (int64_t)r * BM;
    if (rr >= a.offsets[a.G]) return false;
    int lo = 0, hi = a.G;  // offsets[lo] <= rr < offsets[lo + 1]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.offsets[mid] <= rr) lo = mid; else hi = mid;
    }
    const int first = a.offsets[lo] / BM, rt = (a.offsets[lo + 1] - a.offsets[lo]) / BM;
    const int bi = (r - first) / GB;
    const int bfirst = first + bi * GB;
    const int gm = rt - bi * GB < GB ? rt - bi * GB : GB;
    const int64_t local = L - (int64_t)bfirst * a.n_tiles;
    const int t = bfirst - first + (int)(local % gm);  // row tile of the expert
    n0 = (int)(local / gm) * BN;
    g = lo;
    if constexpr (FR > 0) {
      // rt = ceil(count / BM) tiles share ceil(count / FR) >= rt fragments:
      // tile t gets q or q + 1 (<= BM / FR) of them, at least one row each
      const int frags = (a.counts[g] + FR - 1) / FR;
      const int q = frags / rt, rem = frags % rt;
      const int f0 = t * q + (t < rem ? t : rem), nf = q + (t < rem ? 1 : 0);
      row0 = (int64_t)a.offsets[g] + (int64_t)f0 * FR;
      const int left = a.counts[g] - f0 * FR;
      rows = left < nf * FR ? left : nf * FR;
      return rows > 0;
    }
    row0 = (int64_t)(first + t) * BM;
    const int64_t left = a.counts[g] - (row0 - a.offsets[g]);
    rows = (int)(left < BM ? left : BM);
    return rows > 0;
  }
  const int64_t band = (int64_t)GM * a.n_tiles;
  const int64_t bnd = L / band;
  const int first_m = (int)(bnd * GM);
  const int gm = m_used - first_m < GM ? m_used - first_m : GM;
  const int rem = (int)(L - bnd * band);
  const int mt = first_m + rem % gm;
  const int nt = rem / gm;
  row0 = (int64_t)mt * BM;
  n0 = nt * BN;
  return tile_group<BM>(a, row0, g, rows);
}

// Epilogue of one tile: lane holds out[m][n .. n+3] for m = lane % MF and,
// per group q4 of four accumulators, n = (MF == 16 ? 4 * lk : 8 * q4 + 4 * lk);
// scale (fp8), bias, optional exact GeLU, round, store the valid rows.
// Accumulator element k.  AREAD: the accumulators live in AGPRs and are read
// one element at a time with v_accvgpr_read where they are used; otherwise
// the register allocator may copy all of them to VGPRs at once.
template <bool AREAD, typename acc_t>
__device__ __forceinline__ float acc_get(const acc_t& v, int k) {
  if constexpr (AREAD) {
    float f;
    asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(f) : "a"(v[k]));
    return f;
  } else {
    return v[k];
  }
}

template <int BN, int WM, int WN, bool BFP8, int EPI, int MF, int FM, int FN, int NACC, bool AREAD = false,
          bool A8 = false, typename acc_t>
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& a, const acc_t (&acc)[FM][FN], int g, int rows,
                                              int64_t row0, int n0, int wm, int wn, int lr, int lk) {
  constexpr int WTN = BN / WN;
  const int WTM = FM * MF;
  // the lane's output addresses are computed here, not hoisted before the
  // main loop (where they would stay live through it)
  asm volatile("" : "+v"(lr), "+v"(lk));
#pragma unroll
  for (int j = 0; j < FN; ++j) {
#pragma unroll
    for (int q4 = 0; q4 < NACC / 4; ++q4) {
      // one group of output channels at a time: keeps the scheduler from
      // lifting every accumulator into VGPRs at once
      __builtin_amdgcn_sched_barrier(0);
      const int n = n0 + wn * WTN + j * MF + q4 * 8 + lk * 4;
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
        if (wm * WTM + i * MF >= rows) continue;  // uniform: fragment wholly past the rows
        const int m = wm * WTM + i * MF + lr;
        if (m < rows) {
          const float rs = A8 ? a.a_scale[a.a_rows != nullptr ? (int64_t)a.a_rows[row0 + m] : row0 + m] : 1.f;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x = acc_get<AREAD>(acc[i][j], q4 * 4 + q);
            float t = BFP8 ? x * sc[q] : x;
            if constexpr (A8) t *= rs;
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
}

// Tile shapes of the general kernel that can read rows in place.
constexpr bool in_place_tiles(int BM, int BN) { return !(BM == 256 && BN == 256); }

// MF selects the MFMA: 16 (v_mfma_f32_16x16x32_bf16) or 32
// (v_mfma_f32_32x32x16_bf16).  Operand lanes: row (lane % MF) of the
// fragment, 8 consecutive k values starting at 8 * (lane / MF).  Result
// lanes (weights as the first operand): activation row m = lane % MF, four
// consecutive output channels n per group of four accumulator registers.
// A8 (e4m3 activations, requires BFP8): the fp8 MFMAs
// v_mfma_f32_{16x16x128,32x32x64}_f8f6f4 (issued through the block-scaled
// form with unit scales); each lane supplies 32 codes of its row for both
// operands, taken from the same k positions, so the products pair up
// whatever order the hardware reads the 32 bytes in.
// INP: the rows are read in place (a.a_rows, the up product of the layer);
// a separate instance, so that the other launches keep their registers.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool BFP8, int EPI, int GM, int MF, bool A8 = false,
          bool INP = false>
__global__ void __launch_bounds__(64 * WM * WN)
grouped_gemm_bf16_kernel(const GemmArgs a) {
  static_assert(!A8 || BFP8, "e4m3 activations go with e4m3 weights");
  constexpr int NT = 64 * WM * WN;
  constexpr int BSZ = BFP8 ? 1 : 2;
  constexpr int ASZ = A8 ? 1 : 2;
  constexpr bool PAIR = BFP8 && !A8;  // fp8 weights widened to bf16: k-steps in pairs
  constexpr int CA = BK * ASZ / 16;  // 16-byte chunks per A row
  constexpr int CB = BK * BSZ / 16;  // 16-byte chunks per B row
  constexpr int A_BYTES = BM * BK * ASZ;
  constexpr int B_BYTES = BN * BK * BSZ;
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
  constexpr int A_LOADS = BM * CA / NT;
  constexpr int B_LOADS = BN * CB / NT;
  constexpr int LOADS = A_LOADS + B_LOADS;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int KSTEP = A8 ? (MF == 16 ? 128 : 64) : (MF == 16 ? 32 : 16);  // k per MFMA
  constexpr int KS = BK / KSTEP;             // MFMA k-steps per stage
  // The loads that refill a freed LDS slot are issued a share per k-step
  // over the next stage (all but its last k-step) instead of in one burst
  // after the barrier: with 4+ k-steps per stage (W8A16 DeepSeek shape:
  // expert_up 1.386 -> 1.355-1.360 ms, layer 2.96-2.99 -> 2.89 ms/step).
  // Not with 2 (W8A8: all loads in one k-step, 1 % slower) nor for the
  // 16-row decode tiles (expert_up 0.128 -> 0.132 ms).
  constexpr bool SPREAD = KS >= 4 && BM > 16;
  constexpr int NACC = MF == 16 ? 4 : 16;
  constexpr int RD = A8 ? 2 : 1;             // 16-byte LDS reads per fragment
  typedef typename std::conditional<MF == 16, f32x4_t, f32x16_t>::type acc_t;
  typedef typename std::conditional<A8, i32x8_t, bf16x8_t>::type frag_t;
  // Rows read in place (a.a_rows) keep per-tile A offsets in the work items;
  // the 256 x 256 tiles have no registers left for them.
  constexpr bool IN_PLACE = INP;
  static_assert(!INP || in_place_tiles(BM, BN), "tile shape without rows read in place");
  // Large wave tiles keep their accumulators in AGPRs (MFMAs issued as
  // inline asm with AGPR operands), leaving the VGPRs to the fragments.
  constexpr bool AGPR_ACC = MF == 32 && !BFP8 && FM * FN * NACC > 128;
  static_assert(KS >= 1 && BK % KSTEP == 0, "whole MFMA k-steps per stage");
  // Expert-aligned bands deal each expert's rows evenly over its row tiles
  // (in whole MFMA fragments).
  constexpr int BAL_FR = GM < 0 ? MF : 0;
  // Decode tiles (a few rows per expert) read every weight exactly once:
  // those loads are marked non-temporal.
  constexpr int B_AUX = BM <= 16 ? 2 : 0;
  static_assert(RD * (FM + FN) < 16, "lgkmcnt range");
  static_assert(MF == 16 || MF == 32, "MFMA shape");
  static_assert(BM * CA % NT == 0 && BN * CB % NT == 0, "tile loads must divide evenly");
  static_assert(FM >= 1 && FN >= 1 && WTM % MF == 0 && WTN % MF == 0, "wave tile");
  static_assert((CA & (CA - 1)) == 0 && (CB & (CB - 1)) == 0, "chunk counts are powers of two");
  static_assert((STAGES - 1) * LOADS < 64, "vmcnt range");
  static_assert(STAGES >= 2, "at least two stages");
  static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS size");
  static_assert(!BFP8 || CB >= 1, "fp8 rows hold at least one chunk");

  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % MF, lk = lane / MF;

  // ---- persistent, XCD-sliced tile loop
  const int m_used = rows_tiles_used<BM>(a);
  const int64_t T = (int64_t)m_used * a.n_tiles;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, xj = blockIdx.x >> 3;
  const int nx = (nwg - xcd + 7) >> 3;  // workgroups with this blockIdx % 8
  const int KT_ALL = a.K / BK;
  const TailPlan tp = tail_plan(T, xcd, nx, a.partial != nullptr && KT_ALL >= 16);

  // Work items: whole tiles of the full rounds, then (with a split) this
  // workgroup's k-slice of a tail tile.  Global -> LDS copies are buffer
  // loads with a scalar resource per tile (its base is the tile's first row
  // / channel) and one 32-bit offset per copied chunk; the k position goes
  // into the scalar offset.  The resources cover exactly the tile's valid
  // rows (num_records in bytes), so chunks of rows past the group's count
  // are dropped by the buffer range check: no memory access, zeros in LDS,
  // and those rows are never stored.  With rows read in place (a.a_rows),
  // the A resource covers the whole source and each chunk's offset comes
  // from its row's source row; rows past the count get the offset
  // num_records, which the range check drops the same way.  Every access
  // stays inside the operands by construction.
  struct Item {
    int64_t row0;
    int n0, g, rows, kt0, kt1;
    float* part;     // split-K slice: raw float32 accumulators go here
    i32x4_t ra, rb;  // buffer resources of the tile's A rows and B rows
    uint32_t aoff[IN_PLACE ? A_LOADS : 1];  // this thread's A chunk offsets in ra (rows read in place)
  };
  // per-thread chunk offsets inside a tile (the same for every tile)
  uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int q = i * NT + tid;
    const int r = q / CA, s = q % CA;
    a_off[i] = (uint32_t)(r * a.lda * ASZ + (s ^ swz<CA>(r)) * 16);
  }
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int q = i * NT + tid;
    const int r = q / CB, s = q % CB;
    b_off[i] = (uint32_t)(r * a.ldb * BSZ + (s ^ swz<CB>(r)) * 16);
  }
  const int64_t loop_end = tp.split ? tp.full_end : tp.t_hi;
  const bool has_slice = tp.split && xj < tp.tail * tp.split;
  // the first valid item at tile index >= L (L is advanced past it)
  auto next_item = [&](int64_t& L, Item& it) -> bool {
    for (;; L += nx) {
      int64_t Lt = L;
      it.kt0 = 0;
      it.kt1 = KT_ALL;
      it.part = nullptr;
      if (L >= loop_end) {
        if (!has_slice || L - nx >= loop_end) return false;  // the slice comes once, after the whole tiles
        const int tau = xj / tp.split, sig = xj % tp.split;
        Lt = tp.full_end + tau;
        it.kt0 = KT_ALL * sig / tp.split;
        it.kt1 = KT_ALL * (sig + 1) / tp.split;
        it.part = a.partial + (size_t)blockIdx.x * (BM * BN);
      }
      if (!tile_coords<BM, BN, GM, BAL_FR>(a, m_used, Lt, it.row0, it.n0, it.g, it.rows)) continue;
      auto uni = [](i32x4_t v) {
        return i32x4_t{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                       __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w)};
      };
      if constexpr (!IN_PLACE) {
        it.ra = uni(make_rsrc((const char*)a.A + it.row0 * a.lda * ASZ, (uint32_t)((int64_t)it.rows * a.lda * ASZ)));
      } else {
        const uint32_t nrec = (uint32_t)(a.a_src_rows * a.lda * ASZ);
        it.ra = uni(make_rsrc(a.A, nrec));
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
          const int q = i * NT + tid;
          const int r = q / CA, s = q % CA;
          it.aoff[i] = r < it.rows ? (uint32_t)((int64_t)a.a_rows[it.row0 + r] * a.lda * ASZ + (s ^ swz<CA>(r)) * 16)
                                   : nrec;
        }
      }
      it.rb = uni(make_rsrc((const char*)a.B + (int64_t)it.g * a.b_gstride * BSZ + (int64_t)it.n0 * a.ldb * BSZ,
                            (uint32_t)((int64_t)BN * a.ldb * BSZ)));
      L += nx;
      return true;
    }
  };
  // copy l of stage kt of item t into LDS slot `slot`: the A chunks first,
  // then the B chunks
  auto issue_one = [&](const Item& t, int kt, int slot, int l) {
    char* sa = smem + slot * STAGE_BYTES;
    char* sb = sa + A_BYTES;
    if (l < A_LOADS)
      buffer_load_lds_16(t.ra, sa + (l * NT + wave * 64) * 16, IN_PLACE ? t.aoff[IN_PLACE ? l : 0] : a_off[l],
                         (uint32_t)((t.kt0 + kt) * BK * ASZ));
    else
      buffer_load_lds_16<B_AUX>(t.rb, sb + ((l - A_LOADS) * NT + wave * 64) * 16, b_off[l - A_LOADS],
                                (uint32_t)((t.kt0 + kt) * BK * BSZ));
  };
  auto issue = [&](const Item& t, int kt, int slot) {
#pragma unroll
    for (int l = 0; l < LOADS; ++l) issue_one(t, kt, slot, l);
  };

  // One tile.  The LDS slots form one ring across the workgroup's tiles:
  // stage kt of this tile lives in slot (base + kt) % STAGES.  pre: stages
  // 0 .. STAGES-2 are already in flight (issued by the previous tile); pf:
  // the last STAGES-1 stages of this tile refill their freed slots with
  // stages 0 .. STAGES-2 of `nit`, so the next tile's loads fly during this
  // tile's last stages and its epilogue instead of after them.  pf requires
  // KT >= STAGES here and >= STAGES-1 k-tiles in `nit`: then exactly
  // STAGES-2 stages are always issued after the one a k-step waits for.
  auto run_tile = [&](const Item& it, int base, bool pre, bool pf, const Item& nit) {
    const int64_t row0 = it.row0;
    const int n0 = it.n0, g = it.g, rows = it.rows;
    float* const part = it.part;

    // Fragment reads go through inline-asm ds_read so that the compiler does
    // not insert its own (conservative) LDS waits: the k-step whose MFMAs
    // run next is always waited for explicitly with lgkmcnt, after the reads
    // of the following k-step have been issued.  Each fragment keeps one LDS
    // address (slot 0, k-step 0); k-step ks XORs its chunk index into the
    // chunk bits (disjoint from the lane's own chunk bits, and the slot and
    // row parts of the address are multiples of the row size), and the slot
    // adds a multiple of the stage size.
    //
    // fp8 weights: a dot product does not depend on the order of k, so k is
    // dealt to the MFMA k-steps in pairs.  For k-steps 2u and 2u+1 a lane of
    // half h (= lk) holds the 16 codes at k = 2 KSTEP u + 16 h + [0, 16): the
    // low 8 for k-step 2u, the high 8 for k-step 2u+1.  One 16-byte read per
    // pair, the same conflict-free pattern as the bf16 reads; the activation
    // fragments use the same k assignment (k-step 2u: chunk 2 KC u + 2 h,
    // k-step 2u+1: the next chunk).
    //
    // e4m3 activations (A8): a k-step is KSTEP bytes of a row, KC 16-byte
    // chunks; the lane of k half / quarter h = lk holds chunks 2h and 2h+1
    // of the k-step, for both operands.
    constexpr int KC = A8 ? KSTEP / 16 : KSTEP / 8;  // 16-byte chunks per k-step
    static_assert(!PAIR || KS % 2 == 0, "fp8 weights pair the k-steps of a stage");
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
    uint32_t a_rd[FM], b_rd[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int r = wm * WTM + i * MF + lr;
      const int c0 = (BFP8 || A8) ? 2 * lk : lk;
      a_rd[i] = lds0 + (uint32_t)(r * CA * 16 + ((c0 ^ swz<CA>(r)) << 4));
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = wn * WTN + j * MF + lr;
      const int c0 = A8 ? 2 * lk : lk;
      b_rd[j] = lds0 + (uint32_t)(A_BYTES + r * CB * 16 + ((c0 ^ swz<CB>(r)) << 4));
    }
    // chunk-index XOR of k-step ks (A) and of the k-step pair u (fp8 B)
    auto a_kx = [](int ks) -> uint32_t {
      return (uint32_t)((PAIR ? (2 * KC * (ks >> 1) + (ks & 1)) : (KC * ks)) << 4);
    };
    // one fragment: a 16-byte read, or (A8) the two chunks 2h, 2h+1
    auto read_frag = [](uint32_t addr, frag_t& f) {
      if constexpr (A8) {
        i32x4_t lo, hi;
        asm volatile("ds_read_b128 %0, %1" : "=v"(lo) : "v"(addr));
        asm volatile("ds_read_b128 %0, %1" : "=v"(hi) : "v"(addr ^ 16u));
        f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        asm volatile("ds_read_b128 %0, %1" : "=v"(f) : "v"(addr));
      }
    };
    auto read_a = [&](int slot, int ks, frag_t (&af)[FM]) {
      const uint32_t so = (uint32_t)(slot * STAGE_BYTES);
#pragma unroll
      for (int i = 0; i < FM; ++i) read_frag((a_rd[i] ^ a_kx(ks)) + so, af[i]);
    };
    // bf16 / A8: the fragments of k-step q; fp8 weights with bf16
    // activations: the codes of k-step pair q
    auto read_b = [&](int slot, int q, frag_t (&bfr)[FN]) {
      const uint32_t so = (uint32_t)(slot * STAGE_BYTES);
#pragma unroll
      for (int j = 0; j < FN; ++j) read_frag((b_rd[j] ^ (uint32_t)((KC * q) << 4)) + so, bfr[j]);
    };

    acc_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < NACC; ++v) acc[i][j][v] = 0.f;
    if constexpr (AGPR_ACC) {
      // the zeroed accumulators are written to AGPRs by VALU moves; give
      // them the wait states an MFMA source-C read needs after such a write
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 4" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }

    // MFMAs of one k-step; for fp8 weights with bf16 activations `hi`
    // selects the half of the pair's codes that belongs to this k-step
    auto mma_sub = [&](const frag_t (&af)[FM], const frag_t (&braw)[FN], bool hi) {
      if constexpr (A8) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (wm * WTM + i * MF >= rows) continue;
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            if constexpr (MF == 16)
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(braw[j], af[i], acc[i][j], 0, 0, 0, 127,
                                                                           0, 127);
            else
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(braw[j], af[i], acc[i][j], 0, 0, 0, 127,
                                                                          0, 127);
          }
        }
      } else {
      bf16x8_t bfr[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (PAIR) {
          const uint4 q4 = __builtin_bit_cast(uint4, braw[j]);
          const uint32_t w0 = hi ? q4.z : q4.x, w1 = hi ? q4.w : q4.y;
          const bf16x2_t p0 = fp8x2_to_bf16x2<false>(w0), p1 = fp8x2_to_bf16x2<true>(w0);
          const bf16x2_t p2 = fp8x2_to_bf16x2<false>(w1), p3 = fp8x2_to_bf16x2<true>(w1);
          bfr[j] = bf16x8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
        } else {
          bfr[j] = braw[j];
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        // row fragments wholly past the group's last row do no MFMAs
        // (uniform per wave: the tile's partly filled SIMDs finish early)
        if (wm * WTM + i * MF >= rows) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (AGPR_ACC)
            asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[i][j]) : "v"(bfr[j]), "v"(af[i]));
          else if constexpr (MF == 16)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        }
      }
      }
    };

    // Pipeline over k-steps (KS per stage) with two fragment buffers: the
    // fragments of the next k-step are read from LDS while the MFMAs of the
    // current one run.  Before the last k-step of stage kt the barrier makes
    // stage kt+1 visible (its first k-step is prefetched across the stage
    // boundary) and proves every wave has finished reading stage kt, whose
    // slot is then refilled with stage kt+STAGES.
    const int KT = it.kt1 - it.kt0;
    auto slot_of = [&](int kt) { return (base + kt) % STAGES; };
    __syncthreads();  // every wave is done with the previous tile's LDS
    if (pre) {
      if (STAGES - 1 < KT) issue(it, STAGES - 1, slot_of(STAGES - 1));
    } else {
#pragma unroll
      for (int s = 0; s < STAGES; ++s)
        if (s < KT) issue(it, s, slot_of(s));
    }
    // stage 0 has landed (anything issued after it counts too: the wait
    // only gets stricter)
    if (KT >= STAGES) wait_vmcnt<(STAGES - 1) * LOADS>();
    else wait_vmcnt<0>();
    barrier_lds();
    // A fragments alternate per k-step; B fragments per k-step (bf16) or per
    // k-step pair (fp8).  Buffer parities of a stage's k-step 0 come in as
    // compile-time tags (stages are unrolled by two).
    frag_t fa[2][FM], fb[2][FN];
    read_a(slot_of(0), 0, fa[0]);
    read_b(slot_of(0), 0, fb[0]);

    auto stage = [&](int kt, auto pa_tag, auto pb_tag) {
      constexpr int pa = decltype(pa_tag)::value, pb = decltype(pb_tag)::value;
      const int slot = slot_of(kt);
      const bool more = kt + 1 < KT;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int acur = (pa + ks) & 1, anxt = (pa + ks + 1) & 1;
        const int bcur = PAIR ? ((pb + (ks >> 1)) & 1) : ((pb + ks) & 1);
        const int bnxt = PAIR ? ((pb + ((ks + 1) >> 1)) & 1) : ((pb + ks + 1) & 1);
        // does the next k-step start a new B fragment set?
        const bool nb = PAIR ? ((ks + 1) % 2 == 0) : true;
        if (ks + 1 < KS) {
          read_a(slot, ks + 1, fa[anxt]);
          if (nb) read_b(slot, PAIR ? (ks + 1) / 2 : ks + 1, fb[bnxt]);
          if (nb) wait_lgkmcnt<RD * (FM + FN)>();  // k-step ks has landed; the next may be in flight
          else wait_lgkmcnt<RD * FM>();
        } else if (more) {
          if (kt + STAGES - 1 < KT || pf) wait_vmcnt<(STAGES - 2) * LOADS>();
          else wait_vmcnt<0>();
          barrier_lds();
          if constexpr (!SPREAD) {
            if (kt + STAGES < KT) issue(it, kt + STAGES, slot);
            else if (pf) issue(nit, kt + STAGES - KT, slot);  // the next tile's stage, into the freed slot
          }
          read_a(slot_of(kt + 1), 0, fa[anxt]);
          read_b(slot_of(kt + 1), 0, fb[bnxt]);
          wait_lgkmcnt<RD * (FM + FN)>();
        } else {
          wait_lgkmcnt<0>();
        }
        __builtin_amdgcn_sched_barrier(0);
        mma_sub(fa[acur], fb[bcur], PAIR && (ks & 1));
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (SPREAD) {
          // the stage that refills the slot of stage kt - 1 (freed by the
          // barrier that ended it), a share per k-step before the last
          if (ks < KS - 1 && kt >= 1) {
            const int tgt = kt - 1 + STAGES;
            const int pslot = slot_of(kt - 1);
#pragma unroll
            for (int l = ks * LOADS / (KS - 1); l < (ks + 1) * LOADS / (KS - 1); ++l) {
              if (tgt < KT) issue_one(it, tgt, pslot, l);
              else if (pf) issue_one(nit, tgt - KT, pslot, l);
            }
          }
        }
      }
    };
    using P0 = std::integral_constant<int, 0>;
    using PA1 = std::integral_constant<int, (KS & 1)>;
    using PB1 = std::integral_constant<int, PAIR ? ((KS / 2) & 1) : (KS & 1)>;
    // every item has at least one k stage; a loop that may run zero times
    // would merge the zeroed accumulators with the loop's results (copies of
    // every accumulator after it, and more registers in use)
    int kt = 0;
    do {
      stage(kt, P0{}, P0{});
      if (kt + 1 < KT) stage(kt + 1, PA1{}, PB1{});
      kt += 2;
    } while (kt < KT);

    if constexpr (AGPR_ACC) {
      // the last MFMAs wrote the accumulators (AGPRs) behind the compiler's
      // back: wait out the MFMA-write -> accvgpr-read hazard before the
      // epilogue copies them
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    }
    if (part != nullptr) {
      // split-K slice: raw accumulators in 16-byte groups, group-major so
      // consecutive threads store consecutive 16 bytes
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < NACC; v += 4) {
            const int q = ((i * FN + j) * NACC + v) / 4;
            *(float4*)(part + ((size_t)q * NT + tid) * 4) =
                make_float4(acc[i][j][v], acc[i][j][v + 1], acc[i][j][v + 2], acc[i][j][v + 3]);
          }
      return;
    }
    gemm_epilogue<BN, WM, WN, BFP8, EPI, MF, FM, FN, NACC, false, A8>(a, acc, g, rows, row0, n0, wm, wn, lr, lk);
  };

  // one call site keeps the tile body inlined once
  int64_t L = tp.t_lo + xj;
  Item cur, nit;
  bool have = next_item(L, cur), pre = false;
  int base = 0;
  while (have) {
    const bool has_next = next_item(L, nit);
    const bool pf = has_next && cur.kt1 - cur.kt0 >= STAGES && nit.kt1 - nit.kt0 >= STAGES - 1;
    run_tile(cur, base, pre, pf, nit);
    base = (base + cur.kt1 - cur.kt0) % STAGES;
    pre = pf;
    cur = nit;
    have = has_next;
  }
}

// sum[q] += slice sig's group q for sig = 0 .. split-1, in slice order:
// slice sig's group q is at p + sig * slice_stride + q * q_stride (floats).
// Two slices are loaded before either is added, so each round trip to
// memory brings two slices.
template <int QB>
__device__ __forceinline__ void fixup_add_slices(float4* sum, const float* p, size_t q_stride, size_t slice_stride,
                                                 int split) {
  int sig = 0;
  for (; sig + 1 < split; sig += 2) {
    float4 t0[QB], t1[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) t0[q] = *(const float4*)(p + sig * slice_stride + q * q_stride);
#pragma unroll
    for (int q = 0; q < QB; ++q) t1[q] = *(const float4*)(p + (sig + 1) * slice_stride + q * q_stride);
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      sum[q].x += t0[q].x; sum[q].y += t0[q].y; sum[q].z += t0[q].z; sum[q].w += t0[q].w;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      sum[q].x += t1[q].x; sum[q].y += t1[q].y; sum[q].z += t1[q].z; sum[q].w += t1[q].w;
    }
  }
  if (sig < split) {
    float4 t0[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) t0[q] = *(const float4*)(p + sig * slice_stride + q * q_stride);
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      sum[q].x += t0[q].x; sum[q].y += t0[q].y; sum[q].z += t0[q].z; sum[q].w += t0[q].w;
    }
  }
}

// Second pass of the tail split: adds the float32 partial sums of each
// split tile in slice order and runs the epilogue.  It recomputes the GEMM's
// tail plan; workgroups without a tail tile return at once.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool BFP8, int EPI, int GM, int MF, bool A8 = false>
__global__ void __launch_bounds__(64)
grouped_gemm_fixup_kernel(const GemmArgs a) {
  // One single-wave workgroup per wave of each tail tile (the reduction is
  // bound by load latency, so spreading a tile over WM WN compute units
  // shortens it): workgroup xcd + 8 (NW tau + w) takes wave w's sums of tail
  // tile tau, exactly what that wave of the GEMM wrote.
  constexpr int NT = 64 * WM * WN, NW = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / MF, FN = WTN / MF;
  constexpr int NACC = MF == 16 ? 4 : 16;
  typedef typename std::conditional<MF == 16, f32x4_t, f32x16_t>::type acc_t;
  const int lane = threadIdx.x;
  const int xcd = blockIdx.x & 7, r = blockIdx.x >> 3, tau = r / NW, wave = r % NW;
  const int tid = wave * 64 + lane;  // the GEMM thread whose sums these are
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane % MF, lk = lane / MF;
  const int m_used = rows_tiles_used<BM>(a);
  const int64_t T = (int64_t)m_used * a.n_tiles;
  const int nwg = a.grid;
  const int nx = (nwg - xcd + 7) >> 3;
  if (a.partial == nullptr || a.K / BK < 16) return;
  const TailPlan tp = tail_plan(T, xcd, nx, true);
  if (tp.split == 0 || tau >= tp.tail) return;
  int64_t row0;
  int n0, g, rows;
  constexpr int BAL_FR = GM < 0 ? MF : 0;  // balanced row tiles, as in the GEMM
  if (!tile_coords<BM, BN, GM, BAL_FR>(a, m_used, tp.full_end + tau, row0, n0, g, rows)) return;
  if (wm * WTM >= rows) return;  // this wave's rows are all past the tile's rows: nothing to store
  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < NACC; ++v) acc[i][j][v] = 0.f;
  // slice sums in slice order, 16-byte loads: a batch of up to 16 groups
  // (64 values) of this thread from two slices at a time (the reduction is
  // bound by load latency; split >= 2 whenever it runs)
  constexpr int NQ = FM * FN * NACC / 4;  // 16-byte groups per thread
  constexpr int QB = NQ < 16 ? NQ : 16;
  static_assert(NQ % QB == 0, "group batches");
  float4 sum[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) sum[q] = make_float4(0.f, 0.f, 0.f, 0.f);
  const float* part0 = a.partial + (size_t)(xcd + 8 * tau * tp.split) * (BM * BN);
#pragma unroll
  for (int q0 = 0; q0 < NQ; q0 += QB)
    fixup_add_slices<QB>(sum + q0, part0 + ((size_t)q0 * NT + tid) * 4, (size_t)NT * 4,
                         (size_t)8 * (BM * BN), tp.split);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < NACC / 4; ++v) {
        const float4 u = sum[(i * FN + j) * (NACC / 4) + v];
        acc[i][j][4 * v] = u.x; acc[i][j][4 * v + 1] = u.y; acc[i][j][4 * v + 2] = u.z; acc[i][j][4 * v + 3] = u.w;
      }
  gemm_epilogue<BN, WM, WN, BFP8, EPI, MF, FM, FN, NACC, false, A8>(a, acc, g, rows, row0, n0, wm, wn, lr, lk);
}

// bf16 prefill tiles of 256 x 256 with eight waves, two per SIMD, each
// owning 128 rows x 64 channels: 8 accumulator blocks of 32 x 32 in AGPRs
// (128 registers), so the two waves of a SIMD fit its register file and one
// issues MFMAs while the other waits on LDS or on the vector-memory queue.
// Every 16-byte fragment read from LDS feeds two (A) or four (B) MFMAs.
//
// The tile's global loads are staged in VGPRs: stage kt + 2 is loaded during
// stage kt and written to LDS during stage kt + 1, into the slot that the
// barrier ending stage kt freed.  Every k-step interleaves its LDS reads, LDS
// writes and global loads with the MFMAs, at most one of each per MFMA; the
// loads of a stage are spread over two k-steps.  The last stage of a tile
// loads the next tile's first stage the same way, so those loads fly during
// the epilogue.  Padding rows of a partly filled tile read zeros; a wave
// skips the MFMAs and A-fragment reads of its 32-row fragments that hold
// only padding, through one copy of the k loop per count of valid fragments
// (4, 2 or 1, chosen once per tile; a copy for 3 does not fit the registers
// beside the others): Mixtral shape expert_up 0.913-0.918 -> 0.892-0.911 ms,
// expert_down 0.852-0.857 -> 0.835-0.846 ms, output unchanged.  Row tiles
// are balanced as in the general kernel, whose split-K fixup reduces the
// tail: the partial sums are laid out as that kernel's with 2 x 4 waves of
// 128 x 64.
//
// Against the 256 x 256 tile on four waves of 128 x 128 (one per SIMD, all
// 512 registers each) that preceded it: Mixtral shape expert_up 0.92-0.93 ->
// 0.89-0.92 ms, expert_down 0.84-0.86 -> 0.84-0.85 ms, layer 1.85-1.87 ->
// 1.82-1.84 ms/step; Zipf shape 1.76 -> 1.72-1.75 ms/step.
//
// Bands of the tile order: expert-aligned, up to 8 row tiles (each band
// re-reads the weights of its expert once; against bands of 8 (up) and 4
// (down) consecutive row tiles of the whole tile space: Mixtral shape 1.96 ->
// 1.94 ms/step, Zipf shape 1.86 -> 1.82 ms/step; bands of 4 or 16 expert row
// tiles measured no better).
constexpr int kW8Band = -8;

// Epilogue of the eight-wave kernel, through LDS: bias (+ GeLU) and bf16
// rounding in the MFMA layout, into a per-wave 128 x 64 tile in LDS (16-byte
// chunk c of row r at slot c ^ (r & 7)), then stored by whole 128-byte row
// segments (8 lanes per row, 8 rows per store instruction) instead of 8-byte
// pieces of 32 rows.  The caller has made every wave finish with the
// k-stages in LDS.
template <int EPI>
__device__ __forceinline__ void w8_epilogue(const GemmArgs& a, const f32x16_t (&acc)[4][2], int g, int rows,
                                            int64_t row0, int n0, int wm, int wn, int lr, int lk, int lane, char* wt) {
  asm volatile("" : "+v"(lr), "+v"(lk));  // addresses computed here, not hoisted into the main loop
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint2 bias[4];  // one block's channels at a time (registers are scarce with two waves per SIMD)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int n = n0 + wn * 64 + j * 32 + q4 * 8 + lk * 4;
      bias[q4] = a.bias != nullptr ? *(const uint2*)((const uint16_t*)a.bias + (int64_t)g * a.N + n) : make_uint2(0, 0);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      __builtin_amdgcn_sched_barrier(0);
      const uint2 b2 = bias[q4];
      const float bi[4] = {bf16_bits_to_f32(b2.x & 0xffff), bf16_bits_to_f32(b2.x >> 16),
                           bf16_bits_to_f32(b2.y & 0xffff), bf16_bits_to_f32(b2.y >> 16)};
      const int cc = j * 4 + q4;  // 16-byte chunk of the wave tile's row (8 per row)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (wm * 128 + i * 32 >= rows) continue;
        const int r = i * 32 + lr;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float t = acc_get<true>(acc[i][j], q4 * 4 + q) + bi[q];
          if constexpr (EPI == EPI_GELU) t = gelu_erf(t);
          v[q] = t;
        }
        *(uint2*)(wt + r * 128 + ((cc ^ (r & 7)) << 4) + lk * 8) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
  wait_lgkmcnt<0>();
  const int c = lane & 7;
#pragma unroll 4
  for (int rr = 0; rr < 128; rr += 8) {
    const int r = rr + (lane >> 3);
    const uint4 val = *(const uint4*)(wt + r * 128 + ((c ^ (r & 7)) << 4));
    const int m = wm * 128 + r;
    if (m < rows) *(uint4*)((uint16_t*)a.C + (row0 + m) * a.ldc + n0 + wn * 64 + c * 8) = val;
  }
}

template <int EPI>
__global__ void __launch_bounds__(512, 1) grouped_gemm_bf16_w8_kernel(const GemmArgs a) {
  constexpr int BM = 256, BN = 256, BK = 64, NT = 512, GM = kW8Band, MF = 32, WN = 4;
  constexpr int CA = BK * 2 / 16;
  constexpr int A_BYTES = BM * BK * 2, STAGE_BYTES = A_BYTES + BN * BK * 2;
  constexpr int A_LOADS = BM * CA / NT, B_LOADS = BN * CA / NT, LOADS = A_LOADS + B_LOADS;
  constexpr int FM = 4, FN = 2, NACC = 16, KS = BK / 16, KC = 2, NMF = FM * FN;
  static_assert(LOADS == 8 && NMF == 8, "the k-step schedule below assumes 8 loads and 8 MFMAs");
  static_assert(2 * STAGE_BYTES >= 8 * 128 * 128, "the epilogue's per-wave tiles fit in the stage buffers");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lk = lane >> 5;

  const int m_used = rows_tiles_used<BM>(a);
  const int64_t T = (int64_t)m_used * a.n_tiles;
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x & 7, xj = blockIdx.x >> 3;
  const int nx = (nwg - xcd + 7) >> 3;
  const int KT_ALL = a.K / BK;
  const TailPlan tp = tail_plan(T, xcd, nx, a.partial != nullptr && KT_ALL >= 16);

  struct Item {
    int64_t row0;
    int n0, g, rows, kt0, kt1;
    float* part;
    i32x4_t ra, rb;
  };
  const int64_t loop_end = tp.split ? tp.full_end : tp.t_hi;
  const bool has_slice = tp.split && xj < tp.tail * tp.split;
  auto next_item = [&](int& k, Item& it) -> bool {
    for (;; ++k) {
      const int64_t L = tp.t_lo + xj + (int64_t)k * nx;
      int64_t Lt = L;
      it.kt0 = 0;
      it.kt1 = KT_ALL;
      it.part = nullptr;
      if (L >= loop_end) {
        if (!has_slice || L - nx >= loop_end) return false;
        const int tau = xj / tp.split, sig = xj % tp.split;
        Lt = tp.full_end + tau;
        it.kt0 = KT_ALL * sig / tp.split;
        it.kt1 = KT_ALL * (sig + 1) / tp.split;
        it.part = a.partial + (size_t)blockIdx.x * (BM * BN);
      }
      if (!tile_coords<BM, BN, GM, MF>(a, m_used, Lt, it.row0, it.n0, it.g, it.rows)) continue;
      auto uni = [](i32x4_t v) {
        return i32x4_t{__builtin_amdgcn_readfirstlane(v.x), __builtin_amdgcn_readfirstlane(v.y),
                       __builtin_amdgcn_readfirstlane(v.z), __builtin_amdgcn_readfirstlane(v.w)};
      };
      it.ra = uni(make_rsrc((const char*)a.A + it.row0 * a.lda * 2, (uint32_t)((int64_t)it.rows * a.lda * 2)));
      it.rb = uni(make_rsrc((const char*)a.B + (int64_t)it.g * a.b_gstride * 2 + (int64_t)it.n0 * a.ldb * 2,
                            (uint32_t)((int64_t)BN * a.ldb * 2)));
      ++k;
      return true;
    }
  };

  // chunk l of this thread: row l * (NT / CA) + tid / CA, chunk tid % CA;
  // the swizzle depends on the row only through bits that l does not touch,
  // so one offset per operand and a uniform row stride cover all loads
  static_assert((NT / CA) % 32 == 0, "row stride keeps the swizzle bits");
  // (A and B rows both hold the K contraction values: lda == ldb, checked
  // by the launcher, so one offset serves both operands)
  const int r0 = tid / CA, s0 = tid % CA;
  const uint32_t g_off0 = (uint32_t)(r0 * a.lda * 2 + (s0 ^ swz<CA>(r0)) * 16);
  const uint32_t g_step = (uint32_t)((NT / CA) * a.lda * 2);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  // fragment i of A / j of B: rows 32 apart, the same swizzle (32, 64 and
  // 128 rows keep bits 0-4 of the row), so one lane address plus uniform
  // offsets: wave row / column base, then 32 * CA * 16 bytes per fragment
  const uint32_t rd0 = lds0 + (uint32_t)(lr * CA * 16 + ((lk ^ swz<CA>(lr)) << 4));
  const uint32_t a_base = (uint32_t)(wm * 128 * CA * 16), b_base = (uint32_t)(A_BYTES + wn * 64 * CA * 16);
  constexpr uint32_t FRAG_STEP = MF * CA * 16;
  i32x4_t R[LOADS];
  auto gload = [&](const Item& it, int kt, int l) {
    const uint32_t ko = (uint32_t)((it.kt0 + kt) * BK * 2);
    R[l] = l < A_LOADS ? buffer_load_16(it.ra, g_off0 + (uint32_t)l * g_step, ko)
                       : buffer_load_16(it.rb, g_off0 + (uint32_t)(l - A_LOADS) * g_step, ko);
  };
  auto swrite = [&](int slot, int l) {
    char* base = smem + slot * STAGE_BYTES + (l < A_LOADS ? 0 : A_BYTES);
    const int ll = l < A_LOADS ? l : l - A_LOADS;
    *(i32x4_t*)(base + (ll * NT + tid) * 16) = R[l];
  };
  auto read_one = [&](int slot, int ks, int q, bf16x8_t (&af)[FM], bf16x8_t (&bf)[FN]) {
    const uint32_t so = (uint32_t)(slot * STAGE_BYTES), kx = (uint32_t)((KC * ks) << 4);
    if (q < FM)
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(af[q]) : "v"((rd0 ^ kx) + so + a_base), "n"(q * FRAG_STEP));
    else
      asm volatile("ds_read_b128 %0, %1 offset:%2"
                   : "=v"(bf[q - FM]) : "v"((rd0 ^ kx) + so + b_base), "n"((q - FM) * FRAG_STEP));
  };

  auto run_tile = [&](const Item& it, bool pre, bool has_next, const Item& nit) {
    f32x16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int v = 0; v < NACC; ++v) acc[i][j][v] = 0.f;
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 4" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    const int KT = it.kt1 - it.kt0;
    __syncthreads();
    if (!pre) {
#pragma unroll
      for (int l = 0; l < LOADS; ++l) gload(it, 0, l);
    }
#pragma unroll
    for (int l = 0; l < LOADS; ++l) swrite(0, l);
    if (KT > 1) {
#pragma unroll
      for (int l = 0; l < LOADS; ++l) gload(it, 1, l);
    }
    barrier_lds();
    bf16x8_t fa[2][FM], fb[2][FN];
    // MFMAs and A-fragment reads only for the wave's first NV 32-row
    // fragments (the rest are padding rows of the tile): one copy of the k
    // loop per NV in {4, 2, 1}, chosen once per tile
    auto main_loop = [&](auto nv_tag) {
      constexpr int NV = decltype(nv_tag)::value;
#pragma unroll
      for (int q = 0; q < FM + FN; ++q)
        if (q >= FM || q < NV) read_one(0, 0, q, fa[0], fb[0]);

      auto stage = [&](int kt, auto w_tag, auto l_tag) {
        constexpr bool W = decltype(w_tag)::value, Lq = decltype(l_tag)::value;
        constexpr bool LAST = !W && !Lq;
        const int s = kt & 1;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int cur = ks & 1, nxt = cur ^ 1;
          wait_lgkmcnt<0>();
          if (ks == KS - 1 && W) barrier_lds();
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int t = 0; t < NMF; ++t) {
            const int i = t / FN, j = t % FN;
            if (i < NV)
              asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                           : "+a"(acc[i][j]) : "v"(fb[cur][j]), "v"(fa[cur][i]));
            __builtin_amdgcn_sched_barrier(0);
            // the next k-step's six fragments, one after each of the first six MFMAs
            if (t < FM + FN && (t >= FM || t < NV)) {
              if (ks + 1 < KS) read_one(s, ks + 1, t, fa[nxt], fb[nxt]);
              else if (W) read_one(s ^ 1, 0, t, fa[nxt], fb[nxt]);
            }
            // writes of the staged stage kt + 1: registers 0-3 in k-step 0,
            // 4-7 in k-step 1; reloaded after their write: 0-3 in k-step 0,
            // one slot after each write, 4-7 in k-step 2 (loads take the
            // longest lead that fits: reloading 4-7 in k-step 1 spills,
            // spreading the reloads two per k-step over all four k-steps
            // cut their lead and cost 11 %; this order, against 0-3 in
            // k-step 1: Mixtral expert_down 0.827-0.829 -> 0.820 ms)
            if (W && ks < 2 && (t & 1) == 0) swrite(s ^ 1, ks * 4 + t / 2);
            int l = -1;
            if (ks == 0 && (t & 1) == 1) l = t / 2;
            if (ks == 2 && (t & 1) == 1) l = 4 + t / 2;
            if (l >= 0) {
              if constexpr (Lq) gload(it, kt + 2, l);
              if constexpr (LAST) {
                if (has_next) gload(nit, 0, l);
              }
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };
      using T1 = std::integral_constant<bool, true>;
      using T0 = std::integral_constant<bool, false>;
      int kt = 0;
      for (; kt + 2 < KT; ++kt) stage(kt, T1{}, T1{});
      if (kt + 1 < KT) {
        stage(kt, T1{}, T0{});
        ++kt;
      }
      stage(kt, T0{}, T0{});
    };
    const int nv = __builtin_amdgcn_readfirstlane((it.rows - wm * 128 + MF - 1) / MF);
    if (nv >= 3) main_loop(std::integral_constant<int, 4>{});
    else if (nv == 2) main_loop(std::integral_constant<int, 2>{});
    else main_loop(std::integral_constant<int, 1>{});

    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (it.part != nullptr) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int v = 0; v < NACC; v += 4) {
            const int q = ((i * FN + j) * NACC + v) / 4;
            *(float4*)(it.part + ((size_t)q * NT + tid) * 4) =
                make_float4(acc_get<true>(acc[i][j], v), acc_get<true>(acc[i][j], v + 1),
                            acc_get<true>(acc[i][j], v + 2), acc_get<true>(acc[i][j], v + 3));
          }
      return;
    }
    __syncthreads();
    {
      const int ln = threadIdx.x & 63;  // recomputed here: not kept live through the main loop
      w8_epilogue<EPI>(a, acc, it.g, it.rows, it.row0, it.n0, wm, wn, ln & 31, ln >> 5, ln, smem + wave * (128 * 128));
    }
  };

  int k = 0;
  Item cur, nit;
  bool have = next_item(k, cur), pre = false;
  while (have) {
    const bool has_next = next_item(k, nit);
    run_tile(cur, pre, has_next, nit);
    pre = has_next;
    cur = nit;
    have = has_next;
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
// 0: prefill (many rows per expert)  1: mid  2: decode (few rows per expert)
int gemm_regime(const Problem& p) {
  if (p.act == DT_F32) return 3;
  const int64_t per_expert = p.S * p.K / p.E;
  if (per_expert >= 256) return 0;
  if (per_expert >= 64) return 1;
  return 2;
}
// Padding granule of the expert groups: the row tile of the regime.
int gemm_tile_m(const Problem& p) {
  switch (gemm_regime(p)) {
    case 0: return 256;
    case 1: return 128;
    case 2: return 16;
    default: return 64;
  }
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Workgroups of a persistent launch the split-K workspace is sized for; a
// larger launch (more CUs than an MI355X) simply runs without the split.
constexpr int kSplitGrid = 512;

// Persistent launch: as many workgroups as fit on the device at once (a
// multiple of 8, at least 8), never more than there are tiles.  With a
// split-K workspace (a.partial) the tail tiles are split and a second
// kernel reduces them.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, bool BFP8, int EPI, int GM, int MF = 16, bool A8 = false>
hipError_t run_bf16(GemmArgs a, int64_t rows_cap, hipStream_t st, size_t partial_bytes = 0) {
  auto kern = grouped_gemm_bf16_kernel<BM, BN, BK, WM, WN, STAGES, BFP8, EPI, GM, MF, A8, false>;
  constexpr int NT = 64 * WM * WN;
  if (a.a_rows != nullptr) {
    // rows read in place: up products on tile shapes that keep the offsets
    // (expert_up_reads_in_place chooses them; anything else is a caller bug)
    if constexpr (EPI == EPI_GELU && in_place_tiles(BM, BN))
      kern = grouped_gemm_bf16_kernel<BM, BN, BK, WM, WN, STAGES, BFP8, EPI, GM, MF, A8, true>;
    else
      return hipErrorInvalidValue;
  }
  a.m_tiles = (int)ceil_div(rows_cap, BM);
  a.n_tiles = a.N / BN;
  const int64_t tiles = (int64_t)a.m_tiles * a.n_tiles;
  if (tiles == 0) return hipSuccess;
  static int occ[2] = {0, 0};  // resident workgroups per CU of each instance (same on every gfx950 device)
  int& oc = occ[a.a_rows != nullptr];
  if (oc == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, NT, 0) != hipSuccess || n < 1) n = 1;
    oc = n;
  }
  int64_t grid = (int64_t)device_cus() * oc;
  if (grid > tiles) grid = tiles;
  grid = grid < 8 ? 8 : grid / 8 * 8;
  a.grid = (int)grid;
  if (a.partial != nullptr && (size_t)grid * BM * BN * sizeof(float) > partial_bytes) a.partial = nullptr;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.partial == nullptr) return e;
  hipLaunchKernelGGL((grouped_gemm_fixup_kernel<BM, BN, BK, WM, WN, STAGES, BFP8, EPI, GM, MF, A8>),
                     dim3((unsigned)grid * (NT / 64)), dim3(64), 0, st, a);
  return hipGetLastError();
}

// The eight-wave 256 x 256 kernel: one workgroup per CU (128 KB of LDS), the
// general kernel's split-K fixup for its tail.  lda == ldb: the two operands
// share their load offsets (both rows hold the K contraction values).
template <int EPI>
hipError_t run_bf16_w8(GemmArgs a, int64_t rows_cap, hipStream_t st, size_t partial_bytes) {
  a.m_tiles = (int)ceil_div(rows_cap, 256);
  a.n_tiles = a.N / 256;
  const int64_t tiles = (int64_t)a.m_tiles * a.n_tiles;
  if (tiles == 0) return hipSuccess;
  int64_t grid = (int64_t)device_cus();
  if (grid > tiles) grid = tiles;
  grid = grid < 8 ? 8 : grid / 8 * 8;
  a.grid = (int)grid;
  if (a.partial != nullptr && (size_t)grid * 256 * 256 * sizeof(float) > partial_bytes) a.partial = nullptr;
  if (a.a_rows != nullptr || a.lda != a.ldb) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_gemm_bf16_w8_kernel<EPI>, dim3((unsigned)grid), dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.partial == nullptr) return e;
  hipLaunchKernelGGL((grouped_gemm_fixup_kernel<256, 256, 64, 2, 4, 2, false, EPI, kW8Band, 32, false>),
                     dim3((unsigned)grid * 8), dim3(64), 0, st, a);
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
// multiples of 64, so the wider variants fall back when needed.
// Whether the up product of problem p (N = d_ff, K = d) runs on a kernel
// that reads rows in place (a_rows): the choices of run_regime and
// run_regime_a8 below, minus the eight-wave kernel and the 256 x 256 tiles of
// the general one (their launchers refuse a_rows), and the fp32 kernel.
bool expert_up_reads_in_place(const Problem& p) {
  if (p.act != DT_BF16) return false;
  if (p.act_quant || gemm_regime(p) != 0) return true;
  return p.d_ff % 256 != 0;  // prefill: 256 x 256 tiles (eight-wave for bf16 weights) unless N % 256 != 0
}

template <bool BFP8, int EPI>
static hipError_t run_regime(int regime, const GemmArgs& a, int64_t rows_cap, hipStream_t st, size_t pb) {
  const bool n256 = a.N % 256 == 0, n128 = a.N % 128 == 0, k128 = a.K % 128 == 0;
  switch (regime) {
    case 0:
      if (!BFP8 && n256 && a.K % 64 == 0) return run_bf16_w8<EPI>(a, rows_cap, st, pb);
      if (n256) return run_bf16<256, 256, 64, 4, 2, 2, BFP8, EPI, -4, 32>(a, rows_cap, st, pb);
      if (n128) return run_bf16<256, 128, 64, 4, 2, 3, BFP8, EPI, -4, 32>(a, rows_cap, st, pb);
      return run_bf16<256, 64, 64, 4, 1, 3, BFP8, EPI, -4, 32>(a, rows_cap, st, pb);
    case 1:
      // expert-aligned bands of up to 4 row tiles: the row tiles of an expert
      // share each weight panel through L2 (fp8-weight DeepSeek shape, W8A8:
      // 2.53 -> 2.39 ms/step against bands of 2 consecutive row tiles)
      if constexpr (BFP8) {
        // fp8 weights with bf16 rows: 512-wide tiles read each activation
        // row half as often (the larger share of these products' L1 -> L2
        // requests), at the price of k stages of 64 (W8A16 DeepSeek shape:
        // expert_up 1.42-1.46 -> 1.42 ms, expert_down 1.44 -> 1.40 ms);
        // else k stages of 128, so each stage reads whole 128-byte lines of
        // every weight row (3.47 -> 3.31 ms/step against stages of 64)
        if (a.N % 512 == 0) return run_bf16<128, 512, 64, 2, 4, 3, true, EPI, -4, 32>(a, rows_cap, st, pb);
        if (n256 && k128) return run_bf16<128, 256, 128, 2, 4, 2, true, EPI, -4, 32>(a, rows_cap, st, pb);
      }
      if (n256) return run_bf16<128, 256, 64, 2, 4, 3, BFP8, EPI, -4, 32>(a, rows_cap, st, pb);
      if (n128) return run_bf16<128, 128, 64, 2, 4, 3, BFP8, EPI, -4, 32>(a, rows_cap, st, pb);
      return run_bf16<128, 64, 64, 2, 2, 3, BFP8, EPI, -4, 32>(a, rows_cap, st, pb);
    default:
      if (k128) return run_bf16<16, 64, 128, 1, 4, 3, BFP8, EPI, 1>(a, rows_cap, st, pb);
      return run_bf16<16, 64, 64, 1, 2, 8, BFP8, EPI, 1>(a, rows_cap, st, pb);  // 128 threads: A tile is 128 chunks
  }
}

// e4m3 activations and weights (W8A8); K % 128 == 0.  Row tiles of 128 for
// every regime with 64+ rows per expert, 16-row tiles for decode.
template <int EPI>
static hipError_t run_regime_a8(int regime, const GemmArgs& a, int64_t rows_cap, hipStream_t st, size_t pb) {
  const bool n256 = a.N % 256 == 0, n128 = a.N % 128 == 0, k256 = a.K % 256 == 0;
  if (regime <= 1) {
    if (n256) return run_bf16<128, 256, 128, 2, 4, 3, true, EPI, -4, 32, true>(a, rows_cap, st, pb);
    if (n128) return run_bf16<128, 128, 128, 2, 4, 3, true, EPI, -4, 32, true>(a, rows_cap, st, pb);
    return run_bf16<128, 64, 128, 2, 2, 3, true, EPI, -4, 32, true>(a, rows_cap, st, pb);
  }
  if (k256) return run_bf16<16, 64, 256, 1, 4, 5, true, EPI, 1, 16, true>(a, rows_cap, st, pb);
  return run_bf16<16, 64, 128, 1, 2, 8, true, EPI, 1, 16, true>(a, rows_cap, st, pb);
}

// Bytes of split-K workspace the expert GEMMs of problem p can use (one
// float32 tile per workgroup of a persistent launch of up to kSplitGrid).
// The decode regime (a few rows per expert) streams weights with small
// tiles in whole rounds; it gets no split (and no second launch).
size_t expert_split_bytes(const Problem& p) {
  if (p.act == DT_F32) return 0;
  switch (gemm_regime(p)) {
    case 0: return (size_t)kSplitGrid * 256 * 256 * sizeof(float);
    case 1: return (size_t)kSplitGrid * 128 * 256 * sizeof(float);  // also 256 workgroups of 128 x 512
    default: return 0;
  }
}

static GemmArgs expert_args(const Problem& p, const int32_t* counts, const int32_t* offsets) {
  GemmArgs g{};
  g.offsets = offsets; g.counts = counts; g.G = p.E;
  return g;
}

template <int EPI>
static hipError_t run_expert_gemm(const Problem& p, const GemmArgs& g, int64_t rows_cap, hipStream_t st,
                                  size_t partial_bytes) {
  if (p.act == DT_F32) return run_f32<EPI>(g, rows_cap, st);
  if (g.a_scale != nullptr) return run_regime_a8<EPI>(gemm_regime(p), g, rows_cap, st, partial_bytes);
  if (p.w == DT_FP8) return run_regime<true, EPI>(gemm_regime(p), g, rows_cap, st, partial_bytes);
  return run_regime<false, EPI>(gemm_regime(p), g, rows_cap, st, partial_bytes);
}

// h = GeLU(x_perm W1^T + b1) over the expert groups.
// a_scale: row scales of e4m3 activations (W8A8), or null for bf16 rows.
// row_tok (nullable): read the rows in place, row r of the groups from row
// row_tok[r] of x_perm (then the token rows of x, S of them, or their e4m3
// codes with a_scale per token) instead of a gathered copy.
hipError_t launch_expert_up(const Problem& p, int64_t rows_cap, const void* x_perm,
                            const int32_t* counts, const int32_t* offsets, const void* W1,
                            const void* b1, const float* s1, void* h, float* partial,
                            size_t partial_bytes, hipStream_t st, const float* a_scale,
                            const int32_t* row_tok) {
  GemmArgs g = expert_args(p, counts, offsets);
  g.a_scale = a_scale;
  g.a_rows = row_tok;
  g.a_src_rows = p.S;
  g.partial = partial;
  g.A = x_perm; g.lda = p.d;
  g.B = W1; g.ldb = p.d; g.b_gstride = (int64_t)p.d_ff * p.d;
  g.scale = s1; g.bias = b1;
  g.C = h; g.ldc = p.d_ff;
  g.N = p.d_ff; g.K = p.d;
  return run_expert_gemm<EPI_GELU>(p, g, rows_cap, st, partial_bytes);
}

// y_perm = h W2^T + b2 over the expert groups.
hipError_t launch_expert_down(const Problem& p, int64_t rows_cap, const void* h,
                              const int32_t* counts, const int32_t* offsets, const void* W2,
                              const void* b2, const float* s2, void* y_perm, float* partial,
                              size_t partial_bytes, hipStream_t st, const float* a_scale) {
  GemmArgs g = expert_args(p, counts, offsets);
  g.a_scale = a_scale;
  g.partial = partial;
  g.A = h; g.lda = p.d_ff;
  g.B = W2; g.ldb = p.d_ff; g.b_gstride = (int64_t)p.d * p.d_ff;
  g.scale = s2; g.bias = b2;
  g.C = y_perm; g.ldc = p.d;
  g.N = p.d; g.K = p.d_ff;
  return run_expert_gemm<EPI_BIAS>(p, g, rows_cap, st, partial_bytes);
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
  // the largest row tile that still gives every compute unit a tile
  const int64_t nt = p.E / 64, cus = device_cus();
  if (ceil_div(p.S, 128) * nt >= cus) return run_bf16<128, 64, 64, 4, 1, 3, false, EPI_F32, 8>(a, p.S, st);
  if (ceil_div(p.S, 64) * nt >= cus) return run_bf16<64, 64, 64, 2, 2, 3, false, EPI_F32, 8>(a, p.S, st);
  return run_bf16<32, 64, 64, 2, 2, 3, false, EPI_F32, 8>(a, p.S, st);
}

}  // namespace sfl
