// C ABI of the MoE layer: argument validation, workspace layout and launch
// order.  Everything here runs on the host; validation happens before any HIP
// call, so invalid arguments are reported without touching a device.
#include "../../include/moe.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <initializer_list>

#include "common.h"
#include "layer.h"

namespace sfl {
// kernels (router.hip, capacity.hip, permute.hip, quant.hip, gemm.hip, combine.hip)
hipError_t launch_router_fused(const Problem&, const void*, const void*, const float*,
                               const float*, float*, int32_t*, float*, hipStream_t);
hipError_t launch_route_logits(const Problem&, const float*, const float*, float*, int32_t*,
                               float*, hipStream_t);
hipError_t launch_router_gemm(const Problem&, const void*, const void*, const float*, float*,
                              hipStream_t);
hipError_t launch_permute(const Problem&, int, const int32_t*, const void*, int32_t*, int32_t*,
                          int32_t*, int32_t*, void*, int32_t*, hipStream_t, int32_t*);
size_t permute_scratch_ints(int64_t pairs, int E);
hipError_t launch_expert_up(const Problem&, int64_t, const void*, const int32_t*, const int32_t*,
                            const void*, const void*, const float*, void*, float*, size_t,
                            hipStream_t, const float*, const int32_t*);
hipError_t launch_expert_down(const Problem&, int64_t, const void*, const int32_t*,
                              const int32_t*, const void*, const void*, const float*, void*,
                              float*, size_t, hipStream_t, const float*);
hipError_t launch_quantize_rows(const uint16_t*, int64_t, int, int64_t, int, bool, const int32_t*,
                                uint8_t*, int64_t, float*, hipStream_t);
size_t expert_split_bytes(const Problem& p);
hipError_t launch_combine(const Problem&, const void*, const int32_t*, const float*, void*,
                          hipStream_t);
hipError_t launch_load_stats(const Problem&, const int32_t*, const float*, const int32_t*, float,
                             float*, hipStream_t);
hipError_t launch_capacity(const Problem&, int, const float*, const float*, int32_t*, float*,
                           int32_t*, int32_t*, hipStream_t);
size_t capacity_scratch_ints(int64_t pairs, int E);
int gemm_tile_m(const Problem& p);
bool expert_up_reads_in_place(const Problem& p);
}  // namespace sfl

using namespace sfl;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxTokens = int64_t(1) << 24;  // S < 2^24
constexpr int64_t kMaxPairs = int64_t(1) << 26;   // S * K < 2^26
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

// Validate the problem statement itself (no pointers).
int32_t check_problem(const moe_problem* mp, Problem* out) {
  if (mp == nullptr) return MOE_ERR_INVALID_ARG;
  const moe_problem& q = *mp;
  if (q.S < 0 || q.d < 1 || q.d_ff < 1 || q.E < 1 || q.K < 1 || q.K > q.E)
    return MOE_ERR_INVALID_ARG;
  if (q.renormalize != 0 && q.renormalize != 1) return MOE_ERR_INVALID_ARG;
  // gate temperature: 0 means 1; otherwise positive and finite (NaN fails too)
  const float tau = q.gate_temperature == 0.f ? 1.f : q.gate_temperature;
  if (!(tau > 0.f) || !(tau < INFINITY)) return MOE_ERR_INVALID_ARG;
  if (q.capacity < 0) return MOE_ERR_INVALID_ARG;
  if (q.act_quant != 0 && q.act_quant != 1) return MOE_ERR_INVALID_ARG;
  if (q.act_dtype < MOE_F32 || q.act_dtype > MOE_FP8_E4M3 || q.w_dtype < MOE_F32 ||
      q.w_dtype > MOE_FP8_E4M3)
    return MOE_ERR_INVALID_ARG;
  if (q.n_groups > 1) {
    if (q.E % q.n_groups != 0) return MOE_ERR_INVALID_ARG;
    const int m = q.E / q.n_groups;
    if ((m & (m - 1)) != 0) return MOE_ERR_INVALID_ARG;
    if (q.topk_groups < 1 || q.topk_groups > q.n_groups) return MOE_ERR_INVALID_ARG;
    if ((int64_t)q.K > (int64_t)q.topk_groups * m) return MOE_ERR_INVALID_ARG;
    if (q.n_groups > 64) return MOE_ERR_UNSUPPORTED;
  }
  const bool combo = (q.act_dtype == MOE_F32 && q.w_dtype == MOE_F32) ||
                     (q.act_dtype == MOE_BF16 && (q.w_dtype == MOE_BF16 || q.w_dtype == MOE_FP8_E4M3));
  if (!combo) return MOE_ERR_UNSUPPORTED;
  if (q.E > 512 || q.K > 64 || q.d % 64 != 0 || q.d_ff % 64 != 0) return MOE_ERR_UNSUPPORTED;
  // every launch stays below 2^32 work-items: the combine takes 256 threads
  // per token, the row gather and the row quantiser 64 per (token, slot) pair
  if (q.S >= kMaxTokens || q.S * q.K >= kMaxPairs) return MOE_ERR_UNSUPPORTED;
  // fp8 activations: bf16 activations and fp8 weights, k a multiple of 128
  if (q.act_quant && (q.act_dtype != MOE_BF16 || q.w_dtype != MOE_FP8_E4M3 || q.d % 128 != 0 ||
                      q.d_ff % 128 != 0))
    return MOE_ERR_UNSUPPORTED;
  if (out != nullptr) {
    out->S = q.S; out->d = q.d; out->d_ff = q.d_ff; out->E = q.E; out->K = q.K;
    out->n_groups = q.n_groups > 1 ? q.n_groups : 1;
    out->topk_groups = q.n_groups > 1 ? q.topk_groups : 1;
    out->renormalize = q.renormalize; out->act = q.act_dtype; out->w = q.w_dtype;
    out->inv_tau = 1.f / tau;
    out->capacity = q.capacity;
    out->act_quant = q.act_quant;
  }
  return MOE_OK;
}

bool uses_router_gemm(const Problem& p) { return p.act == DT_BF16 && p.E >= 64 && p.E % 64 == 0; }

size_t act_size(const Problem& p) { return p.act == DT_F32 ? 4 : 2; }

int64_t rows_capacity(const Problem& p) {
  const int64_t pairs = p.S * p.K;
  const int64_t tm = gemm_tile_m(p);
  return pairs + (pairs < p.E ? pairs : p.E) * (tm - 1);
}

// The layer's up product reads the token rows of x (or, W8A8, their e4m3
// codes) in place through a row -> token map written by the permute, instead
// of a gathered x_perm, when its kernel can (bf16 activations, not the
// eight-wave prefill kernel) and the source fits one 32-bit buffer range.
bool in_place_rows(const Problem& p) {
  const int64_t asz = p.act_quant ? 1 : 2;
  return expert_up_reads_in_place(p) && (p.S + 1) * (int64_t)p.d * asz < (int64_t(1) << 32);
}

size_t route_ws(const Problem& p) { return uses_router_gemm(p) ? align_up((size_t)p.S * p.E * 4) : 0; }
size_t permute_ws(const Problem& p) { return align_up(permute_scratch_ints(p.S * p.K, p.E) * 4); }
size_t capacity_ws(const Problem& p) { return align_up(capacity_scratch_ints(p.S * p.K, p.E) * 4); }

// Layout of the layer workspace: consecutive 256-byte aligned regions.
struct LayerWs {
  float* logits; int32_t* idx; float* gate; int32_t* counts; int32_t* offsets;
  int32_t* perm; int32_t* inv; int32_t* pscratch; int32_t* cscratch; void* x_perm; void* h; void* y_perm;
  int32_t* row_tok;  // rows read in place: the token of every row of the expert groups
  uint8_t* h8; float* xs; float* hs;  // fp8 activations: h codes, row scales of x_perm and h
  float* split; size_t split_bytes;
  size_t bytes;
};
LayerWs layer_layout(const Problem& p, char* base) {
  LayerWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) { char* ptr = base ? base + off : nullptr; off += align_up(bytes); return ptr; };
  const int64_t pairs = p.S * p.K, cap = rows_capacity(p);
  w.logits = (float*)take((size_t)p.S * p.E * 4);
  w.idx = (int32_t*)take((size_t)pairs * 4);
  w.gate = (float*)take((size_t)pairs * 4);
  w.counts = (int32_t*)take((size_t)p.E * 4);
  w.offsets = (int32_t*)take((size_t)(p.E + 1) * 4);
  w.perm = (int32_t*)take((size_t)pairs * 4);
  w.inv = (int32_t*)take((size_t)pairs * 4);
  w.pscratch = (int32_t*)take(permute_scratch_ints(pairs, p.E) * 4);
  w.cscratch = p.capacity > 0 ? (int32_t*)take(capacity_scratch_ints(pairs, p.E) * 4) : nullptr;
  // x_perm holds the gathered rows, or with fp8 activations their e4m3 codes
  // (one row per token when the rows are read in place); it is not needed
  // for bf16 rows read in place
  const bool inplace = in_place_rows(p);
  const int64_t xrows = inplace ? (p.act_quant ? p.S : 0) : cap;
  w.row_tok = inplace ? (int32_t*)take((size_t)cap * 4) : nullptr;
  w.x_perm = take((size_t)xrows * p.d * (p.act_quant ? 1 : act_size(p)));
  w.h = take((size_t)cap * p.d_ff * act_size(p));
  w.y_perm = take((size_t)cap * p.d * act_size(p));
  if (p.act_quant) {
    w.h8 = (uint8_t*)take((size_t)cap * p.d_ff);
    w.xs = (float*)take((size_t)xrows * 4);
    w.hs = (float*)take((size_t)cap * 4);
  }
  w.split_bytes = expert_split_bytes(p);
  w.split = (float*)take(w.split_bytes);
  w.bytes = off;
  return w;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// split: float32 workspace for the split-K tail (nullable; then no split).
// row_tok (nullable): x_perm is x itself, read in place through this map.
int32_t do_expert_ffn(const Problem& p, const void* x_perm, const int32_t* counts,
                      const int32_t* offsets, const void* W1, const void* b1, const void* W2,
                      const void* b2, const float* s1, const float* s2, void* h, void* y_perm,
                      float* split, size_t split_bytes, hipStream_t st, const int32_t* row_tok = nullptr) {
  const bool fp8 = p.w == DT_FP8;
  const int64_t cap = rows_capacity(p);
  int32_t s = hip_status(launch_expert_up(p, cap, x_perm, counts, offsets, W1, b1, fp8 ? s1 : nullptr,
                                          h, split, split_bytes, st, nullptr, row_tok));
  if (s != MOE_OK) return s;
  return hip_status(launch_expert_down(p, cap, h, counts, offsets, W2, b2, fp8 ? s2 : nullptr,
                                       y_perm, split, split_bytes, st, nullptr));
}

// The split-K workspace inside a caller's buffer (aligned start), or null.
float* split_region(void* ws, size_t ws_bytes, size_t* usable) {
  *usable = 0;
  if (ws == nullptr) return nullptr;
  const uintptr_t b = ((uintptr_t)ws + kAlign - 1) / kAlign * kAlign;
  const size_t skip = b - (uintptr_t)ws;
  if (ws_bytes <= skip) return nullptr;
  *usable = ws_bytes - skip;
  return (float*)b;
}

// Common checks of the expert-GEMM entry points.
int32_t check_expert(const moe_problem* mp, Problem* p, std::initializer_list<const void*> req,
                     const float* scale) {
  int32_t s = check_problem(mp, p);
  if (s != MOE_OK) return s;
  if (p->act_quant) return MOE_ERR_UNSUPPORTED;  // fp8 activations: moe_layer_forward only
  if (p->S == 0) return s;
  for (const void* q : req)
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (p->w == DT_FP8 && scale == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(scale)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int32_t do_route(const Problem& p, const void* x, const void* Wr, const float* rb, const float* sb,
                 const float* logits_in, float* logits_out, int32_t* idx, float* gate,
                 float* logits_scratch, hipStream_t st) {
  if (logits_in != nullptr)
    return hip_status(launch_route_logits(p, logits_in, sb, logits_out, idx, gate, st));
  if (uses_router_gemm(p)) {
    float* lg = logits_out != nullptr ? logits_out : logits_scratch;
    hipError_t e = launch_router_gemm(p, x, Wr, rb, lg, st);
    if (e != hipSuccess) return MOE_ERR_HIP;
    return hip_status(launch_route_logits(p, lg, sb, nullptr, idx, gate, st));
  }
  return hip_status(launch_router_fused(p, x, Wr, rb, sb, logits_out, idx, gate, st));
}

}  // namespace

namespace sfl {

int32_t layer_validate(const moe_problem* mp, const LayerArgs& a, size_t* need) {
  *need = 0;
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  if (p.S == 0) return MOE_OK;
  const void* req[] = {a.x, a.W_r, a.W1, a.b1, a.W2, a.b2, a.y};
  for (const void* q : req)
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  const void* opt[] = {a.router_bias, a.select_bias, a.w1_scale, a.w2_scale, a.topk_idx_out,
                       a.topk_gate_out, a.logits_out, a.expert_counts_out};
  for (const void* q : opt)
    if (!aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (p.w == DT_FP8 && (a.w1_scale == nullptr || a.w2_scale == nullptr)) return MOE_ERR_INVALID_ARG;
  *need = layer_layout(p, nullptr).bytes;
  return MOE_OK;
}

int32_t layer_run(const moe_problem* mp, const LayerArgs& a, void* ws, hipStream_t st) {
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  const LayerWs w = layer_layout(p, (char*)ws);
  int32_t* idx = a.topk_idx_out != nullptr ? a.topk_idx_out : w.idx;
  float* gate = a.topk_gate_out != nullptr ? a.topk_gate_out : w.gate;
  int32_t* counts = a.expert_counts_out != nullptr ? a.expert_counts_out : w.counts;
  // the capacity step reads the scores again, so they are kept in that case
  float* lg = (p.capacity > 0 && a.logits_out == nullptr) ? w.logits : a.logits_out;
  s = do_route(p, a.x, a.W_r, a.router_bias, a.select_bias, nullptr, lg, idx, gate, w.logits, st);
  if (s != MOE_OK) return s;
  if (p.capacity > 0) {
    s = hip_status(launch_capacity(p, p.capacity, lg, a.select_bias, idx, gate, nullptr, w.cscratch, st));
    if (s != MOE_OK) return s;
  }
  const bool inplace = in_place_rows(p);
  if (p.act_quant) {
    // W8A8: e4m3 rows and row scales of x -- one per token, read in place by
    // the up product, or gathered per (token, slot) pair; h is quantised per
    // row between the two products
    const int64_t pairs = p.S * p.K, cap = rows_capacity(p);
    uint8_t* x8 = (uint8_t*)w.x_perm;
    s = hip_status(launch_permute(p, gemm_tile_m(p), idx, a.x, counts, w.offsets, w.perm, w.inv, nullptr,
                                  w.pscratch, st, w.row_tok));
    if (s != MOE_OK) return s;
    if (inplace)
      s = hip_status(launch_quantize_rows((const uint16_t*)a.x, p.d, p.d, p.S, 1, false, nullptr, x8, p.d, w.xs, st));
    else
      s = hip_status(launch_quantize_rows((const uint16_t*)a.x, p.d, p.d, pairs, p.K, true, w.inv, x8, p.d, w.xs,
                                          st));
    if (s != MOE_OK) return s;
    s = hip_status(launch_expert_up(p, cap, x8, counts, w.offsets, a.W1, a.b1, a.w1_scale, w.h, w.split,
                                    w.split_bytes, st, w.xs, w.row_tok));
    if (s != MOE_OK) return s;
    s = hip_status(launch_quantize_rows((const uint16_t*)w.h, p.d_ff, p.d_ff, pairs, p.K, false, w.inv, w.h8,
                                        p.d_ff, w.hs, st));
    if (s != MOE_OK) return s;
    s = hip_status(launch_expert_down(p, cap, w.h8, counts, w.offsets, a.W2, a.b2, a.w2_scale, w.y_perm,
                                      w.split, w.split_bytes, st, w.hs));
    if (s != MOE_OK) return s;
    return hip_status(launch_combine(p, w.y_perm, w.inv, gate, a.y, st));
  }
  s = hip_status(launch_permute(p, gemm_tile_m(p), idx, a.x, counts, w.offsets, w.perm, w.inv,
                                inplace ? nullptr : w.x_perm, w.pscratch, st, w.row_tok));
  if (s != MOE_OK) return s;
  s = do_expert_ffn(p, inplace ? a.x : w.x_perm, counts, w.offsets, a.W1, a.b1, a.W2, a.b2, a.w1_scale,
                    a.w2_scale, w.h, w.y_perm, w.split, w.split_bytes, st, w.row_tok);
  if (s != MOE_OK) return s;
  return hip_status(launch_combine(p, w.y_perm, w.inv, gate, a.y, st));
}

}  // namespace sfl

extern "C" {

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported problem";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    case MOE_ERR_TOO_LARGE: return "problem needs more workspace than the no-alloc scratch array holds";
    default: return "unknown status";
  }
}

int32_t moe_tile_m(const moe_problem* mp) {
  Problem p;
  if (check_problem(mp, &p) != MOE_OK) return -1;
  return gemm_tile_m(p);
}

int64_t moe_rows_capacity(const moe_problem* mp) {
  Problem p;
  if (check_problem(mp, &p) != MOE_OK) return -1;
  return rows_capacity(p);
}

size_t moe_workspace_bytes(const moe_problem* mp, int32_t stage) {
  Problem p;
  if (check_problem(mp, &p) != MOE_OK) return 0;
  switch (stage) {
    case MOE_STAGE_ROUTE: return route_ws(p);
    case MOE_STAGE_PERMUTE: return permute_ws(p);
    case MOE_STAGE_EXPERT_FFN: return expert_split_bytes(p) ? expert_split_bytes(p) + kAlign : 0;
    case MOE_STAGE_COMBINE: return 0;
    case MOE_STAGE_LAYER: return layer_layout(p, nullptr).bytes;
    case MOE_STAGE_CAPACITY: return capacity_ws(p);
    default: return 0;
  }
}

int32_t moe_route(const moe_problem* mp, const void* x, const void* W_r, const float* router_bias,
                  const float* select_bias, const float* logits_in, float* logits_out,
                  int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes, void* stream) {
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  if (p.S == 0) return MOE_OK;
  if (topk_idx == nullptr || topk_gate == nullptr) return MOE_ERR_INVALID_ARG;
  if (logits_in == nullptr && (x == nullptr || W_r == nullptr)) return MOE_ERR_INVALID_ARG;
  const void* ptrs[] = {x, W_r, router_bias, select_bias, logits_in, logits_out, topk_idx, topk_gate};
  for (const void* q : ptrs)
    if (!aligned16(q)) return MOE_ERR_INVALID_ARG;
  const size_t need = (logits_in == nullptr && logits_out == nullptr) ? route_ws(p) : 0;
  if (need > 0 && (ws == nullptr || ws_bytes < need)) return MOE_ERR_WORKSPACE;
  return do_route(p, x, W_r, router_bias, select_bias, logits_in, logits_out, topk_idx, topk_gate,
                  (float*)ws, (hipStream_t)stream);
}

int32_t moe_permute(const moe_problem* mp, const int32_t* topk_idx, const void* x,
                    int32_t* expert_counts, int32_t* expert_offsets, int32_t* perm,
                    int32_t* inv_perm, void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  if (p.act_quant) return MOE_ERR_UNSUPPORTED;  // fp8 activations: moe_layer_forward only
  if (p.S == 0) return MOE_OK;
  const void* ptrs[] = {topk_idx, x, expert_counts, expert_offsets, perm, inv_perm, x_perm};
  for (const void* q : ptrs)
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < permute_ws(p)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_permute(p, gemm_tile_m(p), topk_idx, x, expert_counts, expert_offsets,
                                   perm, inv_perm, x_perm, (int32_t*)ws, (hipStream_t)stream, nullptr));
}

int32_t moe_expert_ffn(const moe_problem* mp, const void* x_perm, const int32_t* expert_counts,
                       const int32_t* expert_offsets, const void* W1, const void* b1,
                       const void* W2, const void* b2, const float* w1_scale,
                       const float* w2_scale, void* h, void* y_perm, void* ws, size_t ws_bytes,
                       void* stream) {
  Problem p;
  int32_t s = check_expert(mp, &p, {x_perm, expert_counts, expert_offsets, W1, b1, W2, b2, h, y_perm},
                           w1_scale);
  if (s != MOE_OK || p.S == 0) return s;
  if (p.w == DT_FP8 && w2_scale == nullptr) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w2_scale)) return MOE_ERR_INVALID_ARG;
  size_t usable = 0;
  float* split = split_region(ws, ws_bytes, &usable);
  return do_expert_ffn(p, x_perm, expert_counts, expert_offsets, W1, b1, W2, b2, w1_scale, w2_scale,
                       h, y_perm, split, usable, (hipStream_t)stream);
}

int32_t moe_expert_up(const moe_problem* mp, const void* x_perm, const int32_t* expert_counts,
                      const int32_t* expert_offsets, const void* W1, const void* b1,
                      const float* w1_scale, void* h, void* ws, size_t ws_bytes, void* stream) {
  Problem p;
  int32_t s = check_expert(mp, &p, {x_perm, expert_counts, expert_offsets, W1, b1, h}, w1_scale);
  if (s != MOE_OK || p.S == 0) return s;
  size_t usable = 0;
  float* split = split_region(ws, ws_bytes, &usable);
  return hip_status(launch_expert_up(p, rows_capacity(p), x_perm, expert_counts, expert_offsets, W1,
                                     b1, p.w == DT_FP8 ? w1_scale : nullptr, h, split, usable,
                                     (hipStream_t)stream, nullptr, nullptr));
}

int32_t moe_expert_down(const moe_problem* mp, const void* h, const int32_t* expert_counts,
                        const int32_t* expert_offsets, const void* W2, const void* b2,
                        const float* w2_scale, void* y_perm, void* ws, size_t ws_bytes, void* stream) {
  Problem p;
  int32_t s = check_expert(mp, &p, {h, expert_counts, expert_offsets, W2, b2, y_perm}, w2_scale);
  if (s != MOE_OK || p.S == 0) return s;
  size_t usable = 0;
  float* split = split_region(ws, ws_bytes, &usable);
  return hip_status(launch_expert_down(p, rows_capacity(p), h, expert_counts, expert_offsets, W2, b2,
                                       p.w == DT_FP8 ? w2_scale : nullptr, y_perm, split, usable,
                                       (hipStream_t)stream, nullptr));
}

// W8A8 stage entry points: e4m3 rows with per-row scales in, bf16 out.
int32_t check_expert_a8(const moe_problem* mp, Problem* p, std::initializer_list<const void*> req) {
  int32_t s = check_problem(mp, p);
  if (s != MOE_OK) return s;
  if (!p->act_quant) return MOE_ERR_INVALID_ARG;
  if (p->S == 0) return MOE_OK;
  for (const void* q : req)
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

int32_t moe_expert_up_a8(const moe_problem* mp, const uint8_t* x8, const float* x_scale,
                         const int32_t* expert_counts, const int32_t* expert_offsets, const void* W1,
                         const void* b1, const float* w1_scale, void* h, void* ws, size_t ws_bytes,
                         void* stream) {
  Problem p;
  int32_t s = check_expert_a8(mp, &p, {x8, x_scale, expert_counts, expert_offsets, W1, b1, w1_scale, h});
  if (s != MOE_OK || p.S == 0) return s;
  size_t usable = 0;
  float* split = split_region(ws, ws_bytes, &usable);
  return hip_status(launch_expert_up(p, rows_capacity(p), x8, expert_counts, expert_offsets, W1, b1, w1_scale,
                                     h, split, usable, (hipStream_t)stream, x_scale, nullptr));
}

int32_t moe_expert_down_a8(const moe_problem* mp, const uint8_t* h8, const float* h_scale,
                           const int32_t* expert_counts, const int32_t* expert_offsets, const void* W2,
                           const void* b2, const float* w2_scale, void* y_perm, void* ws, size_t ws_bytes,
                           void* stream) {
  Problem p;
  int32_t s = check_expert_a8(mp, &p, {h8, h_scale, expert_counts, expert_offsets, W2, b2, w2_scale, y_perm});
  if (s != MOE_OK || p.S == 0) return s;
  size_t usable = 0;
  float* split = split_region(ws, ws_bytes, &usable);
  return hip_status(launch_expert_down(p, rows_capacity(p), h8, expert_counts, expert_offsets, W2, b2,
                                       w2_scale, y_perm, split, usable, (hipStream_t)stream, h_scale));
}

int32_t moe_combine(const moe_problem* mp, const void* y_perm, const int32_t* inv_perm,
                    const float* topk_gate, void* y, void* stream) {
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  if (p.S == 0) return MOE_OK;
  const void* ptrs[] = {y_perm, inv_perm, topk_gate, y};
  for (const void* q : ptrs)
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_combine(p, y_perm, inv_perm, topk_gate, y, (hipStream_t)stream));
}

int32_t moe_load_stats(const moe_problem* mp, const int32_t* expert_counts, const float* logits,
                       const int32_t* dropped, float alpha, float* stats, void* stream) {
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  if (!std::isfinite(alpha)) return MOE_ERR_INVALID_ARG;
  if (p.S == 0) return MOE_OK;
  if (expert_counts == nullptr || stats == nullptr) return MOE_ERR_INVALID_ARG;
  for (const void* q : {(const void*)expert_counts, (const void*)logits, (const void*)dropped, (const void*)stats})
    if (q != nullptr && !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_load_stats(p, expert_counts, logits, dropped, alpha, stats, (hipStream_t)stream));
}

int32_t moe_quantize_rows(const void* src, int64_t rows, int32_t n, uint8_t* codes, float* scales,
                          void* stream) {
  if (rows < 0 || n < 8 || n % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (rows >= kMaxPairs) return MOE_ERR_UNSUPPORTED;  // 64 threads per row, < 2^32 in all
  for (const void* q : {(const void*)src, (const void*)codes, (const void*)scales})
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  return hip_status(launch_quantize_rows((const uint16_t*)src, n, n, rows, 1, false, nullptr, codes, n, scales,
                                         (hipStream_t)stream));
}

int32_t moe_apply_capacity(const moe_problem* mp, const float* logits, const float* select_bias,
                           int32_t* topk_idx, float* topk_gate, int32_t* dropped, void* ws,
                           size_t ws_bytes, void* stream) {
  Problem p;
  int32_t s = check_problem(mp, &p);
  if (s != MOE_OK) return s;
  if (p.S == 0) return MOE_OK;
  for (const void* q : {(const void*)logits, (const void*)topk_idx, (const void*)topk_gate})
    if (q == nullptr || !aligned16(q)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(select_bias) || !aligned16(dropped)) return MOE_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < capacity_ws(p)) return MOE_ERR_WORKSPACE;
  return hip_status(launch_capacity(p, p.capacity, logits, select_bias, topk_idx, topk_gate, dropped,
                                    (int32_t*)ws, (hipStream_t)stream));
}

int32_t moe_layer_forward(const moe_problem* mp, const void* x, const void* W_r,
                          const float* router_bias, const float* select_bias, const void* W1,
                          const void* b1, const void* W2, const void* b2, const float* w1_scale,
                          const float* w2_scale, void* y, int32_t* topk_idx_out,
                          float* topk_gate_out, float* logits_out, int32_t* expert_counts_out,
                          void* ws, size_t ws_bytes, void* stream) {
  const LayerArgs a{x, W_r, router_bias, select_bias, W1, b1, W2, b2, w1_scale, w2_scale, y,
                    topk_idx_out, topk_gate_out, logits_out, expert_counts_out};
  size_t need = 0;
  int32_t s = layer_validate(mp, a, &need);
  if (s != MOE_OK || need == 0) return s;
  if (ws == nullptr || ws_bytes < need) return MOE_ERR_WORKSPACE;
  return layer_run(mp, a, ws, (hipStream_t)stream);
}

}  // extern "C"
