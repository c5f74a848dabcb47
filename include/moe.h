/*
 * moe.h -- C ABI of the single-GPU Mixture-of-Experts feed-forward layer
 * (forward pass) for AMD Instinct MI355X (gfx950).
 *
 * The layer (chapter "大模型推理技术 | 第11章 MoE模型推理", jsqmd.com,
 * sections 11.1.1-11.1.2):
 *     y = sum over the K chosen experts i of  gate_i(x) * E_i(x)
 *     E_i(x) = GeLU(x W1_i + b1_i) W2_i + b2_i        (exact erf GeLU)
 *     gates  = softmax of the router scores x W_r (+ router_bias) over the
 *              K experts with the largest scores (renormalize = 1), or their
 *              full-softmax probabilities (renormalize = 0).
 * Optional DeepSeek-V3 style selection ("MoE 推理工程深层实战", ybb.press,
 * section 2.3): a per-expert select_bias is added to the scores for selection
 * only, and with n_groups > 1 the experts are split into n_groups groups of
 * consecutive experts; only the topk_groups groups with the largest summed
 * biased score stay eligible.
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers, row-major, 16-byte aligned, owned by
 *    the caller.  The library keeps no pointer after a call returns.
 *  - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL = the
 *    default stream).  No call synchronises the host, reads device data back,
 *    or allocates memory.  Buffers must stay alive until the stream reaches
 *    the work.
 *  - Arguments are validated on the host before anything is launched.  On a
 *    validation failure the call returns a negative moe_status and writes
 *    nothing.  A failed kernel launch returns MOE_ERR_HIP.  Nothing aborts and
 *    no C++ exception crosses the ABI.
 *  - S == 0 is a no-op that returns MOE_OK (pointers may then be NULL).
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *    Different calls may run concurrently only on distinct buffers.
 *  - Inputs are finite numbers; NaN or Inf inputs are outside the contract.
 *
 * Data types (moe_problem.act_dtype / w_dtype)
 *  - act: x, W_r, b1, b2, x_perm, h, y_perm, y          MOE_F32 or MOE_BF16
 *  - w:   W1, W2    MOE_F32 (with act F32), MOE_BF16 or MOE_FP8_E4M3 (with
 *         act BF16).  fp8 is OCP E4M3FN; the weight value is
 *         decode(code) * scale[e][output channel].
 *  - logits, gates, router_bias, select_bias, scales: float32
 *  - indices, counts, offsets, perm, inv_perm: int32
 *
 * Weight layout: each matrix is stored like a linear layer's weight,
 * [out_features, in_features], so the contraction index is contiguous:
 *     W_r [E][d]    W1 [E][d_ff][d]    W2 [E][d][d_ff]
 *     b1 [E][d_ff]  b2 [E][d]          w1_scale [E][d_ff]   w2_scale [E][d]
 * (x W1 in the pages' notation is x times the transpose of the stored W1.)
 */
#ifndef SPARSE_FFN_LAYER_MOE_H
#define SPARSE_FFN_LAYER_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* bad shape, NULL or misaligned pointer, bad flag */
  MOE_ERR_UNSUPPORTED = -2, /* valid problem outside what the kernels handle */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than required */
  MOE_ERR_HIP = -4,         /* a HIP launch failed */
  MOE_ERR_TOO_LARGE = -5    /* moe_layer_forward_noalloc: the problem needs more
                               than MOE_NOALLOC_SCRATCH_BYTES of workspace */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_FP8_E4M3 = 2 } moe_dtype;

/* Which entry point a workspace is sized for. */
typedef enum {
  MOE_STAGE_ROUTE = 0,
  MOE_STAGE_PERMUTE = 1,
  MOE_STAGE_EXPERT_FFN = 2,
  MOE_STAGE_COMBINE = 3,
  MOE_STAGE_LAYER = 4,
  MOE_STAGE_CAPACITY = 5
} moe_stage;

/* The problem statement: S tokens of width d (S = batch x sequence, chapter
 * 11 section 11.3.1), E experts with hidden width d_ff, K experts per token.
 *  - n_groups <= 1: no group limit.  Otherwise E % n_groups == 0, E/n_groups
 *    a power of two, n_groups <= 64, 1 <= topk_groups <= n_groups and
 *    K <= topk_groups * E / n_groups.
 *  - renormalize: 1 = gates are the softmax over the K chosen scores (sum to
 *    1); 0 = gates are the chosen experts' full-softmax probabilities.
 *  - gate_temperature: the gates are computed from score / tau (chapter 11
 *    section 11.3.3, soft routing: a higher tau spreads the weights more
 *    evenly; with K = E this is the soft-routing layer).  Selection does not
 *    depend on it.  0 means 1 (so a zero-initialised problem keeps plain
 *    gates); tau must otherwise be positive and finite, else
 *    MOE_ERR_INVALID_ARG.
 *  - capacity: the most (token, slot) pairs one expert takes in
 *    moe_layer_forward and moe_apply_capacity (chapter 11 section 11.3.3,
 *    expert dropping); 0 = no limit; negative: MOE_ERR_INVALID_ARG.
 *  - act_quant: 1 = fp8 activations (W8A8) in moe_layer_forward: the rows
 *    entering each expert product (x, then h) are quantised per row as
 *    moe_quantize_rows does, and both products run on fp8 MFMAs; the result
 *    is dequantised by row scale times weight channel scale.  Needs
 *    act_dtype BF16, w_dtype FP8_E4M3, d and d_ff multiples of 128 (else
 *    MOE_ERR_UNSUPPORTED).  moe_permute, moe_expert_ffn, moe_expert_up and
 *    moe_expert_down (bf16 activations) return MOE_ERR_UNSUPPORTED when it
 *    is set; moe_expert_up_a8 and moe_expert_down_a8 require it.
 *    0 = activations in act_dtype; other values: MOE_ERR_INVALID_ARG.
 *  - Limits: 1 <= E <= 512, 1 <= K <= min(E, 64), d and d_ff multiples of 64,
 *    S < 2^24 and S * K < 2^26 (every kernel launch stays below 2^32
 *    work-items).  Outside them: MOE_ERR_UNSUPPORTED. */
typedef struct {
  int64_t S;
  int32_t d;
  int32_t d_ff;
  int32_t E;
  int32_t K;
  int32_t n_groups;
  int32_t topk_groups;
  int32_t renormalize;
  int32_t act_dtype; /* moe_dtype */
  int32_t w_dtype;   /* moe_dtype */
  float gate_temperature;
  int32_t capacity;
  int32_t act_quant;
} moe_problem;

/* Host-only, pure helpers (no HIP call).  They return 0 / -1 for a problem
 * that fails validation. */

/* Bytes of device workspace the entry point `stage` needs for `p`. */
size_t moe_workspace_bytes(const moe_problem* p, int32_t stage);

/* Padding granule of the expert-contiguous buffers (x_perm, h, y_perm): each
 * expert's group of rows starts at a multiple of it. */
int32_t moe_tile_m(const moe_problem* p);

/* Rows x_perm, h and y_perm must hold: S*K + min(E, S*K) * (tile_m - 1). */
int64_t moe_rows_capacity(const moe_problem* p);

/* Static text for a status code. */
const char* moe_status_string(int32_t status);

/* Router and Top-K selection (chapter 11 sections 11.1.1-11.1.2; selection
 * bias and group limit: ybb.press section 2.3; one MoE forward and the
 * worked example: "MoE 混合专家推理", plumephp.com).
 *   x [S][d] act, W_r [E][d] act
 *   router_bias [E] (nullable): added to the scores; enters the gates.
 *   select_bias [E] (nullable): added to the scores for selection only.
 *   logits_in [S][E] (nullable): use these float32 scores instead of x W_r;
 *       x and W_r may then be NULL.  router_bias is not added to them.
 *   logits_out [S][E] (nullable): receives the float32 scores.
 *   topk_idx [S][K]: chosen experts per token, in slot order: key
 *       (score + select_bias) descending, equal keys by lower expert index.
 *   topk_gate [S][K]: float32 gate of each slot.
 *   ws: moe_workspace_bytes(p, MOE_STAGE_ROUTE) bytes (may be 0). */
int32_t moe_route(const moe_problem* p, const void* x, const void* W_r,
                  const float* router_bias, const float* select_bias,
                  const float* logits_in, float* logits_out,
                  int32_t* topk_idx, float* topk_gate,
                  void* ws, size_t ws_bytes, void* stream);

/* Dispatch: regroup the S*K (token, slot) pairs per expert (chapter 11
 * section 11.2.1).  Pair id = t*K + k.  Within an expert pairs keep token
 * order.
 *   topk_idx [S][K] int32 in [0, E) with distinct entries per token.  An
 *       entry outside [0, E) is skipped: that pair gets inv_perm -1, is
 *       counted nowhere, has no row, and moe_combine leaves it out.
 *   expert_counts [E]: pairs routed to each expert.
 *   expert_offsets [E+1]: first padded row of each expert's group; every
 *       entry is a multiple of moe_tile_m(p); entry E is the rows used.
 *   perm [S*K]: pair ids in (expert, token) order (no padding).
 *   inv_perm [S*K]: padded row of each pair.
 *   x_perm [moe_rows_capacity(p)][d] act: x_perm[inv_perm[t*K+k]] = x[t];
 *       padding rows are left untouched.
 *   ws: moe_workspace_bytes(p, MOE_STAGE_PERMUTE) bytes. */
int32_t moe_permute(const moe_problem* p, const int32_t* topk_idx, const void* x,
                    int32_t* expert_counts, int32_t* expert_offsets,
                    int32_t* perm, int32_t* inv_perm, void* x_perm,
                    void* ws, size_t ws_bytes, void* stream);

/* Expert FFN as a grouped GEMM over the expert-contiguous rows (chapter 11
 * section 11.1.2): for each real row r of expert e,
 *   h[r]      = GeLU(x_perm[r] W1_e + b1_e)   (act dtype; bf16 rounds once)
 *   y_perm[r] = h[r] W2_e + b2_e             (act dtype)
 * Padding rows of h and y_perm are unspecified.  Experts with no rows read
 * no weights.
 *   expert_counts, expert_offsets: as produced by moe_permute for this p.
 *   w1_scale, w2_scale: required for MOE_FP8_E4M3 weights, else ignored.
 *   h [rows_capacity][d_ff], y_perm [rows_capacity][d].
 *   ws: moe_workspace_bytes(p, MOE_STAGE_EXPERT_FFN) bytes, or NULL / fewer
 *       bytes.  With the full workspace the last, partly filled round of
 *       tiles of a GEMM is split along k over idle compute units (float32
 *       partial sums, reduced in a fixed order by a second kernel: results
 *       stay deterministic); without it the call runs unsplit.  Results of
 *       the two modes can differ in the last float32 bits. */
int32_t moe_expert_ffn(const moe_problem* p, const void* x_perm,
                       const int32_t* expert_counts, const int32_t* expert_offsets,
                       const void* W1, const void* b1, const void* W2, const void* b2,
                       const float* w1_scale, const float* w2_scale,
                       void* h, void* y_perm, void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe_expert_ffn, for callers that schedule them apart:
 *   moe_expert_up:   h[r]      = GeLU(x_perm[r] W1_e + b1_e)
 *   moe_expert_down: y_perm[r] = h[r] W2_e + b2_e
 * Arguments as for moe_expert_ffn (w1_scale / w2_scale required for fp8);
 * ws / ws_bytes as for moe_expert_ffn (nullable; may be shared by the two
 * calls when they run in order on one stream). */
int32_t moe_expert_up(const moe_problem* p, const void* x_perm, const int32_t* expert_counts,
                      const int32_t* expert_offsets, const void* W1, const void* b1,
                      const float* w1_scale, void* h, void* ws, size_t ws_bytes, void* stream);
int32_t moe_expert_down(const moe_problem* p, const void* h, const int32_t* expert_counts,
                        const int32_t* expert_offsets, const void* W2, const void* b2,
                        const float* w2_scale, void* y_perm, void* ws, size_t ws_bytes,
                        void* stream);

/* The two expert products with fp8 activations (W8A8, "MoE 推理工程深层实战"
 * section 3.3: FP8 E4M3 experts), stage by stage, for a problem with
 * act_quant = 1 (else MOE_ERR_INVALID_ARG):
 *   moe_expert_up_a8:   h[r]      = GeLU(dq(x8[r]) W1_e + b1_e)        (bf16)
 *   moe_expert_down_a8: y_perm[r] = dq(h8[r]) W2_e + b2_e             (bf16)
 * where dq(codes[r]) = decode(codes[r]) * scale[r]: e4m3 rows with one
 * float32 scale per row, as moe_quantize_rows writes them (the layer with
 * act_quant = 1 computes exactly what moe_permute's gather (for the same
 * problem with act_quant = 0), moe_quantize_rows of the gathered rows,
 * moe_expert_up_a8, moe_quantize_rows of h and moe_expert_down_a8 compute;
 * it quantises each token's row once and the up product reads those codes
 * in place).  Both operands go to the fp8 MFMAs; the float32 sum
 * is multiplied by row scale x channel scale in the epilogue.
 *   x8 [rows_capacity][d], h8 [rows_capacity][d_ff]: uint8 codes;
 *   x_scale, h_scale [rows_capacity] float32; w1_scale / w2_scale required.
 *   Other arguments and ws as for moe_expert_up / moe_expert_down. */
int32_t moe_expert_up_a8(const moe_problem* p, const uint8_t* x8, const float* x_scale,
                         const int32_t* expert_counts, const int32_t* expert_offsets,
                         const void* W1, const void* b1, const float* w1_scale, void* h,
                         void* ws, size_t ws_bytes, void* stream);
int32_t moe_expert_down_a8(const moe_problem* p, const uint8_t* h8, const float* h_scale,
                           const int32_t* expert_counts, const int32_t* expert_offsets,
                           const void* W2, const void* b2, const float* w2_scale, void* y_perm,
                           void* ws, size_t ws_bytes, void* stream);

/* Combine (chapter 11 sections 11.1.1 and 11.2.1; "MoE 混合专家推理", one
 * MoE forward): y[t] = sum over k = 0..K-1, in slot order, of
 * topk_gate[t][k] * y_perm[inv_perm[t*K+k]], accumulated in float32 and
 * rounded once to the act dtype; slots with inv_perm < 0 add nothing.  No
 * atomics. */
int32_t moe_combine(const moe_problem* p, const void* y_perm, const int32_t* inv_perm,
                    const float* topk_gate, void* y, void* stream);

/* Load statistics of one routing, computed on the device into
 * stats[MOE_STATS_N] (float32):
 *   MOE_STAT_MEAN, MOE_STAT_STD: mean and population standard deviation of
 *       expert_counts over the E experts ("MoE 推理工程深层实战" section 1.2:
 *       expert load balance is the standard deviation of the tokens each
 *       expert processes);
 *   MOE_STAT_MAX_OVER_MEAN: max / mean of expert_counts (chapter 11 section
 *       11.3.2: 1 is perfectly even, 3-5 is common); 0 when the mean is 0;
 *   MOE_STAT_DROP_RATE: dropped / (S*K) (section 1.2: token drop rate);
 *       0 when `dropped` is NULL or S = 0;
 *   MOE_STAT_AUX_LOSS: alpha * sum_i f_i * P_i (chapter 11 section 11.1.2,
 *       the balance loss) with f_i = expert_counts[i] / sum(expert_counts)
 *       and P_i = the mean over the S tokens of softmax(logits[t] / tau)[i],
 *       tau = p->gate_temperature (0 means 1); 0 when `logits` is NULL or
 *       there are no counts;
 *   MOE_STAT_MAX, MOE_STAT_MIN, MOE_STAT_EMPTY: largest and smallest count
 *       and the number of experts with none.
 * Arguments (device pointers): expert_counts [E] int32 (as moe_permute
 * writes them), logits [S][E] float32 (nullable; as moe_route writes them),
 * dropped [1] int32 (nullable: pairs that were routed to no expert), stats
 * [MOE_STATS_N] float32 (written).  The sums are taken in a fixed order, so
 * the result is deterministic.  Needs no workspace. */
enum {
  MOE_STAT_MEAN = 0,
  MOE_STAT_STD = 1,
  MOE_STAT_MAX_OVER_MEAN = 2,
  MOE_STAT_DROP_RATE = 3,
  MOE_STAT_AUX_LOSS = 4,
  MOE_STAT_MAX = 5,
  MOE_STAT_MIN = 6,
  MOE_STAT_EMPTY = 7,
  MOE_STATS_N = 8
};
int32_t moe_load_stats(const moe_problem* p, const int32_t* expert_counts, const float* logits,
                       const int32_t* dropped, float alpha, float* stats, void* stream);

/* Per-row fp8 quantisation of bf16 activations ("MoE 推理工程深层实战"
 * section 3.3: FP8 E4M3 is the production format for experts; here it is
 * applied to the activations of the W8A8 expert products).  For each row r
 * of src [rows][n] (bf16), with amax the largest |value| of the row:
 *     scales[r] = amax / 448,   codes[r][i] = e4m3(clamp(v * (448 / amax),
 *     -448, 448)), round to nearest even (OCP E4M3FN codes),
 * each quotient and product one float32 operation; the row's value is
 * decode(code) * scale.  A row of zeros gets scale 0 and codes 0.  Where
 * 448 / amax overflows float32 (amax below about 1.3e-36) the row and amax
 * are first multiplied by 2^64 (exact): codes = e4m3(clamp((v * 2^64) *
 * (448 / (amax * 2^64)))), what an unbounded exponent range would give.
 *   codes [rows][n] uint8 and scales [rows] float32 are written.
 *   n: a positive multiple of 8; rows >= 0 (0 is a no-op), < 2^26 (else
 *   MOE_ERR_UNSUPPORTED).
 * Needs no workspace and no moe_problem. */
int32_t moe_quantize_rows(const void* src, int64_t rows, int32_t n, uint8_t* codes, float* scales,
                          void* stream);

/* Capacity-limited dispatch (chapter 11 section 11.3.3, expert dropping:
 * the excess of an overloaded expert moves to the next-best expert;
 * "MoE 推理工程深层实战" sections 1.2 and 2.2: token drop rate, tokens past a
 * buffer's capacity are dropped).  The pages leave the rule open; it is:
 *  - rounds: every pending (token, slot) pair proposes its current expert;
 *    the expert accepts proposals in (token, slot) order while it holds
 *    fewer than p->capacity pairs;
 *  - a rejected pair moves to the best expert in its token's selection order
 *    (logit + select_bias, eligible groups only, key descending, lower index
 *    on ties; the order moe_route uses) that has room and that the token
 *    does not hold in another accepted or pending slot; a token's rejected
 *    slots are taken in slot order; with no such expert the pair is dropped
 *    (index -1);
 *  - a slot keeps its position; gates are recomputed over each token's kept
 *    slots as moe_route computes them (dropped slots get 0), so a token that
 *    keeps all its slots keeps its gates bit for bit.
 * p->capacity = 0 means no limit (nothing moves).
 *   logits [S][E] float32: the router scores (as moe_route's logits_out).
 *   select_bias [E] (nullable): the selection-only bias moe_route used.
 *   topk_idx [S][K] int32, in/out: the routing on entry (indices outside
 *       [0, E) count as dropped pairs and become -1); the capacity-limited
 *       routing on return.
 *   topk_gate [S][K] float32, out.
 *   dropped [1] int32 (nullable): pairs with index -1 on return.
 *   ws: moe_workspace_bytes(p, MOE_STAGE_CAPACITY) bytes.
 * moe_permute, moe_combine and moe_load_stats accept the -1 entries.  One
 * workgroup runs the rounds (at most E + 1), so the call costs more than
 * moe_route for large S; the result is deterministic. */
int32_t moe_apply_capacity(const moe_problem* p, const float* logits, const float* select_bias,
                           int32_t* topk_idx, float* topk_gate, int32_t* dropped, void* ws,
                           size_t ws_bytes, void* stream);

/* The whole layer: route, permute, expert FFN, combine on one stream.
 *   y [S][d] act.  Optional outputs (nullable): topk_idx_out [S][K],
 *   topk_gate_out [S][K], logits_out [S][E], expert_counts_out [E].
 *   With p->capacity > 0 the routing passes through moe_apply_capacity's
 *   rule before the permute; dropped pairs then have topk_idx -1 and the
 *   dropped count is S*K minus the sum of expert_counts_out.
 *   ws: moe_workspace_bytes(p, MOE_STAGE_LAYER) bytes. */
int32_t moe_layer_forward(const moe_problem* p, const void* x, const void* W_r,
                          const float* router_bias, const float* select_bias,
                          const void* W1, const void* b1, const void* W2, const void* b2,
                          const float* w1_scale, const float* w2_scale, void* y,
                          int32_t* topk_idx_out, float* topk_gate_out,
                          float* logits_out, int32_t* expert_counts_out,
                          void* ws, size_t ws_bytes, void* stream);

/* Bytes of the library's own scratch array (one per GPU), the workspace of
 * moe_layer_forward_noalloc: 128 MiB. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)

/* moe_layer_forward for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, meaning and results as moe_layer_forward
 * (bit-identical outputs for the same inputs), without ws / ws_bytes: the
 * workspace is a file-scope device array of MOE_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on until the process ends.
 *  - Problems with moe_workspace_bytes(p, MOE_STAGE_LAYER) above
 *    MOE_NOALLOC_SCRATCH_BYTES return MOE_ERR_TOO_LARGE before anything is
 *    launched (this covers decode-sized batches: e.g. up to 255 tokens at
 *    d = 4096, d_ff = 14336, E = 8, K = 2, or 16 tokens at d = 7168,
 *    d_ff = 2048, E = 256, K = 8).  Other validation as moe_layer_forward.
 *  - The call allocates nothing: no hipMalloc, hipFree or allocating
 *    library routine.  The first call on a GPU looks up that GPU's copy of
 *    the array (hipGetSymbolAddress, on the stream's device) and keeps the
 *    address; make that first call outside graph capture.
 *  - Every call on one GPU uses the same array, which keeps the last call's
 *    contents (no kernel of the layer depends on them: each initialises the
 *    state it reads).  Calls that overlap on one GPU -- concurrent streams,
 *    or replays of several captured graphs at once -- race on it; order them
 *    on one stream or use moe_layer_forward with separate workspaces. */
int32_t moe_layer_forward_noalloc(const moe_problem* p, const void* x, const void* W_r,
                                  const float* router_bias, const float* select_bias,
                                  const void* W1, const void* b1, const void* W2, const void* b2,
                                  const float* w1_scale, const float* w2_scale, void* y,
                                  int32_t* topk_idx_out, float* topk_gate_out,
                                  float* logits_out, int32_t* expert_counts_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FFN_LAYER_MOE_H */
