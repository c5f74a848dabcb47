"""Plain, slow CPU reference of the single-GPU MoE-layer forward.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this module.  It shares no code with the HIP path.

Sources (cited below by short name, section and equation):
  [P1] "MoE 推理工程深层实战：专家并行、负载均衡、Expert Offloading 与生产级 Serving"
       (ybb.press) -- section 2.3 gives the DeepSeek-V3 style biased,
       node(group)-limited Top-K router as pseudocode.
  [P2] "大模型推理技术 | 第11章 MoE模型推理" (jsqmd.com) -- section 11.1.1 (MoE
       output as a router-weighted sum of experts, softmax router, TopK
       operator), section 11.1.2 (expert FFN GeLU(xW1+b1)W2+b2, router
       s = Softmax(x W_r), B x L x K expert forwards grouped per expert),
       section 11.2.1 (regrouping tokens per expert and back), section 11.3.1
       (the forward of an expert-parallel layer in PyTorch-like code).
  [P3] "MoE 混合专家推理：路由、负载均衡与显存策略" (plumephp.com) -- the
       'one MoE forward' block and the worked routing example (e0 .55,
       e3 .30 -> Top-2 = e0, e3, normalised weighting).

Precision.  Inputs are decoded exactly to float64 (bf16 and fp8-e4m3 values
are exact in float64; an fp8 weight times its fp32 channel scale is exact
too).  Every sum is taken in float64 with no intermediate rounding.  Routing
is a function of float32 logits (the form the GPU produces and consumes):
the router product is accumulated in float64 and rounded once to float32.

Readings where the pages are silent or ambiguous (each is stated where used):
  * TopK keeps the K largest keys; equal keys go to the lower expert index,
    equal group scores to the lower group index.
  * Softmax then TopK compose as softmax over the K chosen (gates sum to 1),
    which is the 'normalised weighting' of P3's worked example; the
    unnormalised variant (raw full-softmax probabilities of the chosen
    experts, as P2 section 11.3.1's code multiplies) is renormalize=0.
  * Group score = float32 sum of the group's biased logits in a fixed
    pairwise-halving tree: v[j] += v[j+w] for w = m/2, m/4, ..., 1.
  * GeLU is the exact x*Phi(x) with erf.
  * The selection-only bias (P1 section 2.3) enters the keys; gates use the
    unbiased logits.
  * Capacity-limited dispatch (P2 11.3.3, P1 sections 1.2 and 2.2 leave the
    rule open): rounds of in-order acceptance, rejected pairs move to the
    token's best expert that still has room; see apply_capacity.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "decode_bf16", "decode_e4m3fn", "decode", "expert_matrix",
    "router_logits", "softmax", "group_scores_f32", "select_experts",
    "gate_weights", "permute", "gelu", "expert_ffn", "layer_forward",
    "combine", "load_stats", "STAT_NAMES", "selection_keys", "apply_capacity",
    "E4M3_MAX", "encode_e4m3fn", "quantize_rows_e4m3", "dequantize_rows_e4m3", "expert_ffn_w8a8",
]


# ---------------------------------------------------------------- decoding
def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    A bfloat16 is the upper half of an IEEE binary32 word, so widening the
    pattern by 16 zero bits gives the exact float32 value.
    """
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_value(c: np.ndarray) -> np.ndarray:
    """OCP 8-bit floating point E4M3 ('fn': finite, no infinities) -> float64.

    Sign bit 7, exponent bits 6..3 with bias 7, mantissa bits 2..0.  Exponent
    field 0 is subnormal: m/8 * 2^-6.  Otherwise (1 + m/8) * 2^(e-7).  The
    pattern S.1111.111 is NaN; there is no infinity, so the largest finite
    magnitude is 1.75 * 2^8 = 448.
    """
    c = np.asarray(c).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = s * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


_E4M3FN_TABLE = _e4m3fn_value(np.arange(256))


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """e4m3fn codes (uint8) -> float64 by the definition above, evaluated
    once for all 256 codes and looked up."""
    return _E4M3FN_TABLE[np.asarray(codes).astype(np.uint8)]


E4M3_MAX = 448.0


def encode_e4m3fn(v: np.ndarray) -> np.ndarray:
    """float32 values with |v| <= 448 -> the nearest e4m3fn code (uint8),
    ties to the even code (the code's last bit is the mantissa's last bit,
    and codes of one sign are ordered by magnitude).  The sign bit follows
    the sign of v, so -0.0 and small negatives that round to zero give 0x80.
    Written from the format's definition (decode_e4m3fn) by a nearest-value
    search over the 127 finite non-negative codes."""
    v = np.asarray(v, dtype=np.float32)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("encode_e4m3fn takes finite values with |v| <= 448")
    mags = _E4M3FN_TABLE[:0x7F]                      # codes 0x00..0x7E, increasing
    a = np.abs(v).astype(np.float64)
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_rows_e4m3(v: np.ndarray):
    """Per-row fp8 quantisation of activations: for each row with amax the
    largest |v|, the scale is s = amax / 448 and the codes are q =
    encode(clip(v * r, -448, 448)) with r = 448 / amax (each quotient and
    the product one float32 operation); the row's value is decode(q) * s.
    A row of zeros gets s = 0 and codes 0.  When 448 / amax overflows
    float32 (amax below about 1.3e-36, which bf16 rows can reach) the row and amax are first multiplied by 2^64 (exact), so that
    r = 448 / (amax 2^64) and t = (v 2^64) r: the codes the same steps give
    with an unbounded exponent range (reading: the pages fix the per-row
    scale, not float32's overflow).
    FP8 E4M3 is the format the pages recommend for expert weights ([P1]
    section 3.3); applying it to the activations with a per-row (per-token)
    scale is the W8A8 reading, so that both GEMM operands are fp8.
    v: float32 [R, n].  Returns (codes uint8 [R, n], scales float32 [R])."""
    v = np.asarray(v, dtype=np.float32)
    amax = np.abs(v).max(axis=1) if v.shape[1] else np.zeros(v.shape[0], np.float32)
    amax = amax.astype(np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    safe = np.where(amax > 0, amax, np.float32(1.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        tiny = np.isinf((np.float32(E4M3_MAX) / safe).astype(np.float32))   # 448 / amax overflows
    pre = np.where(tiny, np.float32(2.0 ** 64), np.float32(1.0)).astype(np.float32)
    r = (np.float32(E4M3_MAX) / (safe * pre).astype(np.float32)).astype(np.float32)
    t = ((v * pre[:, None]).astype(np.float32) * r[:, None]).astype(np.float32)
    t = np.clip(t, np.float32(-E4M3_MAX), np.float32(E4M3_MAX)).astype(np.float32)
    codes = encode_e4m3fn(t)
    codes[s == 0] = 0
    return codes, s


def dequantize_rows_e4m3(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """decode(q) * s per row, float64 (exact: a 4-bit significand times a
    float32)."""
    return decode_e4m3fn(codes) * np.asarray(scales, dtype=np.float32).astype(np.float64)[:, None]


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float64.  dtype: 'f32' (float32 values), 'bf16'
    (uint16 patterns) or 'fp8' (uint8 e4m3fn codes)."""
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return decode_bf16(arr)
    if dtype == "fp8":
        return decode_e4m3fn(arr)
    raise ValueError(dtype)


def expert_matrix(w: np.ndarray, dtype: str, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """One expert's stored weight [out, in] -> float64 value W[out, in].

    For fp8 weights the value of a code q in output channel n is dec(q) *
    scale[n] (per-output-channel scale)."""
    v = decode(w, dtype)
    if scale is not None:
        v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]
    return v


# ---------------------------------------------------------------- router
def router_logits(x: np.ndarray, w_r: np.ndarray, router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Router scores s = x . W_r (+ bias), rounded once to float32.

    [P2] section 11.1.2 writes the router as Softmax(x W_r) (section 11.1.1
    writes W_r x; both are the same product for row-vector tokens) and its
    section 11.3.1 code uses a linear layer, which may carry a bias.
    x: float64 [S, d]; w_r: float64 [E, d] (linear-layer layout, so the
    product is x @ w_r.T); router_bias: float32 [E] or None.
    """
    acc = x @ w_r.T
    if router_bias is not None:
        acc = acc + np.asarray(router_bias, dtype=np.float32).astype(np.float64)[None, :]
    return acc.astype(np.float32)


def softmax(logits: np.ndarray, temperature: float = 1.0) -> np.ndarray:
    """Softmax over experts (last axis) in float64 ([P2] 11.1.1; [P3] routing
    scores: a probability distribution over the experts).  `temperature` is
    [P2] 11.3.3's tau: the distribution of exp(s_i / tau), s the scores."""
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max(axis=-1, keepdims=True)
    p = np.exp(z)
    return p / p.sum(axis=-1, keepdims=True)


def group_scores_f32(keys: np.ndarray, n_groups: int) -> np.ndarray:
    """Score of each group of m = E/n_groups consecutive experts: the sum of
    the group's (biased) logits ([P1] section 2.3: the biased logits are
    viewed as [tokens, nodes, experts per node] and summed over the last
    axis).  Taken in float32 with a fixed pairwise-halving tree so that both
    implementations round identically: v[j] = v[j] + v[j + w] for
    w = m/2, m/4, ..., 1; the result is v[0].  m must be a power of two.
    """
    keys = np.asarray(keys, dtype=np.float32)
    S, E = keys.shape
    m = E // n_groups
    if m * n_groups != E or m & (m - 1):
        raise ValueError("E/n_groups must be a power of two")
    v = keys.reshape(S, n_groups, m).copy()
    w = m // 2
    while w >= 1:
        v[:, :, :w] = v[:, :, :w] + v[:, :, w:2 * w]
        w //= 2
    return v[:, :, 0].copy()


def select_experts(logits: np.ndarray, K: int, select_bias: Optional[np.ndarray] = None,
                   n_groups: int = 1, topk_groups: int = 1) -> np.ndarray:
    """Top-K expert indices per token, [S, K] int32, in slot order.

    key = logit (float32), plus the selection-only per-expert bias as one
    float32 add when given ([P1] section 2.3, aux-loss-free router).  With
    n_groups > 1 the experts outside the token's topk_groups best groups get
    key -inf before the Top-K ([P1] section 2.3: top-2 nodes by summed biased
    logit, others masked).  TopK keeps the K largest keys and drops the rest
    ([P2] 11.1.1 TopK operator); a stable sort by key descending gives that,
    with equal keys ordered by lower expert index.  The slot order is that
    sort order.
    """
    key = np.asarray(logits, dtype=np.float32)
    if select_bias is not None:
        key = (key + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)
    S, E = key.shape
    if not 1 <= K <= E:
        raise ValueError("need 1 <= K <= E")
    if n_groups > 1:
        gs = group_scores_f32(key, n_groups)
        g_order = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]
        keep = np.zeros((S, n_groups), dtype=bool)
        np.put_along_axis(keep, g_order, True, axis=1)
        keep_e = np.repeat(keep, E // n_groups, axis=1)
        key = np.where(keep_e, key, np.float32(-np.inf)).astype(np.float32)
    order = np.argsort(-key, axis=1, kind="stable")
    return order[:, :K].astype(np.int32)


def gate_weights(logits: np.ndarray, idx: np.ndarray, renormalize: int = 1,
                 temperature: float = 1.0) -> np.ndarray:
    """Gate weight of each chosen expert, float64 [S, K].

    renormalize=1: softmax restricted to the K chosen (unbiased) logits, so
    the gates of a token sum to 1 -- softmax applied after TopK has set the
    other scores to -inf ([P2] 11.1.1), the normalised weighting of [P3]'s
    worked example.  renormalize=0: the chosen experts' probabilities under
    the full softmax, as [P2] section 11.3.1's code multiplies them.
    Both take the scores divided by `temperature` ([P2] 11.3.3, soft routing:
    a higher tau spreads the weights more evenly); selection does not use it.
    """
    l = np.asarray(logits, dtype=np.float32).astype(np.float64)
    chosen = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    if renormalize:
        return softmax(chosen, temperature)
    p = softmax(l, temperature)
    return np.take_along_axis(p, idx.astype(np.int64), axis=1)


# ---------------------------------------------------------------- capacity
def selection_keys(logits: np.ndarray, select_bias: Optional[np.ndarray] = None, n_groups: int = 1,
                   topk_groups: int = 1) -> np.ndarray:
    """The float32 keys select_experts ranks, with -inf for experts outside
    the token's kept groups (the same steps as select_experts)."""
    key = np.asarray(logits, dtype=np.float32)
    if select_bias is not None:
        key = (key + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)
    S, E = key.shape
    if n_groups > 1:
        gs = group_scores_f32(key, n_groups)
        g_order = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]
        keep = np.zeros((S, n_groups), dtype=bool)
        np.put_along_axis(keep, g_order, True, axis=1)
        key = np.where(np.repeat(keep, E // n_groups, axis=1), key, np.float32(-np.inf)).astype(np.float32)
    return key


def apply_capacity(logits: np.ndarray, idx: np.ndarray, capacity: int,
                   select_bias: Optional[np.ndarray] = None, n_groups: int = 1, topk_groups: int = 1,
                   renormalize: int = 1, temperature: float = 1.0):
    """Capacity-limited dispatch: each expert takes at most `capacity` of the
    routed (token, slot) pairs; pairs past the limit go to the next-best
    expert, and are dropped when none has room ([P2] 11.3.3, expert dropping:
    the excess of an overloaded expert moves to the next-best expert; [P1]
    section 1.2, token drop rate: the share of tokens lost to overloaded
    experts; [P1] section 2.2: tokens past a buffer's capacity are dropped or
    held back in an overflow buffer).

    The pages leave the rule open; the reading taken:
      * rounds: every pending pair proposes its current expert; an expert
        accepts proposals in (token, slot) order while it has room;
      * a rejected pair moves to the best expert of its token's ranking (the
        selection keys of select_experts, kept groups only; key descending,
        lower index on ties) that the token does not hold in another
        accepted or pending slot and that still has room; the token's slots
        are taken in slot order, so two of them never pick the same expert;
        with no such expert the pair is dropped (index -1);
      * a slot keeps its position; the gates are those of gate_weights over
        the token's kept slots (dropped slots get 0).
    Each round with a rejection fills at least one more expert, so it ends.
    capacity 0 means no limit.  Input indices outside [0, E) count as
    dropped pairs.  Returns (idx [S,K] int32, gates [S,K] float64, number of
    pairs with index -1).
    """
    if capacity < 0:
        raise ValueError("capacity must be >= 0")
    if capacity == 0:                           # no limit
        capacity = np.iinfo(np.int64).max
    key = selection_keys(logits, select_bias, n_groups, topk_groups)
    S, E = key.shape
    K = idx.shape[1]
    ranking = np.argsort(-key, axis=1, kind="stable")
    allowed = key > -np.inf
    cur = np.asarray(idx, dtype=np.int64).copy()
    cur[(cur < 0) | (cur >= E)] = -1            # pairs routed to no expert stay dropped
    PENDING, ACCEPTED, REJECTED, DROPPED = 0, 1, 2, 3
    state = np.where(cur >= 0, PENDING, DROPPED)
    dropped = int((cur < 0).sum())
    load = np.zeros(E, dtype=np.int64)
    while (state == PENDING).any():
        for t in range(S):                      # acceptance in (token, slot) order
            for k in range(K):
                if state[t, k] == PENDING:
                    e = cur[t, k]
                    if load[e] < capacity:
                        load[e] += 1
                        state[t, k] = ACCEPTED
                    else:
                        state[t, k] = REJECTED
        for t in range(S):                      # rerouting
            for k in range(K):
                if state[t, k] != REJECTED:
                    continue
                held = {int(cur[t, j]) for j in range(K)
                        if j != k and state[t, j] in (PENDING, ACCEPTED)}
                nxt = [int(e) for e in ranking[t] if allowed[t, e] and int(e) not in held and load[e] < capacity]
                if nxt:
                    cur[t, k] = nxt[0]
                    state[t, k] = PENDING
                else:
                    cur[t, k] = -1
                    state[t, k] = DROPPED
                    dropped += 1
    gates = np.zeros((S, K), dtype=np.float64)
    for t in range(S):
        kept = np.nonzero(cur[t] >= 0)[0]
        if kept.size:
            gates[t, kept] = gate_weights(logits[t:t + 1], cur[t:t + 1, kept], renormalize, temperature)[0]
    return cur.astype(np.int32), gates, dropped


# ---------------------------------------------------------------- statistics
STAT_NAMES = ("mean", "std", "max_over_mean", "drop_rate", "aux_loss", "max", "min", "empty")


def load_stats(counts: np.ndarray, S: int, K: int, logits: Optional[np.ndarray] = None,
               alpha: float = 1.0, temperature: float = 1.0, dropped: int = 0) -> Dict[str, float]:
    """Load statistics of one routing, float64.

    [P1] section 1.2: expert load balance is the standard deviation of the
    tokens each expert processes (taken here over the E per-expert counts,
    population form) and the token drop rate is the share of routed pairs
    that overloaded experts dropped (dropped / (S*K)).  [P2] 11.3.2: the
    evaluation metric is max load / mean load.  [P2] 11.1.2: the balance loss
    alpha * sum_i f_i * P_i, with f_i the share of the routed assignments
    that went to expert i and P_i the router's mean probability for expert i
    over the S tokens (the softmax of the scores, at `temperature`).
    """
    c = np.asarray(counts, dtype=np.float64)
    E = c.size
    mean = c.sum() / E
    out = {"mean": mean, "std": float(np.sqrt(((c - mean) ** 2).sum() / E)),
           "max_over_mean": float(c.max() / mean) if mean > 0 else 0.0,
           "drop_rate": float(dropped) / (S * K) if S * K > 0 else 0.0,
           "aux_loss": 0.0, "max": float(c.max()), "min": float(c.min()),
           "empty": float((c == 0).sum())}
    if logits is not None and c.sum() > 0 and S > 0:
        f = c / c.sum()
        P = softmax(np.asarray(logits, dtype=np.float32), temperature).mean(axis=0)
        out["aux_loss"] = float(alpha * (f * P).sum())
    return out


# ---------------------------------------------------------------- dispatch
def permute(idx: np.ndarray, E: int, tile_m: int) -> Dict[str, np.ndarray]:
    """Regroup the S*K (token, slot) pairs per expert ([P2] 11.2.1: tokens of
    one expert are gathered together before the expert runs; 11.1.2: S x K
    expert forwards grouped per expert).

    Pair id p = t*K + k.  Within an expert the pairs keep token order (a
    stable counting sort), so the grouping is unique.
    Returns
      counts [E]         pairs routed to each expert
      dense_offsets [E+1] exclusive prefix sum of counts
      offsets [E+1]      prefix sum of counts rounded up to tile_m (row where
                         each expert's group starts in the padded buffer)
      perm [S*K]         pair ids in (expert, token) order
      rank [S*K]         position of each pair inside its expert's group
      inv_perm [S*K]     padded row of each pair: offsets[e] + rank
    """
    idx = np.asarray(idx, dtype=np.int64)
    S, K = idx.shape
    flat = idx.reshape(-1)
    counts = np.zeros(E, dtype=np.int64)
    rank = np.zeros(S * K, dtype=np.int64)
    for p in range(S * K):            # first pass: ranks in token order
        e = flat[p]
        rank[p] = counts[e]
        counts[e] += 1
    dense = np.zeros(E + 1, dtype=np.int64)
    dense[1:] = np.cumsum(counts)
    padded = np.zeros(E + 1, dtype=np.int64)
    padded[1:] = np.cumsum((counts + tile_m - 1) // tile_m * tile_m)
    perm = np.empty(S * K, dtype=np.int64)
    perm[dense[flat] + rank] = np.arange(S * K)   # second pass: scatter
    inv = padded[flat] + rank
    return {"counts": counts.astype(np.int32), "dense_offsets": dense.astype(np.int32),
            "offsets": padded.astype(np.int32), "perm": perm.astype(np.int32),
            "rank": rank.astype(np.int32), "inv_perm": inv.astype(np.int32)}


# ---------------------------------------------------------------- experts
def gelu(a: np.ndarray) -> np.ndarray:
    """GeLU(a) = a * Phi(a) = a/2 * (1 + erf(a / sqrt 2)) (exact form)."""
    return 0.5 * a * (1.0 + _erf(a / math.sqrt(2.0)))


def expert_ffn(x_rows: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray,
               b2: np.ndarray, return_hidden: bool = False):
    """E_i(x) = GeLU(x W1 + b1) W2 + b2 for each row ([P2] 11.1.2).

    Weights are in linear-layer layout: w1 [d_ff, d], w2 [d, d_ff] (W1 and
    W2 transposed), all float64.
    """
    a = x_rows @ w1.T + b1[None, :]
    h = gelu(a)
    o = h @ w2.T + b2[None, :]
    return (h, o) if return_hidden else o


def expert_ffn_w8a8(x_rows: np.ndarray, w1: np.ndarray, b1: np.ndarray, w2: np.ndarray,
                    b2: np.ndarray, return_hidden: bool = False):
    """The expert FFN with fp8 activations (W8A8): the rows entering each
    product are quantised per row (quantize_rows_e4m3) first.
      x -> (qx, sx);  h = GeLU(dequant(qx, sx) W1 + b1);
      h -> (qh, sh);  out = dequant(qh, sh) W2 + b2.
    x_rows float64 holding float32 values (bf16 activations are exact); h is
    quantised from its float32 rounding.  Weights as in expert_ffn (float64,
    fp8 weights already times their channel scale)."""
    qx, sx = quantize_rows_e4m3(x_rows.astype(np.float32))
    a = dequantize_rows_e4m3(qx, sx) @ w1.T + b1[None, :]
    h = gelu(a)
    qh, sh = quantize_rows_e4m3(h.astype(np.float32))
    o = dequantize_rows_e4m3(qh, sh) @ w2.T + b2[None, :]
    return (h, o) if return_hidden else o


def combine(gates: np.ndarray, outputs: np.ndarray) -> np.ndarray:
    """y[t] = sum_k gate[t,k] * E_{idx[t,k]}(x_t) ([P2] 11.1.1 weighted sum;
    [P3] one MoE forward: outputs weighted by score and summed).
    gates [S,K] float64, outputs [S,K,d] float64 -> [S,d] float64."""
    return np.einsum("sk,skd->sd", gates, outputs)


def layer_forward(x: np.ndarray, w_r: np.ndarray, W1, b1, W2, b2, *, K: int,
                  act: str, w: str, router_bias=None, select_bias=None,
                  n_groups: int = 1, topk_groups: int = 1, renormalize: int = 1,
                  temperature: float = 1.0, w1_scale=None, w2_scale=None, logits_in=None,
                  tokens: Optional[Sequence[int]] = None, capacity: int = 0,
                  act_quant: bool = False, return_parts: bool = False):
    """The whole layer for the tokens `tokens` (default: all), [P2] 11.1.1-2.

    x [S,d] and w_r [E,d] are storage arrays of dtype `act`; W1 [E][d_ff,d],
    W2 [E][d,d_ff] storage arrays of dtype `w` (anything indexable by expert:
    only the experts in use are read); b1 [E][d_ff], b2 [E][d] of dtype
    `act`; w1_scale [E][d_ff], w2_scale [E][d] float32 for fp8 weights.
    logits_in [S,E] float32 replaces the router product when given.
    act_quant: fp8 activations in both expert products (expert_ffn_w8a8).
    capacity > 0 limits each expert to that many (token, slot) pairs with
    apply_capacity; that rule looks at every token, so the routing is then
    computed for all S tokens before `tokens` are picked.

    Steps: router logits -> selection -> gates -> for each expert in index
    order, the expert FFN of every (token, slot) pair routed to it -> gate
    weighted sum per token.  Returns y [n_tokens, d] float64 or, with
    return_parts, a dict with y, logits, idx, gates, hidden/out per pair.
    """
    S = x.shape[0]
    tok = np.arange(S) if tokens is None else np.asarray(tokens, dtype=np.int64)
    xs = decode(np.asarray(x)[tok], act)
    if capacity:
        if logits_in is not None:
            full = np.asarray(logits_in, dtype=np.float32)
        else:
            full = router_logits(decode(np.asarray(x), act), decode(w_r, act), router_bias)
        idx_all = select_experts(full, K, select_bias, n_groups, topk_groups)
        idx_all, gates_all, _ = apply_capacity(full, idx_all, capacity, select_bias, n_groups,
                                               topk_groups, renormalize, temperature)
        logits, idx, gates = full[tok], idx_all[tok], gates_all[tok]
    else:
        if logits_in is not None:
            logits = np.asarray(logits_in, dtype=np.float32)[tok]
        else:
            logits = router_logits(xs, decode(w_r, act), router_bias)
        idx = select_experts(logits, K, select_bias, n_groups, topk_groups)
        gates = gate_weights(logits, idx, renormalize, temperature)
    n, d = xs.shape
    outs = np.zeros((n, K, d), dtype=np.float64)
    hidden = {} if return_parts else None
    for e in np.unique(idx[idx >= 0]):       # experts in index order; dropped pairs add nothing
        rows, slots = np.nonzero(idx == e)   # pairs routed to e, token order
        s1 = None if w1_scale is None else w1_scale[e]
        s2 = None if w2_scale is None else w2_scale[e]
        W1e = expert_matrix(W1[e], w, s1)
        W2e = expert_matrix(W2[e], w, s2)
        ffn = expert_ffn_w8a8 if act_quant else expert_ffn
        h, o = ffn(xs[rows], W1e, decode(b1[e], act), W2e, decode(b2[e], act), return_hidden=True)
        outs[rows, slots] = o
        if return_parts:
            hidden[int(e)] = (rows, slots, h)
    y = combine(gates, outs)
    if not return_parts:
        return y
    return {"y": y, "logits": logits, "idx": idx, "gates": gates, "outs": outs,
            "hidden": hidden, "tokens": tok}
