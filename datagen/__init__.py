"""Seeded synthetic inputs for the MoE-layer forward.

This module is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark.  It holds none of the layer's arithmetic: no router product, no
softmax, no Top-K, no expert FFN.  It only draws random numbers, rounds them
to their storage types and, for fp8 expert weights, quantises each output
channel with its own fp32 scale.

Every value is a pure function of (seed, tensor tag, element index): a
counter-based generator built from a 32-bit integer mixer evaluated with
torch integer ops.  The same code therefore produces bit-identical tensors on
the CPU and on the GPU, and any slice (one expert's weights, one token's row)
can be regenerated alone.

Distributions
-------------
* "N(0, v)" is read as mean 0, variance v (so W ~ N(0, 1/fan_in)).  A normal
  draw is the variance-matched sum of four uniform 16-bit integers
  (Irwin-Hall, n = 4), scaled once in fp32.  It is bounded at +-3.46 sigma;
  nothing downstream depends on the far tails.
* Uniform U(-a, a) uses 24 bits of one word.
* The Zipf(s) draws of the skewed-routing recipe use rejection-inversion
  sampling (Hoermann & Derflinger, 1996) in float64 on the host.

Weight storage follows torch.nn.Linear ([out_features, in_features]):
W_r [E, d], W1 [E, d_ff, d], W2 [E, d, d_ff].  The layer still computes
x.W1 in the pages' notation; the stored matrix is W1 transposed.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

_M32 = 0xFFFFFFFF
# standard deviation of the sum of four independent uniform draws on {0..65535}
_IH4_STD = math.sqrt(4.0 * (65536.0 ** 2 - 1.0) / 12.0)
_IH4_MEAN = 2 * 65535


# ---------------------------------------------------------------- generator
def _mul32(x: torch.Tensor, c: int) -> torch.Tensor:
    """(x * c) mod 2^32 for x in [0, 2^32) held in int64, without overflow."""
    lo, hi = c & 0xFFFF, c >> 16
    return (x * lo + (((x * hi) & 0xFFFF) << 16)) & _M32


def _mix32(x: torch.Tensor) -> torch.Tensor:
    """A 32-bit avalanche mixer (xorshift-multiply, 'lowbias32' constants)."""
    x = x ^ (x >> 16)
    x = _mul32(x, 0x7FEB352D)
    x = x ^ (x >> 15)
    x = _mul32(x, 0x846CA68B)
    x = x ^ (x >> 16)
    return x


def _keys(seed: int, tag: Sequence) -> tuple:
    h = hashlib.blake2b(repr((int(seed),) + tuple(tag)).encode(), digest_size=16).digest()
    return tuple(int.from_bytes(h[4 * i:4 * i + 4], "little") for i in range(4))


def _words(seed: int, tag: Sequence, count: int, device, start: int = 0):
    """Two independent 32-bit words per element index in [start, start+count)."""
    if start + count > 1 << 32:
        raise ValueError("a single stream holds at most 2^32 elements; split the tag")
    k = _keys(seed, tag)
    i = torch.arange(start, start + count, dtype=torch.int64, device=device)
    a = _mix32(_mix32(i ^ k[0]) ^ k[1])
    return _mix32(a ^ k[2]), _mix32(a ^ k[3])


def normal(seed, tag, shape, var: float, device="cpu", start: int = 0) -> torch.Tensor:
    """float32 tensor of approximately N(0, var) draws (Irwin-Hall, n=4)."""
    n = int(np.prod(shape)) if len(shape) else 1
    w1, w2 = _words(seed, tag, n, device, start)
    s = (w1 & 0xFFFF) + (w1 >> 16) + (w2 & 0xFFFF) + (w2 >> 16) - _IH4_MEAN
    c = torch.tensor(math.sqrt(var) / _IH4_STD, dtype=torch.float32, device=device)
    return (s.to(torch.float32) * c).reshape(shape)


def uniform(seed, tag, shape, a: float, device="cpu") -> torch.Tensor:
    """float32 tensor of U(-a, a) draws on a 2^24-point grid."""
    n = int(np.prod(shape)) if len(shape) else 1
    w1, _ = _words(seed, tag, n, device)
    c = torch.tensor(a / float(1 << 23), dtype=torch.float32, device=device)
    return (((w1 >> 8) - (1 << 23)).to(torch.float32) * c).reshape(shape)


def uniform01_host(seed, tag, n: int) -> np.ndarray:
    """float64 uniforms in the open interval (0, 1), 53 random bits each."""
    w1, w2 = _words(seed, tag, n, "cpu")
    w1 = w1.numpy().astype(np.uint64)
    w2 = w2.numpy().astype(np.uint64)
    bits = (w1 << np.uint64(21)) ^ (w2 >> np.uint64(11))
    bits &= np.uint64((1 << 53) - 1)
    return (bits.astype(np.float64) + 0.5) / float(1 << 53)


def zipf_log_ranks(seed, tag, n: int, s: float) -> np.ndarray:
    """ln(k) of n iid Zipf(s) integers k on {1, 2, ...} (s > 1).

    Rejection-inversion (Hoermann & Derflinger, "Rejection-inversion to
    generate variates from monotone discrete distributions", 1996) for the
    unbounded support: H(x) = (x^(1-s) - 1)/(1-s) integrates the hat x^-s; a
    uniform y on [H(1.5) - 1, H(inf)) is inverted to x = H^-1(y), rounded to
    k, and accepted when y >= H(k + 1/2) - k^-s.  Zipf(1.1) has a very heavy
    tail (P(k > 1e15) is about 3%), so the draw is returned as ln k; beyond
    k ~ e^35 the hat and the mass agree to ~1e-30 and x itself is kept.
    """
    if s <= 1.0:
        raise ValueError("zipf exponent must exceed 1")
    one_m_s = 1.0 - s

    def H(x):
        return math.expm1(one_m_s * math.log(x)) / one_m_s

    h_lo = H(1.5) - 1.0          # H(1.5) - h(1)
    h_hi = -1.0 / one_m_s         # limit of H(x) as x -> inf
    out = np.empty(n, dtype=np.float64)
    u = uniform01_host(seed, tuple(tag) + ("u",), 64 * n)
    j = 0
    for i in range(n):
        while True:
            if j >= len(u):
                raise RuntimeError("zipf sampler ran out of uniforms")
            y = h_lo + u[j] * (h_hi - h_lo)
            j += 1
            lnx = math.log1p(one_m_s * y) / one_m_s
            if lnx > 35.0:
                out[i] = lnx
                break
            k = max(1, int(math.exp(lnx) + 0.5))
            if y >= H(k + 0.5) - k ** (-s):
                out[i] = math.log(k)
                break
    return out


# ---------------------------------------------------------------- storage
def to_bf16(t: torch.Tensor) -> torch.Tensor:
    return t.to(torch.bfloat16)  # round to nearest even on CPU and GPU alike


E4M3_MAX = 448.0


def quantize_e4m3_rows(w: torch.Tensor):
    """Per-row (= per output channel) fp8 e4m3fn quantisation.

    scale = max|row| / 448 (fp32, host division); code = RNE(w * (1/scale))
    after clamping to +-448.  Returns (codes float8_e4m3fn, scale float32 [rows]).
    """
    amax = w.abs().amax(dim=-1).cpu().numpy().astype(np.float32)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    recip = (np.float32(1.0) / scale).astype(np.float32)
    r = torch.from_numpy(recip).to(w.device)
    q = (w * r.unsqueeze(-1)).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, torch.from_numpy(scale).to(w.device)


def store(t: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return t
    if dtype == "bf16":
        return to_bf16(t)
    raise ValueError(dtype)


# ---------------------------------------------------------------- configs
@dataclasses.dataclass(frozen=True)
class MoEConfig:
    name: str
    S: int
    d: int
    d_ff: int
    E: int
    K: int
    act: str = "bf16"             # x, W_r, b1, b2, h, y: "f32" | "bf16"
    w: str = "bf16"               # W1, W2: "f32" | "bf16" | "fp8"
    n_groups: int = 1             # >1: group-limited selection
    topk_groups: int = 1
    renormalize: int = 1
    router_w: str = "normal"      # "normal": N(0,1/d); "uniform": U(+-sqrt(3/d))
    router_offset: str = "none"   # "none" | "normal" | "zipf" -> router_bias
    offset_beta: float = 0.0
    zipf_s: float = 1.1
    select_bias_var: float = 0.0  # >0: per-expert selection-only bias N(0, v)
    bias_var: float = 0.01        # b1, b2 ~ N(0, v)
    seed: int = 0

    @property
    def pairs(self) -> int:
        return self.S * self.K

    def replace(self, **kw) -> "MoEConfig":
        return dataclasses.replace(self, **kw)


# Offsets are scaled so that the realised max/mean expert load is about 3
# (Mixtral-shape prefill) and about 5 (Zipf skew).  The two beta values were
# found by bisection with tests/golden/calibrate_skew.py on seed 0.
BETA_MIXTRAL = 0.6201171875
BETA_ZIPF = 0.2841796875

CONFIGS: Dict[str, MoEConfig] = {
    "tiny_f32": MoEConfig("tiny_f32", S=64, d=128, d_ff=256, E=8, K=2, act="f32", w="f32"),
    "mixtral_prefill": MoEConfig("mixtral_prefill", S=4096, d=4096, d_ff=14336, E=8, K=2,
                                 router_offset="normal", offset_beta=BETA_MIXTRAL),
    "decode": MoEConfig("decode", S=16, d=4096, d_ff=14336, E=8, K=2, router_w="uniform"),
    "zipf_skew": MoEConfig("zipf_skew", S=8192, d=2048, d_ff=5632, E=64, K=4,
                           router_offset="zipf", offset_beta=BETA_ZIPF),
    "dsv3_fp8": MoEConfig("dsv3_fp8", S=4096, d=7168, d_ff=2048, E=256, K=8, w="fp8",
                          n_groups=8, topk_groups=2, select_bias_var=0.1),
}
CONFIG_ORDER = ["tiny_f32", "mixtral_prefill", "decode", "zipf_skew", "dsv3_fp8"]


# ---------------------------------------------------------------- tensors
def router_bias(cfg: MoEConfig) -> Optional[torch.Tensor]:
    """Per-expert router logit offset [E] float32 (host), or None."""
    if cfg.router_offset == "none":
        return None
    if cfg.router_offset == "normal":
        z = normal(cfg.seed, ("router_offset",), (cfg.E,), 1.0).double().numpy()
        return torch.from_numpy((cfg.offset_beta * z).astype(np.float32))
    if cfg.router_offset == "zipf":
        lnk = zipf_log_ranks(cfg.seed, ("router_offset",), cfg.E, cfg.zipf_s)
        return torch.from_numpy((-cfg.offset_beta * lnk).astype(np.float32))
    raise ValueError(cfg.router_offset)


def select_bias(cfg: MoEConfig) -> Optional[torch.Tensor]:
    if cfg.select_bias_var <= 0:
        return None
    return normal(cfg.seed, ("select_bias",), (cfg.E,), cfg.select_bias_var)


def tokens(cfg: MoEConfig, device="cpu", start: int = 0, count: Optional[int] = None) -> torch.Tensor:
    """x rows [start, start+count) as [count, d] in the activation dtype."""
    count = cfg.S - start if count is None else count
    x = normal(cfg.seed, ("x",), (count, cfg.d), 1.0, device, start=start * cfg.d)
    return store(x, cfg.act)


def router_weight(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    shape = (cfg.E, cfg.d)
    if cfg.router_w == "uniform":
        w = uniform(cfg.seed, ("W_r",), shape, math.sqrt(3.0 / cfg.d), device)
    else:
        w = normal(cfg.seed, ("W_r",), shape, 1.0 / cfg.d, device)
    return store(w, cfg.act)


def expert_weights(cfg: MoEConfig, e: int, device="cpu") -> Dict[str, torch.Tensor]:
    """One expert's W1 [d_ff,d], b1 [d_ff], W2 [d,d_ff], b2 [d] (+ fp8 scales)."""
    w1 = normal(cfg.seed, ("W1", e), (cfg.d_ff, cfg.d), 1.0 / cfg.d, device)
    w2 = normal(cfg.seed, ("W2", e), (cfg.d, cfg.d_ff), 1.0 / cfg.d_ff, device)
    out = {
        "b1": store(normal(cfg.seed, ("b1", e), (cfg.d_ff,), cfg.bias_var, device), cfg.act),
        "b2": store(normal(cfg.seed, ("b2", e), (cfg.d,), cfg.bias_var, device), cfg.act),
    }
    if cfg.w == "fp8":
        out["W1"], out["w1_scale"] = quantize_e4m3_rows(w1)
        out["W2"], out["w2_scale"] = quantize_e4m3_rows(w2)
    else:
        out["W1"], out["W2"] = store(w1, cfg.w), store(w2, cfg.w)
    return out


def make_inputs(cfg: MoEConfig, device="cpu", experts: Optional[Sequence[int]] = None):
    """All layer inputs as a dict of tensors on `device`.

    Expert tensors are stacked [E, ...]; when `experts` is given only those
    experts are generated and the others are left as zeros (for oracle
    checks that touch a few experts of a large layer).
    """
    E = cfg.E
    wdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}[cfg.w]
    adt = {"f32": torch.float32, "bf16": torch.bfloat16}[cfg.act]
    inp = {
        "x": tokens(cfg, device),
        "W_r": router_weight(cfg, device),
        "W1": torch.zeros((E, cfg.d_ff, cfg.d), dtype=wdt, device=device),
        "W2": torch.zeros((E, cfg.d, cfg.d_ff), dtype=wdt, device=device),
        "b1": torch.zeros((E, cfg.d_ff), dtype=adt, device=device),
        "b2": torch.zeros((E, cfg.d), dtype=adt, device=device),
        "w1_scale": None,
        "w2_scale": None,
    }
    if cfg.w == "fp8":
        inp["w1_scale"] = torch.zeros((E, cfg.d_ff), dtype=torch.float32, device=device)
        inp["w2_scale"] = torch.zeros((E, cfg.d), dtype=torch.float32, device=device)
    rb, sb = router_bias(cfg), select_bias(cfg)
    inp["router_bias"] = None if rb is None else rb.to(device)
    inp["select_bias"] = None if sb is None else sb.to(device)
    for e in (range(E) if experts is None else experts):
        w = expert_weights(cfg, e, device)
        for k, v in w.items():
            inp[k][e].copy_(v)
    return inp
