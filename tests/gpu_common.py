"""Shared helpers of the GPU parity tests (inputs, oracle marshalling)."""
import functools

import numpy as np
import torch

import datagen as D
import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw

DEV = "cuda"
TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}   # max|dy| <= tol * max|y_ref|
GATE_TOL = 1e-6


def tol_of(cfg):
    return TOL["fp8"] if cfg.w == "fp8" else TOL[cfg.act]


def problem(cfg, S=None):
    return M.make_problem(cfg.S if S is None else S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w,
                          cfg.n_groups, cfg.topk_groups, cfg.renormalize)


@functools.lru_cache(maxsize=None)
def gpu_inputs(name):
    cfg = D.CONFIGS[name]
    inp = D.make_inputs(cfg, device=DEV)
    torch.cuda.synchronize()
    return inp


class LazyExperts:
    """Indexable by expert; copies that expert's tensor to the host on demand."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return raw(self.t[int(e)])


def oracle_view(inp):
    """Oracle arguments from device tensors; expert tensors copied lazily."""
    out = {}
    for k in ("x", "W_r", "router_bias", "select_bias", "b1", "b2", "w1_scale", "w2_scale"):
        out[k] = raw(inp[k])
    out["W1"] = LazyExperts(inp["W1"])
    out["W2"] = LazyExperts(inp["W2"])
    return out


def oracle_logits(cfg, ov, tokens=None):
    x = ov["x"] if tokens is None else ov["x"][tokens]
    return O.router_logits(O.decode(x, cfg.act), O.decode(ov["W_r"], cfg.act), ov["router_bias"])


def oracle_select(cfg, logits, ov):
    idx = O.select_experts(logits, cfg.K, ov["select_bias"], cfg.n_groups, cfg.topk_groups)
    return idx, O.gate_weights(logits, idx, cfg.renormalize)


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype) if t.dtype.itemsize == torch.empty((), dtype=dtype).element_size() else t.to(dtype)
    return t.to(DEV)


def act_from_raw(a, act):
    """Oracle storage array (float32 or uint16 bf16 bits) -> device tensor."""
    if act == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def sample_tokens(S, n, seed=0):
    if n >= S:
        return np.arange(S)
    rng = np.random.default_rng(seed)
    base = np.linspace(0, S - 1, n // 2).astype(np.int64)
    extra = rng.choice(S, n - len(base), replace=False)
    return np.unique(np.concatenate([base, extra, [S - 1]]))


def near_tie(keys_row, K, gap):
    """True if the K-th and (K+1)-th largest keys are within `gap`."""
    s = np.sort(np.asarray(keys_row, dtype=np.float64))[::-1]
    return K < len(s) and (s[K - 1] - s[K]) <= gap
