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


def split_tail_tiles(offsets, rows_cap, N, K, BM, BN, BK, GM, grid=256):
    """Tiles whose k range the grouped GEMM splits: the host-side replica of
    its persistent schedule.  The tile space (row tiles in use x N / BN
    channel tiles, in bands of row tiles, the row tile fastest: GM > 0 bands
    of GM consecutive row tiles, GM < 0 bands of at most -GM row tiles
    starting at each expert's first row tile) is cut into 8 contiguous
    slices, one per XCD; each slice runs in rounds of its
    grid / 8 workgroups, and when its last round is partial with at least
    twice as many idle workgroups as tail tiles and K / BK >= 16 k-tiles,
    the tail tiles run split along k.  `grid` is the launch's workgroup
    count (256: one workgroup per compute unit of an MI355X for the 128-row
    tiles).  Returns [(row0, n0, expert)] of the split tiles."""
    offsets = np.asarray(offsets, dtype=np.int64)
    E = len(offsets) - 1
    m_tiles = -(-rows_cap // BM)
    m_used = min(-(-int(offsets[E]) // BM), m_tiles)
    n_tiles = N // BN
    T = m_used * n_tiles
    g = min(grid, m_tiles * n_tiles)
    g = 8 if g < 8 else g // 8 * 8
    if K // BK < 16:
        return []
    out = []
    for xcd in range(8):
        nx = (g - xcd + 7) >> 3
        t_lo, t_hi = T * xcd // 8, T * (xcd + 1) // 8
        tx = t_hi - t_lo
        full_end = t_lo + tx // nx * nx
        tail = tx % nx
        split = nx // tail if tail else 0
        if split < 2:
            continue
        for tau in range(tail):
            L = full_end + tau
            if GM > 0:
                band = GM * n_tiles
                bnd = L // band
                first_m = bnd * GM
                gm = min(m_used - first_m, GM)
                rem = L - bnd * band
                mt, nt = first_m + rem % gm, rem // gm
            else:
                r = L // n_tiles
                e = int(np.searchsorted(offsets, r * BM, side="right") - 1)
                first, rt = int(offsets[e]) // BM, int(offsets[e + 1] - offsets[e]) // BM
                bi = (r - first) // -GM
                bfirst = first + bi * -GM
                gm = min(-GM, rt - bi * -GM)
                local = L - bfirst * n_tiles
                mt, nt = bfirst + local % gm, local // gm
            row0 = mt * BM
            if row0 >= offsets[E]:
                continue
            e = int(np.searchsorted(offsets, row0, side="right") - 1)
            out.append((row0, nt * BN, e))
    return out


def host_x_perm(cfg, xr, pm, cap):
    """x_perm built on the host from the oracle's permutation (padding rows 0)."""
    xp = np.zeros((cap, cfg.d), dtype=xr.dtype)
    xp[pm["inv_perm"]] = xr[np.arange(cfg.S * cfg.K) // cfg.K]
    return xp
