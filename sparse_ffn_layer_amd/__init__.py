"""Python binding of the MoE-layer C ABI (include/moe.h) for MI355X.

Argument marshalling only: every step of the layer runs in the HIP kernels
of libsfl_moe.so.  torch provides device memory and the current stream.
There is no CPU or pure-PyTorch fallback: if the library is missing, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MOE_OK", "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP",
    "MOE_F32", "MOE_BF16", "MOE_FP8_E4M3", "STAGE_ROUTE", "STAGE_PERMUTE", "STAGE_EXPERT_FFN",
    "STAGE_COMBINE", "STAGE_LAYER", "MoEError", "moe_problem", "make_problem", "lib", "LIB_PATH",
    "moe_workspace_bytes", "moe_tile_m", "moe_rows_capacity", "moe_status_string",
    "workspace", "moe_load_stats", "moe_apply_capacity", "moe_quantize_rows", "STAGE_CAPACITY", "MOE_STATS_N", "STAT_NAMES", "moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_up", "moe_expert_down", "moe_combine", "moe_layer_forward",
    "moe_layer_forward_noalloc", "MOE_ERR_TOO_LARGE", "MOE_NOALLOC_SCRATCH_BYTES",
    "moe_expert_up_a8", "moe_expert_down_a8",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsfl_moe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_ERR_TOO_LARGE = -5
MOE_NOALLOC_SCRATCH_BYTES = 128 << 20   # the library's own scratch array per GPU (moe.h)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
STAGE_ROUTE, STAGE_PERMUTE, STAGE_EXPERT_FFN, STAGE_COMBINE, STAGE_LAYER, STAGE_CAPACITY = 0, 1, 2, 3, 4, 5
# moe_load_stats outputs, in order (MOE_STAT_* in include/moe.h)
STAT_NAMES = ("mean", "std", "max_over_mean", "drop_rate", "aux_loss", "max", "min", "empty")
MOE_STATS_N = len(STAT_NAMES)

_DT = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3,
       torch.float32: MOE_F32, torch.bfloat16: MOE_BF16, torch.float8_e4m3fn: MOE_FP8_E4M3}
_ACT_TORCH = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status} ({moe_status_string(status)})")
        self.status = status


class moe_problem(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int64), ("d", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("renormalize", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("w_dtype", ctypes.c_int32),
                ("gate_temperature", ctypes.c_float), ("capacity", ctypes.c_int32),
                ("act_quant", ctypes.c_int32)]


def make_problem(S, d, d_ff, E, K, act="bf16", w="bf16", n_groups=1, topk_groups=1,
                 renormalize=1, temperature=1.0, capacity=0, act_quant=0) -> moe_problem:
    return moe_problem(int(S), int(d), int(d_ff), int(E), int(K), int(n_groups), int(topk_groups),
                       int(renormalize), _DT[act], _DT[w], float(temperature), int(capacity), int(act_quant))


_lib = None
_P = ctypes.POINTER(moe_problem)
_vp, _sz, _i32, _i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64

_SIGS = {
    "moe_workspace_bytes": (_sz, [_P, _i32]),
    "moe_tile_m": (_i32, [_P]),
    "moe_rows_capacity": (_i64, [_P]),
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_route": (_i32, [_P] + [_vp] * 8 + [_vp, _sz, _vp]),
    "moe_permute": (_i32, [_P] + [_vp] * 7 + [_vp, _sz, _vp]),
    "moe_expert_ffn": (_i32, [_P] + [_vp] * 11 + [_vp, _sz, _vp]),
    "moe_expert_up": (_i32, [_P] + [_vp] * 7 + [_vp, _sz, _vp]),
    "moe_expert_down": (_i32, [_P] + [_vp] * 7 + [_vp, _sz, _vp]),
    "moe_expert_up_a8": (_i32, [_P] + [_vp] * 8 + [_vp, _sz, _vp]),
    "moe_expert_down_a8": (_i32, [_P] + [_vp] * 8 + [_vp, _sz, _vp]),
    "moe_combine": (_i32, [_P] + [_vp] * 4 + [_vp]),
    "moe_layer_forward": (_i32, [_P] + [_vp] * 15 + [_vp, _sz, _vp]),
    "moe_layer_forward_noalloc": (_i32, [_P] + [_vp] * 15 + [_vp]),
    "moe_load_stats": (_i32, [_P, _vp, _vp, _vp, ctypes.c_float, _vp, _vp]),
    "moe_apply_capacity": (_i32, [_P] + [_vp] * 5 + [_vp, _sz, _vp]),
    "moe_quantize_rows": (_i32, [_vp, _i64, _i32, _vp, _vp, _vp]),
}


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m sparse_ffn_layer_amd.build` (hipcc, gfx950)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


# ------------------------------------------------------------------ helpers
def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return t.data_ptr() or None


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream or None
    return getattr(stream, "cuda_stream", stream) or None


def _side(stream):
    """The launch stream as a torch stream when it is not the current one, else None.

    Tensors a wrapper allocates come from torch's caching allocator on the
    current stream.  When the kernels run on another stream, such a tensor is
    marked as in use there (record_stream), so that freeing it when the
    wrapper returns cannot hand its bytes to a later allocation on the current
    stream while the launched kernels still read or write them."""
    if stream is None:
        return None
    cur = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return None if stream.cuda_stream == cur.cuda_stream else stream
    h = int(getattr(stream, "cuda_stream", stream) or 0)
    if h == cur.cuda_stream:
        return None
    return torch.cuda.ExternalStream(h) if h else torch.cuda.default_stream()


def _empty(shape, dtype, device, side):
    t = torch.empty(shape, dtype=dtype, device=device)
    if side is not None:
        t.record_stream(side)
    return t


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoEError(fn, status)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_workspace_bytes(p: moe_problem, stage: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(p), int(stage)))


def moe_tile_m(p: moe_problem) -> int:
    return int(lib().moe_tile_m(ctypes.byref(p)))


def moe_rows_capacity(p: moe_problem) -> int:
    return int(lib().moe_rows_capacity(ctypes.byref(p)))


def workspace(p: moe_problem, stage: int, device="cuda", side=None) -> torch.Tensor:
    """Workspace of entry point `stage` for p; `side`: the stream the kernels
    run on when it is not the current one (the tensor is then marked as in
    use there)."""
    n = moe_workspace_bytes(p, stage)
    return _empty(max(n, 1), torch.uint8, device, side)


def _act(p: moe_problem):
    return _ACT_TORCH[p.act_dtype]


_ESZ = {MOE_F32: 4, MOE_BF16: 2, MOE_FP8_E4M3: 1}


def _need_bytes(p: moe_problem, name: str) -> int:
    """Bytes the argument `name` of an entry point spans for problem p (the
    shapes include/moe.h states)."""
    S, d, d_ff, E, K = int(p.S), int(p.d), int(p.d_ff), int(p.E), int(p.K)
    a, w = _ESZ[p.act_dtype], _ESZ[p.w_dtype]
    rows = moe_rows_capacity(p) if name in ("x_perm", "h", "y_perm", "x8", "x_scale", "h8", "h_scale") else 0
    return {
        "x": S * d * a, "W_r": E * d * a, "router_bias": E * 4, "select_bias": E * 4,
        "logits_in": S * E * 4, "logits_out": S * E * 4, "logits": S * E * 4,
        "topk_idx": S * K * 4, "topk_gate": S * K * 4, "topk_idx_out": S * K * 4, "topk_gate_out": S * K * 4,
        "perm": S * K * 4, "inv_perm": S * K * 4,
        "expert_counts": E * 4, "expert_counts_out": E * 4, "expert_offsets": (E + 1) * 4,
        "x_perm": rows * d * a, "h": rows * d_ff * a, "y_perm": rows * d * a,
        "x8": rows * d, "x_scale": rows * 4, "h8": rows * d_ff, "h_scale": rows * 4,
        "W1": E * d_ff * d * w, "W2": E * d * d_ff * w, "b1": E * d_ff * a, "b2": E * d * a,
        "w1_scale": E * d_ff * 4, "w2_scale": E * d * 4, "y": S * d * a,
        "stats": MOE_STATS_N * 4, "dropped": 4,
    }[name]


def _check_sizes(fn: str, p: moe_problem, **tensors) -> None:
    """The library takes plain pointers: a tensor smaller than its argument's
    extent would be read or written past its end.  Raise instead."""
    for name, t in tensors.items():
        if t is None:
            continue
        have, need = t.numel() * t.element_size(), _need_bytes(p, name)
        if have < need:
            raise ValueError(f"{fn}: {name} holds {have} bytes, the problem needs {need}")


# ------------------------------------------------------------------ entry points
def moe_route(p, x, W_r, router_bias=None, select_bias=None, logits_in=None, logits_out=None,
              topk_idx=None, topk_gate=None, ws=None, stream=None):
    dev = (logits_in if logits_in is not None else x).device
    side = _side(stream)
    if topk_idx is None:
        topk_idx = _empty((p.S, p.K), torch.int32, dev, side)
    if topk_gate is None:
        topk_gate = _empty((p.S, p.K), torch.float32, dev, side)
    if ws is None:
        ws = workspace(p, STAGE_ROUTE, dev, side)
    _check_sizes("moe_route", p, x=None if logits_in is not None else x,
                 W_r=None if logits_in is not None else W_r, router_bias=router_bias, select_bias=select_bias,
                 logits_in=logits_in, logits_out=logits_out, topk_idx=topk_idx, topk_gate=topk_gate)
    st = lib().moe_route(ctypes.byref(p), _ptr(x), _ptr(W_r), _ptr(router_bias), _ptr(select_bias),
                         _ptr(logits_in), _ptr(logits_out), _ptr(topk_idx), _ptr(topk_gate),
                         _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_route", st)
    return topk_idx, topk_gate


def moe_permute(p, topk_idx, x, expert_counts=None, expert_offsets=None, perm=None, inv_perm=None,
                x_perm=None, ws=None, stream=None):
    dev = topk_idx.device
    side = _side(stream)
    pairs = p.S * p.K
    expert_counts = _empty(p.E, torch.int32, dev, side) if expert_counts is None else expert_counts
    expert_offsets = _empty(p.E + 1, torch.int32, dev, side) if expert_offsets is None else expert_offsets
    perm = _empty(pairs, torch.int32, dev, side) if perm is None else perm
    inv_perm = _empty(pairs, torch.int32, dev, side) if inv_perm is None else inv_perm
    if x_perm is None:
        x_perm = _empty((moe_rows_capacity(p), p.d), _act(p), dev, side)
    if ws is None:
        ws = workspace(p, STAGE_PERMUTE, dev, side)
    _check_sizes("moe_permute", p, topk_idx=topk_idx, x=x, expert_counts=expert_counts,
                 expert_offsets=expert_offsets, perm=perm, inv_perm=inv_perm, x_perm=x_perm)
    st = lib().moe_permute(ctypes.byref(p), _ptr(topk_idx), _ptr(x), _ptr(expert_counts),
                           _ptr(expert_offsets), _ptr(perm), _ptr(inv_perm), _ptr(x_perm),
                           _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_permute", st)
    return expert_counts, expert_offsets, perm, inv_perm, x_perm


def moe_expert_ffn(p, x_perm, expert_counts, expert_offsets, W1, b1, W2, b2, w1_scale=None,
                   w2_scale=None, h=None, y_perm=None, ws=None, stream=None):
    dev = x_perm.device
    side = _side(stream)
    cap = moe_rows_capacity(p)
    h = _empty((cap, p.d_ff), _act(p), dev, side) if h is None else h
    y_perm = _empty((cap, p.d), _act(p), dev, side) if y_perm is None else y_perm
    if ws is None:
        ws = workspace(p, STAGE_EXPERT_FFN, dev, side)
    _check_sizes("moe_expert_ffn", p, x_perm=x_perm, expert_counts=expert_counts, expert_offsets=expert_offsets,
                 W1=W1, b1=b1, W2=W2, b2=b2, w1_scale=w1_scale, w2_scale=w2_scale, h=h, y_perm=y_perm)
    st = lib().moe_expert_ffn(ctypes.byref(p), _ptr(x_perm), _ptr(expert_counts), _ptr(expert_offsets),
                              _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2), _ptr(w1_scale), _ptr(w2_scale),
                              _ptr(h), _ptr(y_perm), _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_expert_ffn", st)
    return h, y_perm


def moe_expert_up(p, x_perm, expert_counts, expert_offsets, W1, b1, w1_scale=None, h=None, ws=None,
                  stream=None):
    side = _side(stream)
    if h is None:
        h = _empty((moe_rows_capacity(p), p.d_ff), _act(p), x_perm.device, side)
    if ws is None:
        ws = workspace(p, STAGE_EXPERT_FFN, x_perm.device, side)
    _check_sizes("moe_expert_up", p, x_perm=x_perm, expert_counts=expert_counts, expert_offsets=expert_offsets,
                 W1=W1, b1=b1, w1_scale=w1_scale, h=h)
    st = lib().moe_expert_up(ctypes.byref(p), _ptr(x_perm), _ptr(expert_counts), _ptr(expert_offsets),
                             _ptr(W1), _ptr(b1), _ptr(w1_scale), _ptr(h), _ptr(ws), ws.numel(),
                             _stream(stream))
    _check("moe_expert_up", st)
    return h


def moe_expert_down(p, h, expert_counts, expert_offsets, W2, b2, w2_scale=None, y_perm=None, ws=None,
                    stream=None):
    side = _side(stream)
    if y_perm is None:
        y_perm = _empty((moe_rows_capacity(p), p.d), _act(p), h.device, side)
    if ws is None:
        ws = workspace(p, STAGE_EXPERT_FFN, h.device, side)
    _check_sizes("moe_expert_down", p, h=h, expert_counts=expert_counts, expert_offsets=expert_offsets,
                 W2=W2, b2=b2, w2_scale=w2_scale, y_perm=y_perm)
    st = lib().moe_expert_down(ctypes.byref(p), _ptr(h), _ptr(expert_counts), _ptr(expert_offsets),
                               _ptr(W2), _ptr(b2), _ptr(w2_scale), _ptr(y_perm), _ptr(ws), ws.numel(),
                               _stream(stream))
    _check("moe_expert_down", st)
    return y_perm


def moe_expert_up_a8(p, x8, x_scale, expert_counts, expert_offsets, W1, b1, w1_scale, h=None, ws=None,
                     stream=None):
    """W8A8 up product (p.act_quant = 1): e4m3 rows x8 with row scales -> bf16 h."""
    side = _side(stream)
    if h is None:
        h = _empty((moe_rows_capacity(p), p.d_ff), torch.bfloat16, x8.device, side)
    if ws is None:
        ws = workspace(p, STAGE_EXPERT_FFN, x8.device, side)
    _check_sizes("moe_expert_up_a8", p, x8=x8, x_scale=x_scale, expert_counts=expert_counts,
                 expert_offsets=expert_offsets, W1=W1, b1=b1, w1_scale=w1_scale, h=h)
    st = lib().moe_expert_up_a8(ctypes.byref(p), _ptr(x8), _ptr(x_scale), _ptr(expert_counts),
                                _ptr(expert_offsets), _ptr(W1), _ptr(b1), _ptr(w1_scale), _ptr(h), _ptr(ws),
                                ws.numel(), _stream(stream))
    _check("moe_expert_up_a8", st)
    return h


def moe_expert_down_a8(p, h8, h_scale, expert_counts, expert_offsets, W2, b2, w2_scale, y_perm=None, ws=None,
                       stream=None):
    """W8A8 down product (p.act_quant = 1): e4m3 rows h8 with row scales -> bf16 y_perm."""
    side = _side(stream)
    if y_perm is None:
        y_perm = _empty((moe_rows_capacity(p), p.d), torch.bfloat16, h8.device, side)
    if ws is None:
        ws = workspace(p, STAGE_EXPERT_FFN, h8.device, side)
    _check_sizes("moe_expert_down_a8", p, h8=h8, h_scale=h_scale, expert_counts=expert_counts,
                 expert_offsets=expert_offsets, W2=W2, b2=b2, w2_scale=w2_scale, y_perm=y_perm)
    st = lib().moe_expert_down_a8(ctypes.byref(p), _ptr(h8), _ptr(h_scale), _ptr(expert_counts),
                                  _ptr(expert_offsets), _ptr(W2), _ptr(b2), _ptr(w2_scale), _ptr(y_perm),
                                  _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_expert_down_a8", st)
    return y_perm


def moe_combine(p, y_perm, inv_perm, topk_gate, y=None, stream=None):
    if y is None:
        y = _empty((p.S, p.d), _act(p), y_perm.device, _side(stream))
    _check_sizes("moe_combine", p, y_perm=y_perm, inv_perm=inv_perm, topk_gate=topk_gate, y=y)
    st = lib().moe_combine(ctypes.byref(p), _ptr(y_perm), _ptr(inv_perm), _ptr(topk_gate), _ptr(y),
                           _stream(stream))
    _check("moe_combine", st)
    return y


def moe_layer_forward(p, x, W_r, W1, b1, W2, b2, router_bias=None, select_bias=None, w1_scale=None,
                      w2_scale=None, y=None, topk_idx_out=None, topk_gate_out=None, logits_out=None,
                      expert_counts_out=None, ws=None, stream=None):
    side = _side(stream)
    if y is None:
        y = _empty((p.S, p.d), _act(p), x.device, side)
    if ws is None:
        ws = workspace(p, STAGE_LAYER, x.device, side)
    _check_sizes("moe_layer_forward", p, x=x, W_r=W_r, router_bias=router_bias, select_bias=select_bias, W1=W1,
                 b1=b1, W2=W2, b2=b2, w1_scale=w1_scale, w2_scale=w2_scale, y=y, topk_idx_out=topk_idx_out,
                 topk_gate_out=topk_gate_out, logits_out=logits_out, expert_counts_out=expert_counts_out)
    st = lib().moe_layer_forward(ctypes.byref(p), _ptr(x), _ptr(W_r), _ptr(router_bias),
                                 _ptr(select_bias), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                 _ptr(w1_scale), _ptr(w2_scale), _ptr(y), _ptr(topk_idx_out),
                                 _ptr(topk_gate_out), _ptr(logits_out), _ptr(expert_counts_out),
                                 _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_layer_forward", st)
    return y


def moe_layer_forward_noalloc(p, x, W_r, W1, b1, W2, b2, y, router_bias=None, select_bias=None,
                              w1_scale=None, w2_scale=None, topk_idx_out=None, topk_gate_out=None,
                              logits_out=None, expert_counts_out=None, stream=None):
    """moe_layer_forward on the library's own scratch array: the caller passes
    every input and output (y included) and nothing is allocated."""
    _check_sizes("moe_layer_forward_noalloc", p, x=x, W_r=W_r, router_bias=router_bias, select_bias=select_bias,
                 W1=W1, b1=b1, W2=W2, b2=b2, w1_scale=w1_scale, w2_scale=w2_scale, y=y, topk_idx_out=topk_idx_out,
                 topk_gate_out=topk_gate_out, logits_out=logits_out, expert_counts_out=expert_counts_out)
    st = lib().moe_layer_forward_noalloc(ctypes.byref(p), _ptr(x), _ptr(W_r), _ptr(router_bias),
                                         _ptr(select_bias), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                                         _ptr(w1_scale), _ptr(w2_scale), _ptr(y), _ptr(topk_idx_out),
                                         _ptr(topk_gate_out), _ptr(logits_out), _ptr(expert_counts_out),
                                         _stream(stream))
    _check("moe_layer_forward_noalloc", st)
    return y


def moe_load_stats(p, expert_counts, logits=None, dropped=None, alpha=1.0, stats=None, stream=None):
    """Load statistics of one routing as a float32 tensor [MOE_STATS_N] on the
    device, in the order of STAT_NAMES (see moe_load_stats in include/moe.h)."""
    if stats is None:
        # every entry is written by the kernel: no fill on the current stream
        # that could race with a launch on another one
        stats = _empty(MOE_STATS_N, torch.float32, expert_counts.device, _side(stream))
    _check_sizes("moe_load_stats", p, expert_counts=expert_counts, logits=logits, dropped=dropped, stats=stats)
    st = lib().moe_load_stats(ctypes.byref(p), _ptr(expert_counts), _ptr(logits), _ptr(dropped),
                              float(alpha), _ptr(stats), _stream(stream))
    _check("moe_load_stats", st)
    return stats


def moe_apply_capacity(p, logits, topk_idx, select_bias=None, topk_gate=None, dropped=None, ws=None,
                       stream=None):
    """Capacity-limited dispatch with p.capacity pairs per expert; topk_idx
    is updated in place.  Returns (topk_idx, topk_gate, dropped[1])."""
    side = _side(stream)
    if topk_gate is None:
        topk_gate = _empty((p.S, p.K), torch.float32, topk_idx.device, side)
    if dropped is None:
        dropped = _empty(4, torch.int32, topk_idx.device, side)  # entry 0 is written by the kernel
    if ws is None:
        ws = workspace(p, STAGE_CAPACITY, topk_idx.device, side)
    _check_sizes("moe_apply_capacity", p, logits=logits, select_bias=select_bias, topk_idx=topk_idx,
                 topk_gate=topk_gate, dropped=dropped)
    st = lib().moe_apply_capacity(ctypes.byref(p), _ptr(logits), _ptr(select_bias), _ptr(topk_idx),
                                  _ptr(topk_gate), _ptr(dropped), _ptr(ws), ws.numel(), _stream(stream))
    _check("moe_apply_capacity", st)
    return topk_idx, topk_gate, dropped[:1]


def moe_quantize_rows(src, codes=None, scales=None, stream=None):
    """Per-row e4m3 quantisation of a bf16 matrix [rows, n]: returns (codes
    uint8 [rows, n], scales float32 [rows])."""
    rows, n = src.shape
    side = _side(stream)
    if codes is None:
        codes = _empty((rows, n), torch.uint8, src.device, side)
    if scales is None:
        scales = _empty(max(rows, 1), torch.float32, src.device, side)
    if codes.numel() * codes.element_size() < rows * n or scales.numel() * scales.element_size() < rows * 4:
        raise ValueError(f"moe_quantize_rows: codes need {rows * n} bytes and scales {rows * 4} for {rows} rows")
    st = lib().moe_quantize_rows(_ptr(src), int(rows), int(n), _ptr(codes), _ptr(scales), _stream(stream))
    _check("moe_quantize_rows", st)
    return codes, scales[:rows]
