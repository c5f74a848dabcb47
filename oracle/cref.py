"""ctypes binding of the plain C++ reference loops (oracle/moe_oracle_ref.cpp).

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg use this module.  __graft_entry__.build() compiles the
library (g++, OpenMP) next to its source.  Inputs and outputs are numpy
arrays in host memory.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_ref.so")
SOURCE = os.path.join(HERE, "moe_oracle_ref.cpp")

_lib = None
_d, _f, _i32, _u8, _u16 = (np.ctypeslib.ndpointer(dtype=t, flags="C_CONTIGUOUS")
                           for t in (np.float64, np.float32, np.int32, np.uint8, np.uint16))
_i64, _c32 = ctypes.c_int64, ctypes.c_int32


class _Opt:
    """A nullable contiguous array argument."""

    def __init__(self, dtype):
        self.dtype = dtype

    def from_param(self, v):
        if v is None:
            return None
        a = np.ascontiguousarray(v, dtype=self.dtype)
        return a.ctypes.data_as(ctypes.c_void_p)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.oracle_decode_bf16.argtypes = [_u16, _i64, _d]
        L.oracle_decode_e4m3.argtypes = [_u8, _i64, _d]
        L.oracle_router_logits.argtypes = [_d, _d, _Opt(np.float32), _i64, _c32, _c32, _f]
        L.oracle_route.argtypes = [_f, _Opt(np.float32), _i64, _c32, _c32, _c32, _c32, _c32, ctypes.c_double,
                                   _i32, _d]
        L.oracle_route.restype = _c32
        L.oracle_permute.argtypes = [_i32, _i64, _c32, _c32, _c32, _i32, _i32, _i32, _i32]
        L.oracle_dense_ffn.argtypes = [_d, _i64, _c32, _c32, _d, _d, _d, _d, _d]
        L.oracle_layer_forward.argtypes = [_d, _d, _Opt(np.float32), _Opt(np.float32), _d, _d, _d, _d, _i64, _c32,
                                           _c32, _c32, _c32, _c32, _c32, _c32, ctypes.c_double,
                                           _Opt(np.float32), _d, _i32, _d]
        L.oracle_layer_forward.restype = _c32
        L.oracle_set_threads.argtypes = [_c32]
        L.oracle_threads.restype = _c32
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Threads of the OpenMP loops (the library's default: OMP_NUM_THREADS or
    every hardware thread)."""
    lib().oracle_set_threads(int(n))


def threads() -> int:
    return int(lib().oracle_threads())


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array ('f32' values, 'bf16' uint16 patterns, 'fp8' uint8
    e4m3fn codes) -> float64, by the C++ decoders."""
    a = np.ascontiguousarray(arr)
    out = np.empty(a.shape, dtype=np.float64)
    if dtype == "f32":
        out[...] = a.astype(np.float32)
    elif dtype == "bf16":
        lib().oracle_decode_bf16(a.astype(np.uint16).reshape(-1), a.size, out.reshape(-1))
    elif dtype == "fp8":
        lib().oracle_decode_e4m3(a.astype(np.uint8).reshape(-1), a.size, out.reshape(-1))
    else:
        raise ValueError(dtype)
    return out


def router_logits(x: np.ndarray, w_r: np.ndarray, router_bias: Optional[np.ndarray] = None) -> np.ndarray:
    x, w_r = np.ascontiguousarray(x, np.float64), np.ascontiguousarray(w_r, np.float64)
    S, d = x.shape
    E = w_r.shape[0]
    out = np.empty((S, E), np.float32)
    lib().oracle_router_logits(x, w_r, router_bias, S, d, E, out)
    return out


def route(logits: np.ndarray, K: int, select_bias=None, n_groups: int = 1, topk_groups: int = 1,
          renormalize: int = 1, temperature: float = 1.0):
    lg = np.ascontiguousarray(logits, np.float32)
    S, E = lg.shape
    idx = np.empty((S, K), np.int32)
    gate = np.empty((S, K), np.float64)
    if lib().oracle_route(lg, select_bias, S, E, K, n_groups, topk_groups, renormalize, temperature, idx, gate):
        raise ValueError("invalid routing configuration")
    return idx, gate


def permute(idx: np.ndarray, E: int, tile_m: int):
    idx = np.ascontiguousarray(idx, np.int32)
    S, K = idx.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm = np.empty(S * K, np.int32)
    inv = np.empty(S * K, np.int32)
    lib().oracle_permute(idx, S, K, E, tile_m, counts, offsets, perm, inv)
    return counts, offsets, perm[:int(((idx >= 0) & (idx < E)).sum())], inv


def dense_ffn(x, w1, b1, w2, b2) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float64)
    n, d = x.shape
    d_ff = w1.shape[0]
    out = np.empty((n, d), np.float64)
    lib().oracle_dense_ffn(x, n, d, d_ff, np.ascontiguousarray(w1, np.float64), np.ascontiguousarray(b1, np.float64),
                           np.ascontiguousarray(w2, np.float64), np.ascontiguousarray(b2, np.float64), out)
    return out


def layer_forward(x, w_r, W1, b1, W2, b2, *, K: int, router_bias=None, select_bias=None, n_groups: int = 1,
                  topk_groups: int = 1, renormalize: int = 1, temperature: float = 1.0, logits_in=None):
    """The whole layer on decoded float64 inputs (fp8 weights already times
    their channel scales).  Returns (y [S,d], idx [S,K], gates [S,K])."""
    x = np.ascontiguousarray(x, np.float64)
    S, d = x.shape
    E, d_ff = W1.shape[0], W1.shape[1]
    y = np.empty((S, d), np.float64)
    idx = np.empty((S, K), np.int32)
    gate = np.empty((S, K), np.float64)
    c = lambda a: np.ascontiguousarray(a, np.float64)
    st = lib().oracle_layer_forward(x, c(w_r), router_bias, select_bias, c(W1), c(b1), c(W2), c(b2), S, d, d_ff, E,
                                    K, n_groups, topk_groups, renormalize, temperature, logits_in, y, idx, gate)
    if st:
        raise ValueError("invalid routing configuration")
    return y, idx, gate
