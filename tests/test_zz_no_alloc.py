"""moe_layer_forward_noalloc, the entry point for callers that cannot
allocate: through the C ABI, on the library's own scratch array, against
moe_layer_forward with a caller workspace on the same inputs.  Two calls in a
row on each problem, the second with fewer tokens, so the second runs on
whatever the first left in the array."""
import ctypes

import numpy as np
import pytest
import torch

import datagen as D
import sparse_ffn_layer_amd as M

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _outs(cfg, S):
    i32, f32 = dict(dtype=torch.int32, device=DEV), dict(dtype=torch.float32, device=DEV)
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    return dict(y=torch.full((S, cfg.d), 3.0, dtype=act, device=DEV),
                idx=torch.full((S, cfg.K), -7, **i32), gate=torch.full((S, cfg.K), -1.0, **f32),
                logits=torch.full((S, cfg.E), -1.0, **f32), counts=torch.full((cfg.E,), -1, **i32))


def _call(noalloc, p, inp, S, out):
    x = inp["x"][:S]
    args = [ctypes.byref(p)] + [M._ptr(t) for t in (x, inp["W_r"], inp["router_bias"], inp["select_bias"],
                                                     inp["W1"], inp["b1"], inp["W2"], inp["b2"], inp["w1_scale"],
                                                     inp["w2_scale"], out["y"], out["idx"], out["gate"],
                                                     out["logits"], out["counts"])]
    stream = torch.cuda.current_stream().cuda_stream or None
    if noalloc:
        return M.lib().moe_layer_forward_noalloc(*args, stream)
    ws = M.workspace(p, M.STAGE_LAYER, DEV)
    st = M.lib().moe_layer_forward(*args, M._ptr(ws), ws.numel(), stream)
    torch.cuda.synchronize()
    return st


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


CASES = [
    # Mixtral-shape decode: 16-row tiles, four-wave split router, single-block dispatch
    ("decode", dict(), (16, 5)),
    # DeepSeek-shape decode with fp8 weights, 8 groups, the MFMA router; then with fp8 activations
    ("dsv3_fp8", dict(), (16, 3)),
    ("dsv3_fp8", dict(act_quant=1), (16, 7)),
    # a capacity on a small layer (the capacity kernels use the array too)
    ("small_cap", dict(capacity=20), (200, 120)),
]


def _cfg(name):
    if name == "small_cap":
        return D.MoEConfig("small_cap", S=200, d=256, d_ff=512, E=16, K=2, router_offset="normal",
                           offset_beta=1.0, seed=3)
    return D.CONFIGS[name]


@pytest.mark.parametrize("name,kw,sizes", CASES)
def test_noalloc_matches_layer_forward(name, kw, sizes):
    cfg = _cfg(name)
    S0 = max(sizes)
    inp = D.make_inputs(cfg.replace(S=S0) if hasattr(cfg, "replace") else cfg, DEV)
    torch.cuda.synchronize()
    for S in sizes:
        print(f"noalloc {name} {kw} S={S}", flush=True)
        p = M.make_problem(S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                           cfg.renormalize, 1.0, kw.get("capacity", 0), kw.get("act_quant", 0))
        assert M.moe_workspace_bytes(p, M.STAGE_LAYER) <= M.MOE_NOALLOC_SCRATCH_BYTES
        a, b = _outs(cfg, S), _outs(cfg, S)
        assert _call(True, p, inp, S, a) == M.MOE_OK
        torch.cuda.synchronize()
        assert _call(False, p, inp, S, b) == M.MOE_OK
        for k in a:
            assert torch.equal(_bits(a[k]), _bits(b[k])), (name, S, k)
        assert int((a["counts"]).sum()) <= S * cfg.K


def test_noalloc_rejects_too_large_without_launching():
    cfg = D.CONFIGS["mixtral_prefill"]
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K)
    a = ctypes.c_void_p(1 << 20)
    st = M.lib().moe_layer_forward_noalloc(ctypes.byref(p), a, a, None, None, a, a, a, a, None, None, a,
                                           None, None, None, None, None)
    assert st == M.MOE_ERR_TOO_LARGE
