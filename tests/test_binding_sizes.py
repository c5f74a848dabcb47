"""The Python binding refuses tensors smaller than the arguments they stand
for, before any call into the library (which takes plain pointers and would
read or write past them).  CPU only: every case here raises before a launch."""
import pytest
import torch

import sparse_ffn_layer_amd as M

S, D, DFF, E, K = 40, 128, 256, 8, 2


def _p(**kw):
    return M.make_problem(S, D, DFF, E, K, "bf16", "bf16", **kw)


def _t(n, dtype=torch.bfloat16):
    return torch.zeros(n, dtype=dtype)


def test_route_refuses_short_outputs():
    p = _p()
    x, wr = _t(S * D), _t(E * D)
    with pytest.raises(ValueError, match="topk_idx"):
        M.moe_route(p, x, wr, topk_idx=_t(S * K - 1, torch.int32))
    with pytest.raises(ValueError, match="x holds"):
        M.moe_route(p, _t(S * D - 1), wr)
    with pytest.raises(ValueError, match="logits_out"):
        M.moe_route(p, x, wr, logits_out=_t(S * E - 1, torch.float32))


def test_permute_refuses_short_x_perm():
    p = _p()
    cap = M.moe_rows_capacity(p)
    idx = _t(S * K, torch.int32)
    with pytest.raises(ValueError, match="x_perm"):
        M.moe_permute(p, idx, _t(S * D), x_perm=_t((cap - 1) * D))
    with pytest.raises(ValueError, match="expert_offsets"):
        M.moe_permute(p, idx, _t(S * D), expert_offsets=_t(E, torch.int32))


def test_expert_products_refuse_short_buffers():
    p = _p()
    cap = M.moe_rows_capacity(p)
    c, o = _t(E, torch.int32), _t(E + 1, torch.int32)
    w1, b1 = _t(E * DFF * D), _t(E * DFF)
    with pytest.raises(ValueError, match="h holds"):
        M.moe_expert_up(p, _t(cap * D), c, o, w1, b1, h=_t(cap * DFF - 1))
    with pytest.raises(ValueError, match="W1"):
        M.moe_expert_up(p, _t(cap * D), c, o, _t(E * DFF * D - 1), b1)
    with pytest.raises(ValueError, match="y_perm"):
        M.moe_expert_down(p, _t(cap * DFF), c, o, _t(E * D * DFF), _t(E * D), y_perm=_t(cap * D - 8))
    p8 = M.make_problem(S, D, DFF, E, K, "bf16", "fp8", act_quant=1)
    cap8 = M.moe_rows_capacity(p8)
    with pytest.raises(ValueError, match="x8"):
        M.moe_expert_up_a8(p8, _t(cap8 * D - 1, torch.uint8), _t(cap8, torch.float32), c, o,
                           _t(E * DFF * D, torch.uint8), _t(E * DFF), _t(E * DFF, torch.float32))


def test_combine_and_layer_refuse_short_outputs():
    p = _p()
    cap = M.moe_rows_capacity(p)
    with pytest.raises(ValueError, match="y holds"):
        M.moe_combine(p, _t(cap * D), _t(S * K, torch.int32), _t(S * K, torch.float32), y=_t(S * D - 1))
    args = (p, _t(S * D), _t(E * D), _t(E * DFF * D), _t(E * DFF), _t(E * D * DFF), _t(E * D))
    with pytest.raises(ValueError, match="expert_counts_out"):
        M.moe_layer_forward(*args, expert_counts_out=_t(E - 1, torch.int32))
    with pytest.raises(ValueError, match="y holds"):
        M.moe_layer_forward_noalloc(*args, y=_t(S * D - 1))


def test_quantize_rows_refuses_short_codes():
    src = _t(12 * 64).view(12, 64)
    with pytest.raises(ValueError, match="moe_quantize_rows"):
        M.moe_quantize_rows(src, codes=torch.zeros(11 * 64, dtype=torch.uint8))
    with pytest.raises(ValueError, match="moe_quantize_rows"):
        M.moe_quantize_rows(src, scales=torch.zeros(11, dtype=torch.float32))
