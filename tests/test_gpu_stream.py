"""Launch streams other than the current one.

The Python wrappers allocate their workspace and any output the caller
leaves out from torch's caching allocator, which hands memory out per
stream.  When the kernels run on another stream, such a tensor must stay
reserved for that stream until its work is done; otherwise a later
allocation on the current stream could take the same bytes while the
kernels still use them."""
import numpy as np
import pytest
import torch

import datagen as D
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, problem

pytestmark = pytest.mark.gpu


def _busy(stream, n=40):
    """Queue several milliseconds of work on `stream`."""
    a = torch.randn((4096, 4096), device=DEV, dtype=torch.bfloat16)
    with torch.cuda.stream(stream):
        for _ in range(n):
            a = (a @ a) * (1.0 / 64)
    return a


def test_side_stream_workspace_not_reused_while_in_flight():
    cfg = D.MoEConfig("side", S=512, d=512, d_ff=768, E=8, K=2, router_offset="normal", offset_beta=0.3)
    inp = D.make_inputs(cfg, DEV)
    p = problem(cfg)
    args = (p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], inp["router_bias"],
            inp["select_bias"], inp["w1_scale"], inp["w2_scale"])
    ref = M.moe_layer_forward(*args)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    held = []
    orig = M.workspace

    def spy(*a, **k):
        t = orig(*a, **k)
        held.append((t.data_ptr(), t.numel()))
        return t

    M.workspace = spy
    try:
        keep = _busy(side)                      # the layer queues behind this
        y = torch.empty_like(ref)
        y.record_stream(side)
        M.moe_layer_forward(*args, y=y, stream=side)
    finally:
        M.workspace = orig
    (ptr, n), = held
    # the wrapper's workspace has been freed on the host side; while the side
    # stream still has work queued, an allocation of the same size on the
    # current stream must not get those bytes
    junk = torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV)
    assert junk.data_ptr() != ptr
    torch.cuda.synchronize()
    del keep
    assert torch.equal(raw_t(y), raw_t(ref))


def raw_t(t):
    return t.view(torch.int16)


def test_stage_wrappers_on_side_stream_match_current_stream():
    """The stage entry points on a side stream give the same bits as on the
    current stream (their own outputs and workspaces are kept for the side
    stream)."""
    cfg = D.MoEConfig("side2", S=300, d=256, d_ff=512, E=16, K=2, router_offset="normal", offset_beta=0.3)
    inp = D.make_inputs(cfg, DEV)
    p = problem(cfg)

    def run(stream):
        idx, gate = M.moe_route(p, inp["x"], inp["W_r"], inp["router_bias"], inp["select_bias"], stream=stream)
        c, o, perm, inv, xp = M.moe_permute(p, idx, inp["x"], stream=stream)
        h, yp = M.moe_expert_ffn(p, xp, c, o, inp["W1"], inp["b1"], inp["W2"], inp["b2"], stream=stream)
        y = M.moe_combine(p, yp, inv, gate, stream=stream)
        return idx, gate, c, y

    a = run(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    keep = _busy(side, 4)
    b = run(side)
    # allocations on the current stream meanwhile
    junk = [torch.full((1 << 20,), 7, dtype=torch.int32, device=DEV) for _ in range(8)]
    torch.cuda.synchronize()
    del keep, junk
    for u, v in zip(a, b):
        assert np.array_equal(raw(u), raw(v))
