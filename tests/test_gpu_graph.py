"""The layer captured once in a HIP graph (torch.cuda.CUDAGraph) and
replayed.  The library launches kernels only -- no memsets, copies or host
synchronisation -- and every kernel of the layer is deterministic, so each
replay must give the eager output bit for bit, also with the program's own
eager work (another layer call on the same workspace, a fill kernel) and
synchronisations between the replays."""
import pytest
import torch

import datagen as D
import sparse_ffn_layer_amd as M
from tests.gpu_common import DEV, gpu_inputs

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("name,capacity,act_quant", [("tiny_f32", 0, 0), ("decode", 0, 0), ("mixtral_prefill", 0, 0),
                                                     ("mixtral_prefill", 1280, 0), ("zipf_skew", 600, 0),
                                                     ("dsv3_fp8", 0, 1)])
def test_layer_graph_replays_match_eager(name, capacity, act_quant):
    """Also with a per-expert capacity (its rounds keep counters in the
    workspace, reset by the kernels themselves) and with fp8 activations
    (rows quantised between the products)."""
    cfg = D.CONFIGS[name]
    inp = gpu_inputs(name)
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, 1.0, capacity, act_quant)
    print(f"graph replay {name} capacity={capacity} act_quant={act_quant}", flush=True)
    ws = M.workspace(p, M.STAGE_LAYER, DEV)
    act = torch.bfloat16 if cfg.act == "bf16" else torch.float32
    y_eager = torch.empty((cfg.S, cfg.d), dtype=act, device=DEV)
    y_graph = torch.empty_like(y_eager)

    def run(y):
        M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"],
                            y=y, ws=ws)

    run(y_eager)
    torch.cuda.synchronize()
    ref = _bits(y_eager).clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a call on a side stream before capture
        run(y_graph)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(y_graph)
    for _ in range(3):
        y_graph.zero_()
        run(y_eager)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_eager), ref)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(y_graph), ref)
