"""Every token of two full-size layers against the oracle's plain C++ loops.

The layer tests elsewhere sample tokens, since the numpy oracle is slow at
these sizes.  The C++ loop oracle (double precision, OpenMP over tokens)
runs the whole Mixtral-shape prefill (4096 tokens, about 30 s on 16 threads)
and the Zipf-skewed layer (8192 tokens, about 25 s), so here every token's
output row is compared.  The oracle routes from the GPU's own float32
scores (logits_in), so the expert indices must agree exactly and the gates
to 1e-6; the outputs to the bf16 tolerance 2e-2 max|y_ref|.  The DeepSeek
shape would need 60 GB of decoded weights; it is covered expert by expert
in test_gpu_split_tail.py."""
import time

import numpy as np
import pytest
import torch

import datagen as D
from oracle import cref
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, GATE_TOL, TOL, gpu_inputs, problem

pytestmark = pytest.mark.gpu


def _decoded(t, dtype):
    return cref.decode(raw(t), dtype)


@pytest.mark.parametrize("name", ["mixtral_prefill", "zipf_skew"])
def test_layer_every_token_against_cpp_oracle(name):
    cfg = D.CONFIGS[name]
    inp = gpu_inputs(name)
    p = problem(cfg)
    lo = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.S, cfg.K), dtype=torch.float32, device=DEV)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], inp["router_bias"],
                            inp["select_bias"], inp["w1_scale"], inp["w2_scale"], topk_idx_out=idx,
                            topk_gate_out=gate, logits_out=lo)
    torch.cuda.synchronize()
    t0 = time.time()
    x = _decoded(inp["x"], cfg.act)
    W1, W2 = _decoded(inp["W1"], cfg.w), _decoded(inp["W2"], cfg.w)
    b1, b2 = _decoded(inp["b1"], cfg.act), _decoded(inp["b2"], cfg.act)
    wr = _decoded(inp["W_r"], cfg.act)
    print(f"{name}: inputs decoded in {time.time() - t0:.1f}s; oracle over {cfg.S} tokens, "
          f"{cref.threads()} threads", flush=True)
    t0 = time.time()
    y_ref, idx_ref, gate_ref = cref.layer_forward(x, wr, W1, b1, W2, b2, K=cfg.K, n_groups=cfg.n_groups,
                                                  topk_groups=cfg.topk_groups, renormalize=cfg.renormalize,
                                                  logits_in=lo.cpu().numpy())
    print(f"{name}: oracle took {time.time() - t0:.1f}s", flush=True)
    del W1, W2
    assert np.array_equal(idx.cpu().numpy(), idx_ref)
    np.testing.assert_allclose(gate.cpu().numpy(), gate_ref, rtol=0, atol=GATE_TOL)
    yg = _decoded(y, cfg.act)
    err = np.abs(yg - y_ref).max(axis=1)
    scale = np.abs(y_ref).max()
    worst = int(np.argmax(err))
    print(f"{name}: max |dy| {err.max():.3e} (token {worst}) against max |y| {scale:.3e}", flush=True)
    assert err.max() <= TOL[cfg.act] * scale
