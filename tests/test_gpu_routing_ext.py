"""GPU parity of the gate temperature (soft routing, chapter 11 section
11.3.3) and of the load statistics (section 1.2 of "MoE 推理工程深层实战",
chapter 11 sections 11.1.2 and 11.3.2), through the C ABI."""
import dataclasses

import numpy as np
import pytest
import torch

import datagen as D
import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, GATE_TOL, gpu_inputs, oracle_view

pytestmark = pytest.mark.gpu


def sync():
    torch.cuda.synchronize()


def _problem(cfg, S=None, tau=1.0, K=None):
    return M.make_problem(cfg.S if S is None else S, cfg.d, cfg.d_ff, cfg.E, cfg.K if K is None else K,
                          cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups, cfg.renormalize, tau)


@pytest.mark.parametrize("name,tau", [("tiny_f32", 0.5), ("mixtral_prefill", 2.0), ("zipf_skew", 0.7),
                                      ("dsv3_fp8", 1.3)])
def test_route_with_temperature_given_logits(name, tau):
    """Indices do not depend on tau (bit-exact); gates are the oracle's
    softmax of score / tau (over the chosen, or over all for renormalize=0)."""
    cfg = D.CONFIGS[name]
    S = min(cfg.S, 2048)
    rng = np.random.default_rng(21)
    logits = (rng.standard_normal((S, cfg.E)) * 2).astype(np.float32)
    ov = oracle_view(gpu_inputs(name))
    sb = ov["select_bias"]
    for renorm in (1, 0):
        c = dataclasses.replace(cfg, renormalize=renorm)
        p = _problem(c, S=S, tau=tau)
        idx, gate = M.moe_route(p, None, None, select_bias=None if sb is None else torch.from_numpy(sb).to(DEV),
                                logits_in=torch.from_numpy(logits).to(DEV))
        sync()
        o_idx = O.select_experts(logits, cfg.K, sb, cfg.n_groups, cfg.topk_groups)
        assert np.array_equal(idx.cpu().numpy(), o_idx)
        o_gate = O.gate_weights(logits, o_idx, renorm, tau)
        np.testing.assert_allclose(gate.cpu().numpy(), o_gate, rtol=0, atol=GATE_TOL)


def test_fused_router_with_temperature():
    """The fused scores + selection kernel (bf16 x . W_r) applies tau to the
    gates of the scores it computed."""
    cfg = D.CONFIGS["mixtral_prefill"]
    inp = gpu_inputs("mixtral_prefill")
    p = _problem(cfg, tau=0.6)
    logits = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    idx, gate = M.moe_route(p, inp["x"], inp["W_r"], inp["router_bias"], logits_out=logits)
    sync()
    lg = logits.cpu().numpy()
    o_idx = O.select_experts(lg, cfg.K)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(gate.cpu().numpy(), O.gate_weights(lg, o_idx, 1, 0.6), rtol=0, atol=GATE_TOL)


@pytest.mark.parametrize("name,alpha,tau", [("tiny_f32", 0.01, 1.0), ("mixtral_prefill", 1.0, 1.0),
                                            ("decode", 0.5, 2.0), ("zipf_skew", 0.01, 1.0),
                                            ("dsv3_fp8", 0.001, 0.8)])
def test_load_stats_match_oracle(name, alpha, tau):
    cfg = D.CONFIGS[name]
    inp = gpu_inputs(name)
    p = _problem(cfg, tau=tau)
    logits = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                        inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"],
                        logits_out=logits, expert_counts_out=counts)
    dropped = torch.tensor([3], dtype=torch.int32, device=DEV)
    st = M.moe_load_stats(p, counts, logits, dropped, alpha)
    st2 = M.moe_load_stats(p, counts, logits, dropped, alpha)
    sync()
    g = st.cpu().numpy()
    assert np.array_equal(g, st2.cpu().numpy())  # deterministic
    ref = O.load_stats(counts.cpu().numpy(), cfg.S, cfg.K, logits.cpu().numpy(), alpha, tau, dropped=3)
    for i, k in enumerate(M.STAT_NAMES):
        assert g[i] == pytest.approx(ref[k], rel=2e-5, abs=1e-9), (k, g[i], ref[k])
    assert g[M.STAT_NAMES.index("max_over_mean")] >= 1.0
    # without scores or drops those two are 0
    st0 = M.moe_load_stats(p, counts).cpu().numpy()
    assert st0[M.STAT_NAMES.index("aux_loss")] == 0.0 and st0[M.STAT_NAMES.index("drop_rate")] == 0.0


def test_soft_routing_layer_with_temperature():
    """K = E with tau = 2: the layer is sum_i softmax(s / 2)_i E_i(x)
    (section 11.3.3), fp32, against the oracle's whole forward."""
    cfg = dataclasses.replace(D.CONFIGS["tiny_f32"], K=8)
    inp = gpu_inputs("tiny_f32")
    p = _problem(cfg, tau=2.0)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"])
    sync()
    ov = oracle_view(inp)
    ref = O.layer_forward(ov["x"], ov["W_r"], ov["W1"], ov["b1"], ov["W2"], ov["b2"], K=8, act="f32", w="f32",
                          router_bias=ov["router_bias"], temperature=2.0)
    yg = raw(y).astype(np.float64)
    assert np.abs(yg - ref).max() <= 1e-5 * np.abs(ref).max()
