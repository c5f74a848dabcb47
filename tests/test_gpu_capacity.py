"""GPU parity of capacity-limited dispatch (chapter 11 section 11.3.3, expert
dropping; "MoE 推理工程深层实战" sections 1.2 and 2.2, token dropping) through
the C ABI, against the oracle's apply_capacity on identical float32 logits:
indices and drop counts bit-exact, gates within GATE_TOL, layer outputs
within the dtype tolerance."""
import dataclasses
import json
import pathlib

import numpy as np
import pytest
import torch

import datagen as D
import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, GATE_TOL, gpu_inputs, oracle_view, sample_tokens, tol_of

pytestmark = pytest.mark.gpu

GOLDEN = pathlib.Path(__file__).parent / "golden" / "capacity_examples.json"


def sync():
    torch.cuda.synchronize()


def _prob(S, E, K, G=1, TG=1, renorm=1, tau=1.0, cap=0, d=64, d_ff=64, act="f32", w="f32"):
    return M.make_problem(S, d, d_ff, E, K, act, w, G, TG, renorm, tau, cap)


def _logits(S, E, seed, skew):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((S, E)).astype(np.float32)
    return (lg + (skew * np.linspace(1.0, 0.0, E)).astype(np.float32)[None, :]).astype(np.float32)


def _run(S, E, K, G, TG, lg, sb, cap, renorm, tau):
    """Route on the GPU, then limit; returns (routed idx, idx, gates, dropped)."""
    p = _prob(S, E, K, G, TG, renorm, tau, cap)
    sbt = None if sb is None else torch.from_numpy(sb).to(DEV)
    lt = torch.from_numpy(lg).to(DEV)
    idx0, _ = M.moe_route(p, None, None, select_bias=sbt, logits_in=lt)
    idx = idx0.clone()
    _, gate, dropped = M.moe_apply_capacity(p, lt, idx, select_bias=sbt)
    sync()
    return idx0.cpu().numpy(), idx.cpu().numpy(), gate.cpu().numpy(), int(dropped.cpu()[0])


CASES = [
    # id, S, E, K, G, TG, bias, skew, capacity factor, renorm, tau
    ("small_mixtral", 64, 8, 2, 1, 1, False, 2.0, 0.8, 1, 1.0),
    ("ragged_tail", 1000, 8, 2, 1, 1, True, 3.0, 0.6, 0, 1.0),
    ("many_chunks", 5000, 8, 1, 1, 1, False, 4.0, 1.0, 1, 1.0),
    ("groups_tau", 300, 64, 4, 8, 2, True, 1.5, 1.0, 1, 1.3),
    ("dsv3_groups", 512, 256, 8, 8, 4, True, 2.0, 0.9, 1, 1.0),
    ("E512", 200, 512, 8, 1, 1, False, 3.0, 0.5, 1, 1.0),
    ("E3_K1", 50, 3, 1, 1, 1, False, 1.0, 0.7, 1, 1.0),
    ("K64", 40, 128, 64, 1, 1, True, 2.0, 0.7, 0, 2.0),
    ("E1", 30, 1, 1, 1, 1, False, 0.0, 0.5, 1, 1.0),
    ("tight", 257, 16, 4, 4, 2, False, 5.0, 0.3, 1, 1.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_apply_capacity_matches_oracle(case):
    _, S, E, K, G, TG, bias, skew, f, renorm, tau = case
    lg = _logits(S, E, 31 + S, skew)
    sb = (np.random.default_rng(S).standard_normal(E) * 0.3).astype(np.float32) if bias else None
    cap = max(1, int(f * S * K / E))
    print(f"capacity case S={S} E={E} K={K} G={G} cap={cap}", flush=True)
    idx0, idx, gate, dropped = _run(S, E, K, G, TG, lg, sb, cap, renorm, tau)
    o_idx0 = O.select_experts(lg, K, sb, G, TG)
    assert np.array_equal(idx0, o_idx0)
    o_idx, o_gate, o_drop = O.apply_capacity(lg, o_idx0, cap, sb, G, TG, renorm, tau)
    assert np.array_equal(idx, o_idx)
    assert dropped == o_drop
    np.testing.assert_allclose(gate, o_gate, rtol=0, atol=GATE_TOL)
    # the limit was reached somewhere, so the case exercises the rule
    assert np.bincount(o_idx[o_idx >= 0], minlength=E).max() == cap or o_drop > 0
    # deterministic
    _, idx2, gate2, dropped2 = _run(S, E, K, G, TG, lg, sb, cap, renorm, tau)
    assert np.array_equal(idx, idx2) and np.array_equal(gate, gate2) and dropped == dropped2


@pytest.mark.parametrize("S,E,K,cap", [(16, 16, 1, 1), (19, 16, 1, 1), (96, 64, 2, 2), (300, 128, 4, 3),
                                        (64, 64, 1, 1)])
def test_many_rounds(S, E, K, cap):
    """Every token ranks the experts in the same order, so each round fills
    only a few experts: 16 to 64 rounds, past the fixed number of rerouting
    launches, so the single-workgroup finisher runs the rest."""
    lg = np.tile(-np.arange(E, dtype=np.float32), (S, 1))
    _, idx, gate, dropped = _run(S, E, K, 1, 1, lg, None, cap, 1, 1.0)
    o_idx, o_gate, o_drop = O.apply_capacity(lg, O.select_experts(lg, K), cap)
    assert np.array_equal(idx, o_idx)
    assert dropped == o_drop
    np.testing.assert_allclose(gate, o_gate, rtol=0, atol=GATE_TOL)


@pytest.mark.parametrize("cap_of", [lambda S, K: 0, lambda S, K: S * K], ids=["zero", "SK"])
def test_no_limit_keeps_routing_and_gates_bit_for_bit(cap_of):
    S, E, K, G, TG = 700, 64, 6, 8, 3
    lg = _logits(S, E, 3, 2.0)
    sb = (np.random.default_rng(4).standard_normal(E) * 0.2).astype(np.float32)
    for renorm in (1, 0):
        p = _prob(S, E, K, G, TG, renorm, 1.7, cap_of(S, K))
        lt, sbt = torch.from_numpy(lg).to(DEV), torch.from_numpy(sb).to(DEV)
        idx0, gate0 = M.moe_route(p, None, None, select_bias=sbt, logits_in=lt)
        idx = idx0.clone()
        _, gate, dropped = M.moe_apply_capacity(p, lt, idx, select_bias=sbt)
        sync()
        assert torch.equal(idx, idx0)
        assert torch.equal(gate, gate0)
        assert int(dropped.cpu()[0]) == 0


@pytest.mark.parametrize("ex", json.loads(GOLDEN.read_text())["examples"], ids=lambda e: e["name"])
def test_hand_worked_examples_on_gpu(ex):
    lg = np.array(ex["logits"], dtype=np.float32)
    S, E, K = lg.shape[0], ex["E"], ex["K"]
    sb = None if ex["select_bias"] is None else np.array(ex["select_bias"], dtype=np.float32)
    _, idx, gate, dropped = _run(S, E, K, ex["n_groups"], ex["topk_groups"], lg, sb, ex["capacity"],
                                 ex["renormalize"], 1.0)
    assert np.array_equal(idx, np.array(ex["expect_idx"]))
    assert dropped == ex["expect_dropped"]
    np.testing.assert_allclose(gate, np.array(ex["expect_gates"]), rtol=0, atol=GATE_TOL)


def test_indices_outside_range_count_as_dropped():
    S, E, K = 5, 3, 1
    lg = np.array([[2, 1, 0]] * S, dtype=np.float32)
    p = _prob(S, E, K, cap=1)
    idx = torch.tensor([[-1], [0], [7], [0], [-5]], dtype=torch.int32, device=DEV)
    _, gate, dropped = M.moe_apply_capacity(p, torch.from_numpy(lg).to(DEV), idx)
    sync()
    o_idx, o_gate, o_drop = O.apply_capacity(lg, np.array([[-1], [0], [7], [0], [-5]]), 1)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    assert int(dropped.cpu()[0]) == o_drop == 3
    np.testing.assert_allclose(gate.cpu().numpy(), o_gate, rtol=0, atol=GATE_TOL)


SAMPLE = {"tiny_f32": 64, "mixtral_prefill": 48, "decode": 16, "zipf_skew": 48, "dsv3_fp8": 8}


@pytest.mark.parametrize("name,factor", [("mixtral_prefill", 1.0), ("zipf_skew", 1.25), ("dsv3_fp8", 1.0),
                                         ("tiny_f32", 0.75), ("decode", 1.0)])
def test_layer_with_capacity_full_size(name, factor):
    """The whole layer with a capacity of factor * S*K/E pairs per expert at
    the workload's own size and skew: routing bit-exact against the oracle on
    the GPU's logits, the drop count from the expert counts, and sampled
    output rows within the dtype tolerance."""
    cfg = D.CONFIGS[name]
    inp = gpu_inputs(name)
    cap = max(1, int(factor * cfg.S * cfg.K / cfg.E))
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups,
                       cfg.topk_groups, cfg.renormalize, 1.0, cap)
    print(f"layer with capacity {name} cap={cap}", flush=True)
    logits = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.S, cfg.K), dtype=torch.float32, device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"],
                            topk_idx_out=idx, topk_gate_out=gate, logits_out=logits,
                            expert_counts_out=counts)
    sync()
    ov = oracle_view(inp)
    lg = logits.cpu().numpy()
    o_idx = O.select_experts(lg, cfg.K, ov["select_bias"], cfg.n_groups, cfg.topk_groups)
    o_idx, o_gate, o_drop = O.apply_capacity(lg, o_idx, cap, ov["select_bias"], cfg.n_groups,
                                             cfg.topk_groups, cfg.renormalize)
    assert np.array_equal(idx.cpu().numpy(), o_idx)
    np.testing.assert_allclose(gate.cpu().numpy(), o_gate, rtol=0, atol=GATE_TOL)
    c = counts.cpu().numpy()
    assert np.array_equal(c, np.bincount(o_idx[o_idx >= 0], minlength=cfg.E))
    assert c.max() <= cap
    assert cfg.S * cfg.K - int(c.sum()) == o_drop
    tok = sample_tokens(cfg.S, SAMPLE[name], seed=9)
    ref = O.layer_forward(ov["x"], ov["W_r"], ov["W1"], ov["b1"], ov["W2"], ov["b2"], K=cfg.K, act=cfg.act,
                          w=cfg.w, select_bias=ov["select_bias"], n_groups=cfg.n_groups,
                          topk_groups=cfg.topk_groups, renormalize=cfg.renormalize,
                          w1_scale=ov["w1_scale"], w2_scale=ov["w2_scale"], logits_in=lg, tokens=tok,
                          capacity=cap)
    yg = O.decode(raw(y[torch.from_numpy(np.asarray(tok)).to(DEV)]), cfg.act)
    assert np.abs(yg - ref).max() <= tol_of(cfg) * np.abs(ref).max()
    # drop rate through the load statistics
    dropped = torch.tensor([o_drop], dtype=torch.int32, device=DEV)
    st = M.moe_load_stats(p, counts, logits, dropped).cpu().numpy()
    ref_st = O.load_stats(c, cfg.S, cfg.K, lg, dropped=o_drop)
    assert st[M.STAT_NAMES.index("drop_rate")] == pytest.approx(ref_st["drop_rate"], rel=1e-6, abs=1e-9)
