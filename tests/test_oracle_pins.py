"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every test here runs on the CPU.  None compares the oracle with itself: each
uses a printed worked example, a special case that reduces to a library
routine (torch CPU float64), a closed form, an exhaustive check against a
library conversion, an invariant, or a pure-Python brute force.
"""
import itertools
import json
import math
import os
import random
import struct

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import datagen as D
import oracle as O
from tests._util import oracle_forward, raw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32(v):
    return struct.unpack("f", struct.pack("f", v))[0]


# ------------------------------------------------------------ worked example
def _worked():
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        return json.load(f)


def test_worked_example_routing_and_gates():
    g = _worked()
    logits = np.log(np.array(g["probs"], dtype=np.float64)).astype(np.float32)[None, :]
    idx = O.select_experts(logits, g["K"])
    assert idx.tolist() == [g["expect_idx"]]
    gates = O.gate_weights(logits, idx, renormalize=1)
    np.testing.assert_allclose(gates[0], g["expect_gates_renormalized"], atol=1e-7)
    raw_g = O.gate_weights(logits, idx, renormalize=0)
    np.testing.assert_allclose(raw_g[0], g["expect_gates_raw"], atol=1e-7)


def test_worked_example_layer_output():
    """With W1 = 0 and b1 = 0 every expert outputs its b2 (GeLU(0) = 0), so the
    layer output is g0 * b2[e0] + g1 * b2[e3] with the printed gates."""
    g = _worked()
    E, K, d, d_ff = g["E"], g["K"], 4, 8
    rng = np.random.default_rng(1)
    b2 = rng.standard_normal((E, d)).astype(np.float32)
    logits = np.log(np.array(g["probs"])).astype(np.float32)[None, :]
    zeros1 = np.zeros((E, d_ff, d), np.float32)
    w2 = rng.standard_normal((E, d, d_ff)).astype(np.float32)
    for renorm, key in ((1, "expect_gates_renormalized"), (0, "expect_gates_raw")):
        y = O.layer_forward(np.ones((1, d), np.float32), np.zeros((E, d), np.float32), zeros1,
                            np.zeros((E, d_ff), np.float32), w2, b2, K=K, act="f32", w="f32",
                            renormalize=renorm, logits_in=logits)
        gg = g[key]
        expect = gg[0] * b2[0].astype(np.float64) + gg[1] * b2[3].astype(np.float64)
        np.testing.assert_allclose(y[0], expect, rtol=0, atol=1e-6)


# ------------------------------------------------------------ special cases
def _torch_ffn(x, w1, b1, w2, b2):
    return F.linear(F.gelu(F.linear(x, w1, b1), approximate="none"), w2, b2)


@pytest.mark.parametrize("S,d,d_ff", [(7, 16, 40), (33, 24, 8)])
def test_single_expert_is_dense_ffn(S, d, d_ff):
    """E = 1, K = 1: the only gate is exactly 1 and the layer is the dense FFN
    GeLU(x W1 + b1) W2 + b2, here computed by torch CPU float64 ops."""
    rng = np.random.default_rng(S)
    x = rng.standard_normal((S, d)).astype(np.float32)
    w1 = rng.standard_normal((1, d_ff, d)).astype(np.float32) / math.sqrt(d)
    b1 = rng.standard_normal((1, d_ff)).astype(np.float32)
    w2 = rng.standard_normal((1, d, d_ff)).astype(np.float32) / math.sqrt(d_ff)
    b2 = rng.standard_normal((1, d)).astype(np.float32)
    wr = rng.standard_normal((1, d)).astype(np.float32)
    parts = O.layer_forward(x, wr, w1, b1, w2, b2, K=1, act="f32", w="f32", return_parts=True)
    assert np.all(parts["gates"] == 1.0)
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    ref = _torch_ffn(t(x), t(w1[0]), t(b1[0]), t(w2[0]), t(b2[0])).numpy()
    np.testing.assert_allclose(parts["y"], ref, rtol=1e-12, atol=1e-12)


def test_all_experts_is_soft_routing():
    """K = E with renormalised gates gives sum_i softmax(s)_i E_i(x): the soft
    routing formula of section 11.3.3 of the chapter at temperature 1."""
    rng = np.random.default_rng(5)
    S, d, d_ff, E = 9, 12, 20, 5
    x = rng.standard_normal((S, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    w1 = rng.standard_normal((E, d_ff, d)).astype(np.float32) / 3
    b1 = rng.standard_normal((E, d_ff)).astype(np.float32)
    w2 = rng.standard_normal((E, d, d_ff)).astype(np.float32) / 4
    b2 = rng.standard_normal((E, d)).astype(np.float32)
    y = O.layer_forward(x, wr, w1, b1, w2, b2, K=E, act="f32", w="f32")
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    logits = torch.from_numpy((x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)).double()
    p = torch.softmax(logits, dim=-1)
    ref = sum(p[:, i:i + 1] * _torch_ffn(t(x), t(w1[i]), t(b1[i]), t(w2[i]), t(b2[i])) for i in range(E))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------ top-k brute force
def _bf_topk(keys, K):
    return sorted(range(len(keys)), key=lambda e: (-keys[e], e))[:K]


@pytest.mark.parametrize("E,K", [(4, 1), (8, 2), (8, 8), (16, 3), (13, 5)])
def test_topk_matches_bruteforce_with_ties(E, K):
    rnd = random.Random(E * 31 + K)
    S = 64
    keys = np.array([[rnd.choice([-2.0, -0.5, 0.0, 0.5, 1.0, 3.0]) for _ in range(E)] for _ in range(S)],
                    dtype=np.float32)
    idx = O.select_experts(keys, K)
    for t in range(S):
        assert idx[t].tolist() == _bf_topk(keys[t].tolist(), K)


def test_topk_negative_zero_ties_with_zero():
    keys = np.array([[-0.0, 0.0, -1.0, 0.0]], dtype=np.float32)
    assert O.select_experts(keys, 3).tolist() == [[0, 1, 3]]


def _bf_group_limited(keys, K, G, tg, bias=None):
    E = len(keys)
    m = E // G
    kb = [keys[e] if bias is None else f32(keys[e] + bias[e]) for e in range(E)]
    gs = [sum(kb[g * m:(g + 1) * m]) for g in range(G)]
    groups = sorted(range(G), key=lambda g: (-gs[g], g))[:tg]
    masked = [kb[e] if e // m in groups else -math.inf for e in range(E)]
    return _bf_topk(masked, K), groups


@pytest.mark.parametrize("E,G,tg,K", [(16, 4, 2, 3), (16, 4, 1, 4), (32, 8, 2, 5), (256, 8, 2, 8), (64, 2, 1, 7)])
def test_group_limited_matches_bruteforce(E, G, tg, K):
    """Integer-valued keys make every float32 group sum exact, so a plain
    Python sum is an independent reference for the selection rule."""
    rnd = random.Random(E + G + tg + K)
    S = 48
    keys = np.array([[float(rnd.randint(-3, 3)) for _ in range(E)] for _ in range(S)], dtype=np.float32)
    bias = np.array([float(rnd.randint(-1, 1)) for _ in range(E)], dtype=np.float32)
    idx = O.select_experts(keys, K, select_bias=bias, n_groups=G, topk_groups=tg)
    for t in range(S):
        expect, groups = _bf_group_limited(keys[t].tolist(), K, G, tg, bias.tolist())
        assert idx[t].tolist() == expect
        assert all(e // (E // G) in groups for e in idx[t])


def test_group_score_tree_order():
    """The group sum follows the pairwise-halving tree: for [1e8, 1, -1e8, 1]
    the tree gives (1e8 + -1e8) + (1 + 1) = 2 in float32, while a left-to-right
    float32 sum would give 1."""
    keys = np.array([[1e8, 1.0, -1e8, 1.0]], dtype=np.float32)
    assert O.group_scores_f32(keys, 1)[0, 0] == np.float32(2.0)
    keys8 = np.array([[1.0, 2.0, 4.0, 8.0, 16.0, 32.0, 64.0, 128.0]], dtype=np.float32)
    assert O.group_scores_f32(keys8, 2).tolist() == [[15.0, 240.0]]


def test_selection_bias_changes_choice_not_gates():
    """The aux-loss-free bias shifts which experts are chosen but the gates
    are the softmax of the unbiased logits of the chosen experts."""
    logits = np.array([[2.0, 1.0, 0.5, 0.0]], dtype=np.float32)
    bias = np.array([0.0, 0.0, 3.0, 0.0], dtype=np.float32)
    idx = O.select_experts(logits, 2, select_bias=bias)
    assert idx.tolist() == [[2, 0]]
    g = O.gate_weights(logits, idx, 1)[0]
    e = [math.exp(0.5), math.exp(2.0)]
    np.testing.assert_allclose(g, [e[0] / sum(e), e[1] / sum(e)], rtol=1e-14)


# ------------------------------------------------------------ gate invariants
def test_gate_invariants():
    rng = np.random.default_rng(7)
    logits = (rng.standard_normal((200, 64)) * 3).astype(np.float32)
    for K in (1, 2, 6, 64):
        idx = O.select_experts(logits, K)
        g = O.gate_weights(logits, idx, 1)
        np.testing.assert_allclose(g.sum(1), 1.0, atol=1e-12)
        assert np.all(np.diff(g, axis=1) <= 0)        # Mixtral path: non-increasing
        p = O.softmax(logits)
        np.testing.assert_allclose(p.sum(1), 1.0, atol=1e-12)
        graw = O.gate_weights(logits, idx, 0)
        sel = np.take_along_axis(p, idx.astype(np.int64), 1)
        np.testing.assert_allclose(graw, sel, rtol=1e-12)
        np.testing.assert_allclose(g, sel / sel.sum(1, keepdims=True), rtol=1e-12, atol=1e-15)


# ------------------------------------------------------------ permutation
@pytest.mark.parametrize("S,E,K,tile", [(1, 8, 2, 16), (64, 8, 2, 16), (100, 64, 4, 32), (37, 256, 8, 64), (5, 3, 3, 1)])
def test_permutation_invariants(S, E, K, tile):
    rng = np.random.default_rng(S * E + K)
    idx = np.stack([rng.permutation(E)[:K] for _ in range(S)]).astype(np.int32)
    p = O.permute(idx, E, tile)
    flat = idx.reshape(-1)
    assert p["counts"].sum() == S * K
    assert np.array_equal(p["counts"], np.bincount(flat, minlength=E))
    assert sorted(p["perm"].tolist()) == list(range(S * K))
    assert p["perm"].tolist() == sorted(range(S * K), key=lambda q: (flat[q], q))
    for e in range(E):
        seg = p["perm"][p["dense_offsets"][e]:p["dense_offsets"][e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // K) > 0)            # token order inside an expert
        rows = p["inv_perm"][seg]
        assert rows.tolist() == list(range(p["offsets"][e], p["offsets"][e] + len(seg)))
    assert np.all(p["offsets"] % tile == 0)
    assert np.all(np.diff(p["offsets"]) >= p["counts"])
    assert np.all(np.diff(p["offsets"]) < p["counts"] + tile)
    assert len(set(p["inv_perm"].tolist())) == S * K


# ------------------------------------------------------------ FFN pieces
def test_gelu_matches_torch_exact_form():
    a = np.linspace(-9, 9, 2001)
    ref = F.gelu(torch.from_numpy(a), approximate="none").numpy()
    np.testing.assert_allclose(O.gelu(a), ref, rtol=1e-14, atol=1e-15)
    assert O.gelu(np.array([0.0]))[0] == 0.0
    assert abs(O.gelu(np.array([12.0]))[0] - 12.0) < 1e-12
    assert abs(O.gelu(np.array([-12.0]))[0]) < 1e-12
    tanh_form = F.gelu(torch.from_numpy(a), approximate="tanh").numpy()
    assert np.abs(O.gelu(a) - tanh_form).max() > 1e-4     # the erf form was chosen


def test_e4m3_decode_exhaustive():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float32).double().numpy()
    got = O.decode_e4m3fn(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.isnan(got).sum() == 2                       # S.1111.111 only
    assert got[0x7E] == 448.0 and got[0xFE] == -448.0
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert got[0xB8] == -1.0


def test_bf16_decode_exhaustive():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).double().numpy()
    got = O.decode_bf16(bits)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_fp8_weight_value_uses_channel_scale():
    codes = np.array([[0x38, 0xB8, 0x7E], [0x01, 0x00, 0x40]], dtype=np.uint8)
    scale = np.array([0.5, 3.0], dtype=np.float32)
    w = O.expert_matrix(codes, "fp8", scale)
    assert w.tolist() == [[0.5, -0.5, 224.0], [3.0 * 2 ** -9, 0.0, 6.0]]


# ------------------------------------------------------------ brute-force layer
def _bf_layer(x, wr, w1, b1, w2, b2, K, rbias=None):
    """Pure-Python loops, math.fsum and math.erf; no numpy arithmetic."""
    S, d = len(x), len(x[0])
    E, d_ff = len(w1), len(w1[0])
    y = []
    for t in range(S):
        logit = [f32(math.fsum(x[t][i] * wr[e][i] for i in range(d)) + (0.0 if rbias is None else rbias[e]))
                 for e in range(E)]
        sel = _bf_topk(logit, K)
        mx = max(logit[e] for e in sel)
        ex = [math.exp(logit[e] - mx) for e in sel]
        gates = [v / math.fsum(ex) for v in ex]
        out = [0.0] * d
        for g, e in zip(gates, sel):
            h = []
            for j in range(d_ff):
                a = math.fsum([x[t][i] * w1[e][j][i] for i in range(d)] + [b1[e][j]])
                h.append(0.5 * a * (1 + math.erf(a / math.sqrt(2))))
            for c in range(d):
                o = math.fsum([h[j] * w2[e][c][j] for j in range(d_ff)] + [b2[e][c]])
                out[c] += g * o
        y.append(out)
    return y


def test_layer_matches_pure_python_bruteforce():
    rng = np.random.default_rng(11)
    S, d, d_ff, E, K = 6, 5, 7, 4, 2
    x = rng.standard_normal((S, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    w1 = rng.standard_normal((E, d_ff, d)).astype(np.float32)
    b1 = rng.standard_normal((E, d_ff)).astype(np.float32)
    w2 = rng.standard_normal((E, d, d_ff)).astype(np.float32)
    b2 = rng.standard_normal((E, d)).astype(np.float32)
    rb = rng.standard_normal(E).astype(np.float32)
    y = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32", router_bias=rb)
    ref = _bf_layer(x.tolist(), wr.tolist(), w1.tolist(), b1.tolist(), w2.tolist(), b2.tolist(), K, rb.tolist())
    np.testing.assert_allclose(y, np.array(ref), rtol=1e-12, atol=1e-12)


def test_router_logits_bruteforce():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 33)).astype(np.float32)
    wr = rng.standard_normal((6, 33)).astype(np.float32)
    rb = rng.standard_normal(6).astype(np.float32)
    got = O.router_logits(x.astype(np.float64), wr.astype(np.float64), rb)
    for t in range(5):
        for e in range(6):
            exact = f32(math.fsum([float(a) * float(b) for a, b in zip(x[t], wr[e])] + [float(rb[e])]))
            assert got[t, e] == np.float32(exact)


# ------------------------------------------------------------ config data
def test_tiny_config_layer_runs_and_gates_sum_to_one():
    cfg = D.CONFIGS["tiny_f32"]
    inp = D.make_inputs(cfg)
    parts = oracle_forward(O, cfg, inp, return_parts=True)
    assert parts["y"].shape == (cfg.S, cfg.d)
    np.testing.assert_allclose(parts["gates"].sum(1), 1.0, atol=1e-12)
    counts = np.bincount(parts["idx"].reshape(-1), minlength=cfg.E)
    assert counts.sum() == cfg.S * cfg.K


def test_dsv3_routing_respects_groups_on_config_data():
    cfg = D.CONFIGS["dsv3_fp8"]
    x = O.decode(raw(D.tokens(cfg, count=128)), cfg.act)
    wr = O.decode(raw(D.router_weight(cfg)), cfg.act)
    logits = O.router_logits(x, wr)
    sb = raw(D.select_bias(cfg))
    idx = O.select_experts(logits, cfg.K, sb, cfg.n_groups, cfg.topk_groups)
    m = cfg.E // cfg.n_groups
    for t in range(len(idx)):
        assert len({int(e) // m for e in idx[t]}) <= cfg.topk_groups
        assert len(set(idx[t].tolist())) == cfg.K
        expect, _ = _bf_group_limited([float(v) for v in logits[t]], cfg.K, cfg.n_groups,
                                      cfg.topk_groups, [float(v) for v in sb])
        # float sums of non-integer keys may round differently from the tree;
        # the chosen set must still agree unless two group scores nearly tie
        gs = O.group_scores_f32((logits[t] + sb)[None, :].astype(np.float32), cfg.n_groups)[0]
        srt = np.sort(gs)[::-1]
        if srt[cfg.topk_groups - 1] - srt[cfg.topk_groups] > 1e-3:
            assert idx[t].tolist() == expect
