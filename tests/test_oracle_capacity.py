"""Pins of the oracle's capacity-limited dispatch.

Expert dropping (chapter 11 section 11.3.3: an overloaded expert's excess
moves to the next-best expert) and token dropping ("MoE 推理工程深层实战"
sections 1.2 and 2.2).  The pages leave the rule open; the reading (rounds of
in-order acceptance, rejected pairs move to the token's best expert with
room) is pinned by hand-worked examples, by properties any correct result of
that reading has, and by closed forms for the cases that reduce to counting.
"""
import json
import pathlib

import numpy as np
import pytest

import oracle as O

GOLDEN = pathlib.Path(__file__).parent / "golden" / "capacity_examples.json"


def _route(logits, K, sb=None, G=1, TG=1):
    return O.select_experts(logits, K, sb, G, TG)


def _case(seed, S, E, K, G=1, TG=1, bias=False, skew=0.0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((S, E)).astype(np.float32)
    lg += (skew * np.linspace(1.0, 0.0, E)).astype(np.float32)[None, :]   # a few hot experts
    sb = (rng.standard_normal(E) * 0.3).astype(np.float32) if bias else None
    return lg, sb, _route(lg, K, sb, G, TG)


CASES = [
    # seed, S, E, K, G, TG, bias, skew, capacity
    (1, 40, 8, 2, 1, 1, False, 2.0, 8),
    (2, 64, 8, 2, 1, 1, True, 3.0, 5),
    (3, 33, 16, 4, 4, 2, True, 1.5, 7),
    (4, 50, 32, 8, 8, 4, True, 2.0, 10),
    (5, 25, 4, 1, 1, 1, False, 4.0, 3),
    (6, 30, 6, 3, 1, 1, False, 5.0, 4),
    (7, 17, 16, 2, 4, 1, False, 3.0, 1),
]


# ------------------------------------------------------------------ worked examples
def _golden():
    return json.loads(GOLDEN.read_text())["examples"]


@pytest.mark.parametrize("ex", _golden(), ids=lambda e: e["name"])
def test_hand_worked_examples(ex):
    lg = np.array(ex["logits"], dtype=np.float32)
    sb = None if ex["select_bias"] is None else np.array(ex["select_bias"], dtype=np.float32)
    idx0 = _route(lg, ex["K"], sb, ex["n_groups"], ex["topk_groups"])
    idx, gates, dropped = O.apply_capacity(lg, idx0, ex["capacity"], sb, ex["n_groups"],
                                           ex["topk_groups"], ex["renormalize"])
    np.testing.assert_array_equal(idx, np.array(ex["expect_idx"]))
    np.testing.assert_allclose(gates, np.array(ex["expect_gates"]), rtol=1e-13, atol=1e-15)
    assert dropped == ex["expect_dropped"]
    load = np.bincount(idx[idx >= 0], minlength=ex["E"])
    np.testing.assert_array_equal(load, ex["expect_load"])


# ------------------------------------------------------------------ special cases
@pytest.mark.parametrize("c", CASES[:4])
@pytest.mark.parametrize("unlimited", ["zero", "SK", "huge"])
def test_enough_capacity_is_plain_routing(c, unlimited):
    """With room for every pair nothing moves: the indices are the Top-K
    selection and the gates those of the plain layer."""
    seed, S, E, K, G, TG, bias, skew, _ = c
    lg, sb, idx0 = _case(seed, S, E, K, G, TG, bias, skew)
    cap = {"zero": 0, "SK": S * K, "huge": 1 << 40}[unlimited]
    for renorm in (0, 1):
        idx, gates, dropped = O.apply_capacity(lg, idx0, cap, sb, G, TG, renorm)
        np.testing.assert_array_equal(idx, idx0)
        np.testing.assert_allclose(gates, O.gate_weights(lg, idx0, renorm), rtol=0, atol=0)
        assert dropped == 0


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("C", [1, 2, 5, 9])
def test_one_slot_without_groups_drops_only_past_total_room(seed, C):
    """K = 1, no group limit: every expert is a candidate, so a token drops
    only when all E experts are full: dropped = max(0, S - E*C)."""
    rng = np.random.default_rng(100 + seed)
    S, E = int(rng.integers(5, 60)), int(rng.integers(2, 9))
    lg = (rng.standard_normal((S, E)) + 3.0 * np.linspace(1, 0, E)).astype(np.float32)
    idx, _, dropped = O.apply_capacity(lg, _route(lg, 1), C)
    assert dropped == max(0, S - E * C)
    load = np.bincount(idx[idx >= 0], minlength=E)
    assert load.max() <= C


def test_single_expert_keeps_first_tokens():
    """E = K = 1: the expert keeps the first C tokens in token order."""
    lg = np.zeros((9, 1), dtype=np.float32)
    idx, gates, dropped = O.apply_capacity(lg, _route(lg, 1), 4)
    np.testing.assert_array_equal(idx[:, 0], [0, 0, 0, 0, -1, -1, -1, -1, -1])
    np.testing.assert_array_equal(gates[:, 0], [1, 1, 1, 1, 0, 0, 0, 0, 0])
    assert dropped == 5


def test_pairs_routed_to_no_expert_stay_dropped():
    """Index -1 (or any index outside [0, E)) is a dropped pair on entry and
    takes no room."""
    lg = np.array([[2, 1, 0], [2, 1, 0], [2, 1, 0]], dtype=np.float32)
    idx0 = np.array([[-1], [0], [7]], dtype=np.int32)
    idx, gates, dropped = O.apply_capacity(lg, idx0, 1)
    np.testing.assert_array_equal(idx[:, 0], [-1, 0, -1])
    assert dropped == 2
    assert gates[0, 0] == 0 and gates[1, 0] == 1.0


# ------------------------------------------------------------------ properties
def _order_pos(key_row):
    """Position of each expert in the token's ranking (key desc, index asc)."""
    order = np.argsort(-key_row, kind="stable")
    pos = np.empty_like(order)
    pos[order] = np.arange(order.size)
    return pos


@pytest.mark.parametrize("c", CASES)
def test_properties_of_capacity_dispatch(c):
    seed, S, E, K, G, TG, bias, skew, C = c
    lg, sb, idx0 = _case(seed, S, E, K, G, TG, bias, skew)
    key = O.selection_keys(lg, sb, G, TG)
    for renorm in (0, 1):
        idx, gates, dropped = O.apply_capacity(lg, idx0, C, sb, G, TG, renorm)
        kept = idx >= 0
        # room: no expert holds more than C pairs
        load = np.bincount(idx[kept], minlength=E)
        assert load.max() <= C
        # conservation: kept + dropped = S*K
        assert kept.sum() + dropped == S * K
        assert dropped == (~kept).sum()
        for t in range(S):
            ks = idx[t][kept[t]]
            # a token never holds one expert twice, and only eligible ones
            assert len(set(ks.tolist())) == ks.size
            assert np.all(np.isfinite(key[t, ks]))
            # a moved pair never moves up the token's ranking
            pos = _order_pos(key[t])
            for k in range(K):
                if kept[t, k]:
                    assert pos[idx[t, k]] >= pos[idx0[t, k]]
            # a token loses a slot only when every eligible expert it does
            # not hold is full
            if (~kept[t]).any():
                for e in np.nonzero(np.isfinite(key[t]))[0]:
                    if e not in ks:
                        assert load[e] == C
        # first come, first served: pair (t, k) keeps its routed expert
        # exactly when fewer than C earlier pairs were routed there
        seen = np.zeros(E, dtype=np.int64)
        for t in range(S):
            for k in range(K):
                e = idx0[t, k]
                assert (idx[t, k] == e) == (seen[e] < C)
                seen[e] += 1
        # gates: those of the plain layer over the kept slots, 0 elsewhere
        for t in range(S):
            ksl = np.nonzero(kept[t])[0]
            assert np.all(gates[t, ~kept[t]] == 0)
            if ksl.size:
                ref = O.gate_weights(lg[t:t + 1], idx[t:t + 1, ksl], renorm)[0]
                np.testing.assert_allclose(gates[t, ksl], ref, rtol=0, atol=0)
                if renorm:
                    assert abs(gates[t, ksl].sum() - 1.0) < 1e-12


@pytest.mark.parametrize("c", CASES[:3])
def test_temperature_changes_gates_not_dispatch(c):
    seed, S, E, K, G, TG, bias, skew, C = c
    lg, sb, idx0 = _case(seed, S, E, K, G, TG, bias, skew)
    i1, g1, d1 = O.apply_capacity(lg, idx0, C, sb, G, TG, 1, 1.0)
    i2, g2, d2 = O.apply_capacity(lg, idx0, C, sb, G, TG, 1, 2.5)
    np.testing.assert_array_equal(i1, i2)
    assert d1 == d2
    t = 0
    ks = np.nonzero(i2[t] >= 0)[0]
    z = lg[t, i2[t, ks]].astype(np.float64) / 2.5
    np.testing.assert_allclose(g2[t, ks], np.exp(z) / np.exp(z).sum(), rtol=1e-13)


def test_capacity_rejects_negative():
    lg, sb, idx0 = _case(0, 4, 4, 1)
    with pytest.raises(ValueError):
        O.apply_capacity(lg, idx0, -1)


def test_brute_force_tiny_against_exhaustive_candidate_check():
    """Tiny cases with many tied keys, every expert checked: for a moved
    pair, each expert ranked above its new one that the token does not hold
    is full (had one had room, the pair would have gone there)."""
    rng = np.random.default_rng(7)
    for _ in range(200):
        S, E = int(rng.integers(1, 7)), int(rng.integers(1, 6))
        K = int(rng.integers(1, E + 1))
        C = int(rng.integers(1, 4))
        lg = rng.integers(-2, 3, size=(S, E)).astype(np.float32)   # many ties
        idx0 = _route(lg, K)
        idx, _, dropped = O.apply_capacity(lg, idx0, C)
        load = np.bincount(idx[idx >= 0], minlength=E)
        for t in range(S):
            pos = _order_pos(lg[t])
            held = set(idx[t][idx[t] >= 0].tolist())
            for k in range(K):
                e = idx[t, k]
                if e >= 0 and e != idx0[t, k]:
                    for b in range(E):
                        if pos[b] < pos[e] and b not in held:
                            assert load[b] == C
        assert (idx >= 0).sum() + dropped == S * K


def test_layer_with_capacity_sums_kept_slots_only():
    """The layer under a capacity: y[t] is the gate-weighted sum over the
    token's kept slots only, computed here with torch per (token, slot); a
    subset of tokens gives the same rows as the whole batch (the rule looks
    at every token)."""
    import torch
    rng = np.random.default_rng(5)
    S, d, d_ff, E, K, C = 24, 8, 16, 4, 2, 7
    x = rng.standard_normal((S, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    wr[0] += 1.5 * x.mean(axis=0)                      # make expert 0 popular
    w1 = (rng.standard_normal((E, d_ff, d)) / 3).astype(np.float32)
    b1 = rng.standard_normal((E, d_ff)).astype(np.float32)
    w2 = (rng.standard_normal((E, d, d_ff)) / 4).astype(np.float32)
    b2 = rng.standard_normal((E, d)).astype(np.float32)
    parts = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32", capacity=C, return_parts=True)
    idx, gates = parts["idx"], parts["gates"]
    assert (idx < 0).any() or np.bincount(idx[idx >= 0], minlength=E).max() == C
    t64 = lambda a: torch.from_numpy(a.astype(np.float64))
    ref = np.zeros((S, d))
    for t in range(S):
        for k in range(K):
            e = idx[t, k]
            if e >= 0:
                h = torch.nn.functional.gelu(t64(x[t]) @ t64(w1[e]).T + t64(b1[e]), approximate="none")
                ref[t] += gates[t, k] * (h @ t64(w2[e]).T + t64(b2[e])).numpy()
    np.testing.assert_allclose(parts["y"], ref, rtol=1e-12, atol=1e-12)
    sub = [0, 5, 23]
    ys = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32", capacity=C, tokens=sub)
    np.testing.assert_allclose(ys, parts["y"][sub], rtol=1e-13, atol=1e-13)   # fp64 BLAS order
    # a capacity that is never reached gives the plain layer
    y0 = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32")
    yb = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32", capacity=S * K)
    np.testing.assert_allclose(yb, y0, rtol=0, atol=0)
