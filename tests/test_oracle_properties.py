"""Property tests of both CPU oracles on tiny shapes, searched by hypothesis.

Each property follows from what the layer computes, not from the oracles'
own code: the Top-K keeps the K largest keys (equal keys in index order) and
nothing else; relabelling experts relabels the choice and leaves the output
alone; the gates are a softmax, so they ignore a common shift of the scores
and see the temperature only through s / tau; the selection-only bias moves
the choice and not the gates; a token's output depends on that token alone;
the dispatch lists every valid pair once, inside its expert's padded band;
the activation quantiser picks the nearest code.  Integer-valued scores keep
every float32 step exact, so the properties hold bit for bit and ties are
common.  The search is derandomised so the suite is the same on every run.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, assume, given, settings
from hypothesis import strategies as st

import oracle as O
from oracle import cref

SETTINGS = settings(max_examples=60, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@st.composite
def routing_case(draw, groups=False):
    """(logits [S,E] float32 with small integer values, K, n_groups, topk_groups)."""
    if groups:
        G = draw(st.sampled_from([2, 4]))
        m = draw(st.sampled_from([1, 2, 4]))
        E = G * m
        tg = draw(st.integers(1, G))
        K = draw(st.integers(1, tg * m))
    else:
        E = draw(st.integers(1, 12))
        G, tg = 1, 1
        K = draw(st.integers(1, E))
    S = draw(st.integers(1, 4))
    vals = draw(st.lists(st.integers(-4, 4), min_size=S * E, max_size=S * E))
    return np.array(vals, dtype=np.float32).reshape(S, E), K, G, tg


def _assert_topk(keys, idx):
    """idx[t] lists the K largest keys of row t, largest first, equal keys
    in increasing index; every expert left out has a key no larger than the
    last one chosen, and a lower-index expert with the same key is chosen."""
    S, E = keys.shape
    for t in range(S):
        ch = [int(e) for e in idx[t]]
        assert len(set(ch)) == len(ch) and all(0 <= e < E for e in ch)
        for a, b in zip(ch, ch[1:]):
            assert keys[t, a] > keys[t, b] or (keys[t, a] == keys[t, b] and a < b)
        last = ch[-1]
        for e in set(range(E)) - set(ch):
            assert keys[t, e] < keys[t, last] or (keys[t, e] == keys[t, last] and e > last)


@SETTINGS
@given(routing_case())
def test_selection_is_the_k_largest_keys(case):
    logits, K, _, _ = case
    idx_np = O.select_experts(logits, K)
    idx_c, _ = cref.route(logits, K)
    assert np.array_equal(idx_np, idx_c)
    _assert_topk(logits, idx_c)


@SETTINGS
@given(routing_case(groups=True))
def test_group_limit_keeps_the_best_groups(case):
    """The chosen experts come from the topk_groups groups of largest summed
    key (equal sums in group order), and are the K largest keys among them."""
    logits, K, G, tg = case
    idx_np = O.select_experts(logits, K, n_groups=G, topk_groups=tg)
    idx_c, _ = cref.route(logits, K, n_groups=G, topk_groups=tg)
    assert np.array_equal(idx_np, idx_c)
    S, E = logits.shape
    m = E // G
    sums = logits.astype(np.float64).reshape(S, G, m).sum(axis=2)  # small integers: exact
    for t in range(S):
        order = sorted(range(G), key=lambda g: (-sums[t, g], g))
        kept = order[:tg]
        masked = np.where(np.repeat(np.isin(np.arange(G), kept), m), logits[t], -np.inf)
        _assert_topk(masked[None, :], idx_c[t:t + 1])
        assert all(int(e) // m in kept for e in idx_c[t])


@SETTINGS
@given(st.data())
def test_relabelling_experts_relabels_the_choice(data):
    E = data.draw(st.integers(2, 12))
    K = data.draw(st.integers(1, E))
    S = data.draw(st.integers(1, 4))
    rows = [data.draw(st.permutations(list(range(-E, 0)))) for _ in range(S)]  # distinct keys: no ties
    logits = np.array(rows, dtype=np.float32)
    pi = np.array(data.draw(st.permutations(list(range(E)))))
    idx, gate = cref.route(logits, K)
    idx_p, gate_p = cref.route(logits[:, pi], K)   # expert j of the new labels is expert pi[j]
    assert np.array_equal(pi[idx_p], idx)
    assert np.array_equal(gate_p, gate)


@SETTINGS
@given(routing_case(), st.integers(-6, 6), st.sampled_from([0, 1]))
def test_gates_ignore_a_common_shift(case, c, renorm):
    logits, K, _, _ = case
    idx, g = cref.route(logits, K, renormalize=renorm)
    idx_s, g_s = cref.route(logits + np.float32(c), K, renormalize=renorm)
    assert np.array_equal(idx, idx_s)
    np.testing.assert_allclose(g_s, g, rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.gate_weights(logits + np.float32(c), idx, renorm), g, rtol=1e-14, atol=0)


@SETTINGS
@given(routing_case(), st.sampled_from([0.5, 2.0, 4.0]), st.sampled_from([0, 1]))
def test_temperature_acts_as_scaled_scores(case, tau, renorm):
    """Gates at temperature tau equal gates of s / tau at temperature 1
    (s / tau is exact here); the choice does not depend on tau."""
    logits, K, _, _ = case
    idx, g = cref.route(logits, K, renormalize=renorm, temperature=tau)
    idx1, g1 = cref.route((logits / np.float32(tau)).astype(np.float32), K, renormalize=renorm)
    assert np.array_equal(idx, cref.route(logits, K)[0])
    assert np.array_equal(idx, idx1)
    np.testing.assert_allclose(g, g1, rtol=1e-14, atol=0)
    np.testing.assert_allclose(O.gate_weights(logits, idx, renorm, tau), g, rtol=1e-14, atol=0)


@SETTINGS
@given(routing_case())
def test_plain_gates_are_renormalised_gates_scaled_by_their_mass(case):
    logits, K, _, _ = case
    _, g1 = cref.route(logits, K, renormalize=1)
    _, g0 = cref.route(logits, K, renormalize=0)
    mass = g0.sum(axis=1, keepdims=True)
    assert np.all(mass <= 1 + 1e-14) and np.all(g0 > 0)
    np.testing.assert_allclose(g1.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(g0, g1 * mass, rtol=1e-13, atol=0)
    if K == logits.shape[1]:
        np.testing.assert_allclose(g0, g1, rtol=1e-14, atol=0)


@SETTINGS
@given(routing_case(), st.data())
def test_selection_bias_moves_choice_not_gates(case, data):
    logits, K, _, _ = case
    E = logits.shape[1]
    b = np.array(data.draw(st.lists(st.integers(-3, 3), min_size=E, max_size=E)), dtype=np.float32)
    idx, g = cref.route(logits, K, select_bias=b)
    idx_sum, _ = cref.route((logits + b[None, :]).astype(np.float32), K)
    assert np.array_equal(idx, idx_sum)
    np.testing.assert_allclose(g, O.gate_weights(logits, idx, 1), rtol=1e-14, atol=0)
    assert np.array_equal(O.select_experts(logits, K, select_bias=b), idx)


@SETTINGS
@given(st.data())
def test_dispatch_lists_every_valid_pair_once(data):
    E = data.draw(st.integers(1, 6))
    K = data.draw(st.integers(1, 3))
    S = data.draw(st.integers(0, 9))
    tile = data.draw(st.sampled_from([1, 2, 3, 8]))
    vals = data.draw(st.lists(st.integers(-1, E), min_size=S * K, max_size=S * K))  # -1 and E: dropped
    idx = np.array(vals, dtype=np.int32).reshape(S, K)
    counts, offsets, perm, inv = cref.permute(idx, E, tile)
    flat = idx.reshape(-1)
    valid = (flat >= 0) & (flat < E)
    assert np.array_equal(counts, np.bincount(flat[valid], minlength=E))
    assert offsets[0] == 0 and np.all(offsets % tile == 0)
    assert np.array_equal(np.diff(offsets), (counts + tile - 1) // tile * tile)
    # perm: the valid pairs sorted by (expert, pair id), each once
    assert np.array_equal(perm, np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")])
    dense = np.concatenate([[0], np.cumsum(counts)])
    for i, p in enumerate(perm):
        e = flat[p]
        assert inv[p] == offsets[e] + (i - dense[e])
    assert np.all(inv[~valid] == -1)
    if valid.all() and S > 0:
        P = O.permute(idx, E, tile)
        assert np.array_equal(P["perm"], perm) and np.array_equal(P["inv_perm"], inv)
        assert np.array_equal(P["offsets"], offsets)


def _layer_weights(rng, E, d, d_ff):
    return (rng.normal(size=(E, d)) * 0.5, rng.normal(size=(E, d_ff, d)) * 0.3, rng.normal(size=(E, d_ff)) * 0.1,
            rng.normal(size=(E, d, d_ff)) * 0.3, rng.normal(size=(E, d)) * 0.1)


@st.composite
def layer_case(draw):
    E = draw(st.sampled_from([1, 2, 4, 8]))
    K = draw(st.integers(1, E))
    S = draw(st.integers(1, 6))
    d = draw(st.integers(1, 8))
    d_ff = draw(st.integers(1, 12))
    seed = draw(st.integers(0, 2**31 - 1))
    return E, K, S, d, d_ff, seed


@SETTINGS
@given(layer_case(), st.data())
def test_layer_relabelling_and_token_order(case, data):
    """Relabelling experts (router row, W1, b1, W2, b2 together) and
    reordering tokens leave each token's output unchanged bit for bit; a
    subset of tokens gets the rows it gets in the full batch."""
    E, K, S, d, d_ff, seed = case
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(S, d))
    wr, W1, b1, W2, b2 = _layer_weights(rng, E, d, d_ff)
    y, idx, _ = cref.layer_forward(x, wr, W1, b1, W2, b2, K=K)
    pi = np.array(data.draw(st.permutations(list(range(E)))))
    y_p, idx_p, _ = cref.layer_forward(x, wr[pi], W1[pi], b1[pi], W2[pi], b2[pi], K=K)
    assert np.array_equal(pi[idx_p], idx)
    assert np.array_equal(y_p, y)
    sigma = np.array(data.draw(st.permutations(list(range(S)))))
    y_s, _, _ = cref.layer_forward(x[sigma], wr, W1, b1, W2, b2, K=K)
    assert np.array_equal(y_s, y[sigma])
    y_1, _, _ = cref.layer_forward(x[sigma[:1]], wr, W1, b1, W2, b2, K=K)
    assert np.array_equal(y_1, y[sigma[:1]])


@SETTINGS
@given(layer_case(), st.sampled_from([0, 1]))
def test_layer_output_bias_enters_by_gate_mass(case, renorm):
    """Adding a vector delta to every expert's b2 adds delta times the sum of
    the token's gates (delta itself when the gates are renormalised)."""
    E, K, S, d, d_ff, seed = case
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(S, d))
    wr, W1, b1, W2, b2 = _layer_weights(rng, E, d, d_ff)
    delta = rng.normal(size=d)
    y, _, g = cref.layer_forward(x, wr, W1, b1, W2, b2, K=K, renormalize=renorm)
    y2, _, _ = cref.layer_forward(x, wr, W1, b1, W2, b2 + delta[None, :], K=K, renormalize=renorm)
    np.testing.assert_allclose(y2 - y, g.sum(axis=1, keepdims=True) * delta[None, :], rtol=1e-9, atol=1e-12)


@SETTINGS
@given(layer_case())
def test_layer_oracles_agree(case):
    E, K, S, d, d_ff, seed = case
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(S, d)).astype(np.float32)
    wr, W1, b1, W2, b2 = (a.astype(np.float32) for a in _layer_weights(rng, E, d, d_ff))
    y_c, idx_c, g_c = cref.layer_forward(x, wr, W1, b1, W2, b2, K=K)
    parts = O.layer_forward(x, wr, list(W1), list(b1), list(W2), list(b2), K=K, act="f32", w="f32",
                            return_parts=True)
    assert np.array_equal(parts["idx"], idx_c)
    np.testing.assert_allclose(parts["gates"], g_c, rtol=1e-13, atol=0)
    np.testing.assert_allclose(parts["y"], y_c, rtol=1e-11, atol=1e-12)


@SETTINGS
@given(st.lists(st.floats(-1e4, 1e4, width=32), min_size=1, max_size=24), st.integers(1, 3),
       st.integers(-150, 0))
def test_activation_quantiser_picks_the_nearest_code(vals, rows, shift):
    """Each code is the e4m3 value nearest to v * (448 / amax) (clipped),
    equal distances going to the even code, and a row's largest |v| maps to
    448.  A row scaled by 2^shift, down into the range where 448 / amax
    overflows float32 and into float32 subnormals, gets the codes of the
    same (rounded) row scaled back up, and the scale amax / 448."""
    v = np.array(vals * rows, dtype=np.float32).reshape(rows, -1)
    v[1:] *= np.float32(0.5)
    assume(np.abs(v).max() >= 1e-20)
    small = (v * np.float32(2.0 ** shift)).astype(np.float32)
    back = (small.astype(np.float64) * 2.0 ** -shift).astype(np.float32)   # exact: a power of two
    q_small, s_small = O.quantize_rows_e4m3(small)
    codes, s = O.quantize_rows_e4m3(back)
    np.testing.assert_array_equal(q_small, codes)
    np.testing.assert_array_equal(s_small, (np.abs(small).max(axis=1) / np.float32(448)).astype(np.float32))
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    table = O.decode_e4m3fn(np.array(finite, dtype=np.uint8))
    for r in range(rows):
        amax = np.float32(np.abs(back[r]).max())
        if amax == 0:
            assert s[r] == 0 and np.all(codes[r] == 0)
            continue
        assume(amax >= 1e-30)
        rcp = np.float32(np.float32(448.0) / amax)
        t = np.clip((back[r] * rcp).astype(np.float32), -448, 448).astype(np.float64)
        got = O.decode_e4m3fn(codes[r])
        for ti, gi, ci in zip(t, got, codes[r]):
            dist = np.abs(table - ti)
            assert abs(gi - ti) == dist.min()
            if np.count_nonzero(dist == dist.min()) > 1 and ti != 0:
                assert ci % 2 == 0
        assert np.abs(got).max() == 448.0
