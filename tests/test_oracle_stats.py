"""Pins of the oracle's gate temperature and load statistics.

Soft routing with a temperature (chapter 11 section 11.3.3), the load metrics
of "MoE 推理工程深层实战" section 1.2 and chapter 11 section 11.3.2, and the
balance loss of chapter 11 section 11.1.2, each pinned by hand-computed
values, closed forms or a library routine, not by re-typing the formula.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _torch_ffn(x, w1, b1, w2, b2):
    return torch.nn.functional.gelu(x @ w1.T + b1, approximate="none") @ w2.T + b2


# ------------------------------------------------------------------ temperature
@pytest.mark.parametrize("tau", [0.5, 2.0, 3.7])
def test_soft_routing_with_temperature_matches_torch(tau):
    """K = E gives sum_i softmax(s / tau)_i E_i(x) (section 11.3.3)."""
    rng = np.random.default_rng(11)
    S, d, d_ff, E = 7, 10, 16, 6
    x = rng.standard_normal((S, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    w1 = rng.standard_normal((E, d_ff, d)).astype(np.float32) / 3
    b1 = rng.standard_normal((E, d_ff)).astype(np.float32)
    w2 = rng.standard_normal((E, d, d_ff)).astype(np.float32) / 4
    b2 = rng.standard_normal((E, d)).astype(np.float32)
    y = O.layer_forward(x, wr, w1, b1, w2, b2, K=E, act="f32", w="f32", temperature=tau)
    t = lambda a: torch.from_numpy(a.astype(np.float64))
    logits = torch.from_numpy((x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)).double()
    p = torch.softmax(logits / tau, dim=-1)
    ref = sum(p[:, i:i + 1] * _torch_ffn(t(x), t(w1[i]), t(b1[i]), t(w2[i]), t(b2[i])) for i in range(E))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_temperature_limits():
    """tau -> inf: every chosen expert gets 1/K (renormalised) or 1/E (raw
    softmax); tau -> 0: all weight on the top slot."""
    rng = np.random.default_rng(3)
    logits = rng.standard_normal((20, 9)).astype(np.float32)
    idx = O.select_experts(logits, 3)
    np.testing.assert_allclose(O.gate_weights(logits, idx, 1, 1e9), 1 / 3, rtol=1e-7)
    np.testing.assert_allclose(O.gate_weights(logits, idx, 0, 1e9), 1 / 9, rtol=1e-7)
    g = O.gate_weights(logits, idx, 1, 1e-4)
    np.testing.assert_allclose(g[:, 0], 1.0, atol=1e-12)
    np.testing.assert_allclose(g[:, 1:], 0.0, atol=1e-12)


def test_temperature_divides_the_scores():
    """Scaling scores and tau by the same power of two changes nothing
    (exact): tau divides the scores, it does not multiply them."""
    rng = np.random.default_rng(4)
    logits = rng.standard_normal((15, 8)).astype(np.float32)
    idx = O.select_experts(logits, 2)
    for renorm in (0, 1):
        a = O.gate_weights(logits, idx, renorm, 0.75)
        b = O.gate_weights(logits * np.float32(4), idx, renorm, 3.0)
        np.testing.assert_array_equal(a, b)
    # and tau = 2 on two chosen scores 0 and ln 4 gives weights 1/3, 2/3
    l = np.array([[math.log(4.0), 0.0, -5.0]], dtype=np.float32)
    g = O.gate_weights(l, O.select_experts(l, 2), 1, 2.0)
    np.testing.assert_allclose(g, [[2 / 3, 1 / 3]], rtol=1e-7)


# ------------------------------------------------------------------ load statistics
def test_load_stats_hand_computed():
    """counts [3, 1, 0, 4]: mean 2, population std sqrt(2.5), max/mean 2,
    one empty expert; 2 of S*K = 8 pairs dropped: drop rate 1/4."""
    st = O.load_stats(np.array([3, 1, 0, 4]), S=5, K=2, dropped=2)
    assert st["mean"] == 2.0
    assert st["std"] == pytest.approx(math.sqrt(2.5), rel=1e-15)
    assert st["max_over_mean"] == 2.0
    assert st["drop_rate"] == 0.2
    assert (st["max"], st["min"], st["empty"]) == (4.0, 0.0, 1.0)
    assert st["aux_loss"] == 0.0  # no scores given


def test_balance_loss_closed_forms():
    """sum_i f_i P_i = 1/E when either factor is uniform; it tends to 1 when
    one expert takes all assignments and all probability."""
    rng = np.random.default_rng(9)
    E, S = 8, 50
    counts = rng.integers(0, 30, E)
    flat = np.zeros((S, E), dtype=np.float32)
    assert O.load_stats(counts, S, 2, flat, alpha=0.01)["aux_loss"] == pytest.approx(0.01 / E, rel=1e-12)
    logits = rng.standard_normal((S, E)).astype(np.float32)
    even = np.full(E, 7)
    for tau in (1.0, 0.3):
        st = O.load_stats(even, S, 2, logits, alpha=2.0, temperature=tau)
        assert st["aux_loss"] == pytest.approx(2.0 / E, rel=1e-12)
    one = np.zeros(E, dtype=np.int64)
    one[3] = 100
    peaked = np.zeros((S, E), dtype=np.float32)
    peaked[:, 3] = 60.0
    assert O.load_stats(one, S, 2, peaked)["aux_loss"] == pytest.approx(1.0, abs=1e-20)


def test_balance_loss_bruteforce():
    """Loop form with math.exp on a small case."""
    rng = np.random.default_rng(10)
    S, E, tau = 6, 5, 1.7
    counts = np.array([4, 0, 3, 2, 3])
    logits = rng.standard_normal((S, E)).astype(np.float32)
    P = [0.0] * E
    for t in range(S):
        z = [math.exp(float(v) / tau) for v in logits[t]]
        for i in range(E):
            P[i] += z[i] / math.fsum(z) / S
    ref = 0.3 * math.fsum(counts[i] / counts.sum() * P[i] for i in range(E))
    assert O.load_stats(counts, S, 2, logits, alpha=0.3, temperature=tau)["aux_loss"] == pytest.approx(ref, rel=1e-13)
