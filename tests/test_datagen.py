"""The seeded input generator: deterministic, sliceable, calibrated."""
import json
import os

import numpy as np
import torch

import datagen as D
import oracle as O
from tests._util import raw

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_deterministic_and_sliceable():
    cfg = D.CONFIGS["tiny_f32"]
    a = D.tokens(cfg)
    b = D.tokens(cfg)
    assert torch.equal(a, b)
    assert torch.equal(D.tokens(cfg, start=10, count=5), a[10:15])
    w = D.expert_weights(cfg, 3)
    assert torch.equal(w["W1"], D.make_inputs(cfg)["W1"][3])


def test_moments():
    x = D.normal(0, ("moments",), (1 << 20,), 4.0).double()
    assert abs(x.mean().item()) < 0.01
    assert abs(x.var().item() - 4.0) < 0.02
    u = D.uniform(0, ("moments_u",), (1 << 20,), 2.0).double()
    assert abs(u.mean().item()) < 0.01 and abs(u.var().item() - 4.0 / 3.0) < 0.01


def test_zipf_sampler_pmf():
    """Empirical P(k) for small k against k^-s / zeta(s)."""
    s = 1.1
    zeta = sum(k ** -s for k in range(1, 200000)) + 200000 ** (1 - s) / (s - 1)
    k = np.rint(np.exp(D.zipf_log_ranks(0, ("pmf",), 40000, s))).astype(np.int64)
    for kk in (1, 2, 3, 5):
        p = kk ** -s / zeta
        emp = np.mean(k == kk)
        assert abs(emp - p) < 4 * np.sqrt(p * (1 - p) / len(k))


def test_fp8_quantiser_roundtrip():
    w = D.normal(0, ("q",), (16, 256), 1.0 / 256)
    q, s = D.quantize_e4m3_rows(w)
    assert q.dtype == torch.float8_e4m3fn and s.shape == (16,)
    deq = O.expert_matrix(raw(q), "fp8", raw(s))
    assert np.all(np.abs(deq).max(1) <= raw(s) * 448 * (1 + 1e-6))
    rel = np.abs(deq - w.double().numpy()).max() / np.abs(w.double().numpy()).max()
    assert rel < 2 ** -4


def test_skew_recipes_in_band():
    """Realised max/mean expert load of the two skewed recipes."""
    with open(os.path.join(GOLDEN, "skew_calibration.json")) as f:
        cal = json.load(f)
    for name, lo, hi in (("mixtral_prefill", 2.95, 3.05), ("zipf_skew", 4.75, 5.25)):
        cfg = D.CONFIGS[name]
        assert cfg.offset_beta == cal[name]["beta"]
        x = O.decode(raw(D.tokens(cfg)), cfg.act)
        wr = O.decode(raw(D.router_weight(cfg)), cfg.act)
        logits = O.router_logits(x, wr, raw(D.router_bias(cfg)))
        idx = O.select_experts(logits, cfg.K)
        c = np.bincount(idx.reshape(-1), minlength=cfg.E)
        r = c.max() / (cfg.S * cfg.K / cfg.E)
        assert lo <= r <= hi, (name, r)
        if name == "zipf_skew":
            assert (c == 0).sum() >= 1
