"""A seeded sweep of small random layer configurations against the oracle.

Each case draws a shape (rows per expert from a few to several hundred, so
the decode, mid and prefill tile regimes all occur, with d and d_ff that
need the narrower channel tiles), a dtype combination (fp32, bf16, fp8
weights, fp8 activations), a routing variant (group limit with a selection
bias, raw or renormalised gates, a gate temperature, a skewing router
offset) and sometimes a per-expert capacity, and runs the whole layer.  The
oracle routes from the GPU's float32 scores (the scores themselves are
checked against their rounding bound elsewhere), so expert indices --
capacity decisions included -- must agree exactly, gates to 1e-6 and every
output row within the dtype tolerance."""
import numpy as np
import pytest
import torch

import datagen as D
import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, GATE_TOL, TOL

pytestmark = pytest.mark.gpu


def draw_case(seed):
    rng = np.random.default_rng(1000 + seed)
    act = "f32" if rng.random() < 0.2 else "bf16"
    w = "f32" if act == "f32" else ("fp8" if rng.random() < 0.4 else "bf16")
    act_quant = int(w == "fp8" and rng.random() < 0.5)
    unit = 128 if act_quant else 64
    d = unit * int(rng.integers(1, 6)) if rng.random() < 0.5 else int(rng.choice([256, 512]))
    d_ff = unit * int(rng.integers(1, 6)) if rng.random() < 0.5 else int(rng.choice([256, 512]))
    E = int(rng.choice([1, 2, 3, 4, 5, 8, 16, 32, 64, 100, 128, 256]))
    K = int(rng.integers(1, min(E, 8) + 1))
    n_groups, topk_groups, sbv = 1, 1, 0.0
    if E >= 4 and rng.random() < 0.4:
        gs = [g for g in (2, 4, 8, 16) if E % g == 0 and (E // g) & (E // g - 1) == 0]
        if gs:
            n_groups = int(rng.choice(gs))
            m = E // n_groups
            topk_groups = int(rng.integers(-(-K // m), n_groups + 1))
            sbv = 0.1
    per_expert = float(rng.choice([2, 20, 80, 300, 700]))
    S = max(1, min(3000, int(per_expert * E / K * rng.uniform(0.6, 1.4))))
    temperature = 1.0 if rng.random() < 0.6 else float(rng.uniform(0.5, 2.0))
    capacity = 0 if rng.random() < 0.6 else max(1, int(rng.uniform(0.5, 1.5) * S * K / E))
    cfg = D.MoEConfig(f"sweep{seed}", S=S, d=d, d_ff=d_ff, E=E, K=K, act=act, w=w, n_groups=n_groups,
                      topk_groups=topk_groups, renormalize=int(rng.random() < 0.8),
                      router_offset="normal" if rng.random() < 0.5 else "none",
                      offset_beta=float(rng.uniform(0.0, 1.0)), select_bias_var=sbv, seed=seed)
    return cfg, temperature, capacity, act_quant


@pytest.mark.parametrize("seed", range(32))
def test_random_layer_matches_oracle(seed):
    cfg, tau, cap, aq = draw_case(seed)
    print(f"sweep {seed}: {cfg} tau={tau:.3f} capacity={cap} act_quant={aq}", flush=True)
    inp = D.make_inputs(cfg, DEV)
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, tau, cap, aq)
    lo = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.S, cfg.K), dtype=torch.float32, device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"],
                            topk_idx_out=idx, topk_gate_out=gate, logits_out=lo, expert_counts_out=counts)
    torch.cuda.synchronize()
    host = {k: (None if v is None else raw(v)) for k, v in inp.items()}
    sb = None if inp["select_bias"] is None else inp["select_bias"].cpu().numpy()
    lg = lo.cpu().numpy()
    ref = O.layer_forward(host["x"], host["W_r"], host["W1"], host["b1"], host["W2"], host["b2"], K=cfg.K,
                          act=cfg.act, w=cfg.w, select_bias=sb, n_groups=cfg.n_groups,
                          topk_groups=cfg.topk_groups, renormalize=cfg.renormalize, temperature=tau,
                          w1_scale=host["w1_scale"], w2_scale=host["w2_scale"], logits_in=lg, capacity=cap,
                          act_quant=bool(aq), return_parts=True)
    g_idx = idx.cpu().numpy()
    assert np.array_equal(g_idx, ref["idx"])
    np.testing.assert_allclose(gate.cpu().numpy(), ref["gates"], rtol=0, atol=GATE_TOL)
    kept = g_idx[g_idx >= 0]
    assert np.array_equal(counts.cpu().numpy(), np.bincount(kept, minlength=cfg.E))
    tol = TOL["fp8"] if cfg.w == "fp8" else TOL[cfg.act]
    yg = O.decode(raw(y), cfg.act)
    yr = ref["y"]
    assert np.abs(yg - yr).max() <= tol * max(np.abs(yr).max(), 1e-30)
