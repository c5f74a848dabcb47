"""Pins of the plain C++ reference loops (oracle/moe_oracle_ref.cpp), and the
C++ and numpy oracles against each other.

The C++ loops are the method written as loops over tokens, slots and
experts; they share no code with the numpy oracle (decoders included) nor
with the HIP path.  Each is pinned the same way as the numpy oracle (printed
worked example, special cases that reduce to library routines, brute force),
and the two agree on random problems: bit for bit on decoded values, indices
and permutations, to float64 rounding on gates and outputs.
"""
import json
import math
import pathlib

import numpy as np
import pytest
import torch

import oracle as O
from oracle import cref as C

GOLDEN = pathlib.Path(__file__).parent / "golden"


def test_decoders_exhaustive_against_torch():
    b = np.arange(1 << 16, dtype=np.uint16)
    ref = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = C.decode(b, "bf16")
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin], ref[fin])
    c = np.array([v for v in range(256) if (v & 0x7F) != 0x7F], dtype=np.uint8)
    ref8 = torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(C.decode(c, "fp8"), ref8)
    assert np.isnan(C.decode(np.array([0x7F, 0xFF], np.uint8), "fp8")).all()


def test_worked_example():
    ex = json.loads((GOLDEN / "worked_example.json").read_text())
    lg = np.log(np.array(ex["probs"], dtype=np.float64)).astype(np.float32)[None, :]
    idx, g = C.route(lg, ex["K"])
    assert idx[0].tolist() == ex["expect_idx"]
    np.testing.assert_allclose(g[0], ex["expect_gates_renormalized"], rtol=1e-6)
    _, g0 = C.route(lg, ex["K"], renormalize=0)
    np.testing.assert_allclose(g0[0], ex["expect_gates_raw"], rtol=1e-6)


@pytest.mark.parametrize("d,d_ff", [(8, 16), (12, 5)])
def test_single_expert_is_a_dense_ffn(d, d_ff):
    rng = np.random.default_rng(1)
    S = 9
    x = rng.standard_normal((S, d))
    w1, b1 = rng.standard_normal((1, d_ff, d)), rng.standard_normal((1, d_ff))
    w2, b2 = rng.standard_normal((1, d, d_ff)), rng.standard_normal((1, d))
    y, idx, g = C.layer_forward(x, rng.standard_normal((1, d)), w1, b1, w2, b2, K=1)
    assert np.all(idx == 0) and np.all(g == 1.0)
    t = lambda a: torch.from_numpy(a)
    ref = torch.nn.functional.gelu(t(x) @ t(w1[0]).T + t(b1[0]), approximate="none") @ t(w2[0]).T + t(b2[0])
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_all_experts_is_soft_routing():
    rng = np.random.default_rng(2)
    S, d, d_ff, E, tau = 6, 8, 10, 5, 1.7
    x, wr = rng.standard_normal((S, d)), rng.standard_normal((E, d))
    w1, b1 = rng.standard_normal((E, d_ff, d)) / 3, rng.standard_normal((E, d_ff))
    w2, b2 = rng.standard_normal((E, d, d_ff)) / 3, rng.standard_normal((E, d))
    y, _, _ = C.layer_forward(x, wr, w1, b1, w2, b2, K=E, temperature=tau)
    t = lambda a: torch.from_numpy(a)
    lg = torch.from_numpy(C.router_logits(x, wr)).double()
    p = torch.softmax(lg / tau, dim=-1)
    ref = sum(p[:, i:i + 1] * (torch.nn.functional.gelu(t(x) @ t(w1[i]).T + t(b1[i]), approximate="none")
                              @ t(w2[i]).T + t(b2[i])) for i in range(E))
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_router_logits_against_fsum():
    rng = np.random.default_rng(3)
    x, wr = rng.standard_normal((5, 33)), rng.standard_normal((4, 33))
    rb = rng.standard_normal(4).astype(np.float32)
    got = C.router_logits(x, wr, rb)
    for t in range(5):
        for e in range(4):
            ref = np.float32(math.fsum(list(x[t] * wr[e]) + [float(rb[e])]))
            assert abs(float(got[t, e]) - float(ref)) <= abs(float(ref)) * 2.0 ** -23


def test_topk_and_groups_brute_force_with_ties():
    rng = np.random.default_rng(4)
    for _ in range(200):
        E = int(rng.choice([4, 8, 16]))
        G = int(rng.choice([g for g in (1, 2, 4) if E % g == 0]))
        TG = int(rng.integers(1, G + 1))
        K = int(rng.integers(1, (E // G) * TG + 1))
        lg = rng.integers(-3, 4, size=(3, E)).astype(np.float32)
        idx, _ = C.route(lg, K, None, G, TG)
        for t in range(3):
            keys = lg[t].astype(np.float64)
            if G > 1:
                m = E // G
                gs = [sum(keys[g * m:(g + 1) * m]) for g in range(G)]      # exact: small integers
                keep = sorted(range(G), key=lambda g: (-gs[g], g))[:TG]
                keys = np.array([keys[e] if e // m in keep else -np.inf for e in range(E)])
            ref = sorted(range(E), key=lambda e: (-keys[e], e))[:K]
            assert idx[t].tolist() == ref


def test_permutation_brute_force():
    rng = np.random.default_rng(5)
    S, K, E, tm = 40, 3, 6, 4
    idx = np.stack([rng.permutation(E)[:K] for _ in range(S)]).astype(np.int32)
    idx[3, 1] = -1
    counts, offsets, perm, inv = C.permute(idx, E, tm)
    pairs = [(int(idx.reshape(-1)[p]), p) for p in range(S * K) if idx.reshape(-1)[p] >= 0]
    assert perm.tolist() == [p for _, p in sorted(pairs)]
    assert counts.tolist() == [sum(1 for e, _ in pairs if e == x) for x in range(E)]
    assert offsets[-1] == sum((c + tm - 1) // tm * tm for c in counts)
    assert inv[3 * K + 1] == -1
    for e in range(E):
        rows = sorted(inv[p] for ee, p in pairs if ee == e)
        assert rows == list(range(offsets[e], offsets[e] + counts[e]))


@pytest.mark.parametrize("seed,E,K,G,TG,renorm,w", [(0, 8, 2, 1, 1, 1, "bf16"), (1, 16, 4, 4, 2, 0, "fp8"),
                                                    (2, 32, 6, 8, 3, 1, "fp8"), (3, 4, 4, 1, 1, 1, "f32")])
def test_cpp_and_numpy_oracles_agree(seed, E, K, G, TG, renorm, w):
    rng = np.random.default_rng(seed)
    S, d, d_ff = 24, 32, 48
    x = torch.randn(S, d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    wr = (torch.randn(E, d) / 6).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    if w == "fp8":
        W1 = torch.randn(E, d_ff, d).clamp(-400, 400).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        W2 = torch.randn(E, d, d_ff).clamp(-400, 400).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        s1 = (rng.random((E, d_ff)) / 8).astype(np.float32)
        s2 = (rng.random((E, d)) / 8).astype(np.float32)
    else:
        wt = torch.bfloat16 if w == "bf16" else torch.float32
        conv = (lambda t: t.to(wt).view(torch.int16).numpy().view(np.uint16)) if w == "bf16" else (lambda t: t.numpy())
        W1, W2 = conv(torch.randn(E, d_ff, d) / 6), conv(torch.randn(E, d, d_ff) / 7)
        s1 = s2 = None
    bf = lambda t: t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    b1, b2 = bf(torch.randn(E, d_ff) / 10), bf(torch.randn(E, d) / 10)     # act dtype storage
    sb = (rng.standard_normal(E) * 0.3).astype(np.float32)
    rb = (rng.standard_normal(E) * 0.2).astype(np.float32)
    # decoders agree bit for bit
    for arr, dt in ((x, "bf16"), (W1, w), (W2, w)):
        np.testing.assert_array_equal(C.decode(arr, dt), O.decode(arr, dt))
    W1d = C.decode(W1, w) * (s1[:, :, None] if s1 is not None else 1.0)
    W2d = C.decode(W2, w) * (s2[:, :, None] if s2 is not None else 1.0)
    xd, wrd = C.decode(x, "bf16"), C.decode(wr, "bf16")
    # scores within one float32 rounding of each other (different summation orders)
    lc = C.router_logits(xd, wrd, rb)
    lo = O.router_logits(xd, wrd, rb)
    assert np.all(np.abs(lc.astype(np.float64) - lo) <= np.abs(lo) * 2.0 ** -23 + 1e-30)
    # same scores in: same indices, gates to float64 rounding, same permutation
    ic, gc = C.route(lo, K, sb, G, TG, renorm)
    io = O.select_experts(lo, K, sb, G, TG)
    np.testing.assert_array_equal(ic, io)
    np.testing.assert_allclose(gc, O.gate_weights(lo, io, renorm), rtol=1e-13, atol=1e-15)
    counts, offsets, perm, inv = C.permute(ic, E, 16)
    po = O.permute(io, E, 16)
    np.testing.assert_array_equal(counts, po["counts"])
    np.testing.assert_array_equal(perm, po["perm"])
    np.testing.assert_array_equal(inv, po["inv_perm"])
    # the whole layer
    yc, _, _ = C.layer_forward(xd, wrd, W1d, C.decode(b1, "bf16"), W2d, C.decode(b2, "bf16"), K=K,
                               select_bias=sb, n_groups=G, topk_groups=TG, renormalize=renorm, logits_in=lo)
    yo = O.layer_forward(x, wr, W1, b1, W2, b2, K=K, act="bf16", w=w, select_bias=sb, n_groups=G, topk_groups=TG,
                         renormalize=renorm, w1_scale=s1, w2_scale=s2, logits_in=lo)
    np.testing.assert_allclose(yc, yo, rtol=1e-11, atol=1e-11 * np.abs(yo).max())
