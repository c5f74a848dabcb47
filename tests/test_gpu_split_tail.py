"""The general grouped GEMM's split-K tail at the sizes that take it.

A persistent launch runs the tile space in rounds; when the last round of an
XCD's slice is partly empty, its tail tiles run split along k over the idle
workgroups (float32 partial sums, added in slice order by a second kernel).
That needs K / BK >= 16 k-tiles, so among the five workloads only the
DeepSeek shape (fp8 weights, 128-row tiles) reaches it in the general kernel.
These tests compare, against the oracle, every row of every expert that owns
a split tile, plus experts spread over the index range, and the split result
against the unsplit one (no workspace) on every valid row."""
import dataclasses

import numpy as np
import pytest
import torch

import datagen as D
import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import (DEV, GATE_TOL, TOL, act_from_raw, gpu_inputs, host_x_perm, oracle_logits,
                              oracle_select, oracle_view, problem, split_tail_tiles, tol_of)

pytestmark = pytest.mark.gpu

# Tile shape (BM, BN, BK, GM) of the general kernel for 64-255 rows per
# expert and a contraction of K: 128 x 256 tiles in expert-aligned bands of up
# to 4 row tiles (GM = -4); k stages of 64 with bf16 weights, of 128 with fp8
# weights when K % 128 == 0 (and always with e4m3 activations).
BM = 128


def tile_shape(w, K, a8=False):
    fp8_k128 = a8 or (w == "fp8" and K % 128 == 0)
    return BM, 256, 128 if fp8_k128 else 64, -4


def split_tails(cfg, offsets, cap, a8=False):
    """Split tail tiles of (the up product, the down product)."""
    _, BN, BKu, GM = tile_shape(cfg.w, cfg.d, a8)
    BKd = tile_shape(cfg.w, cfg.d_ff, a8)[2]
    return (split_tail_tiles(offsets, cap, cfg.d_ff, cfg.d, BM, BN, BKu, GM),
            split_tail_tiles(offsets, cap, cfg.d, cfg.d_ff, BM, BN, BKd, GM))


def sync():
    torch.cuda.synchronize()


def valid_rows(counts, offsets):
    return np.concatenate([np.arange(offsets[e], offsets[e] + counts[e]) for e in range(len(counts))])


def _split_vs_plain(a, b, rows):
    """a (split) and b (unsplit) on the valid rows: the same float32 products
    summed in a different grouping, each rounded once to bf16."""
    vi = torch.from_numpy(rows).to(DEV)
    x, y = a[vi].float(), b[vi].float()
    err = (x - y).abs().max().item()
    scale = y.abs().max().item()
    assert err <= 2 ** -7 * scale, (err, scale)
    return err / scale


def _oracle_rows(cfg, ov, pm, idx, experts, h, y_perm, ffn=O.expert_ffn):
    """Every routed row of `experts`: h and y_perm against the oracle's expert
    FFN (y_perm computed by the GPU from its own h)."""
    flat_e = idx.reshape(-1)
    flat_t = np.arange(cfg.S * cfg.K) // cfg.K
    herr = hmax = yerr = ymax = 0.0
    n = 0
    for e in sorted(set(int(v) for v in experts)):
        ps = np.flatnonzero(flat_e == e)
        if ps.size == 0:
            continue
        x64 = O.decode(ov["x"][flat_t[ps]], cfg.act)
        W1e = O.expert_matrix(ov["W1"][e], cfg.w, None if ov["w1_scale"] is None else ov["w1_scale"][e])
        W2e = O.expert_matrix(ov["W2"][e], cfg.w, None if ov["w2_scale"] is None else ov["w2_scale"][e])
        hr, yr = ffn(x64, W1e, O.decode(ov["b1"][e], cfg.act), W2e, O.decode(ov["b2"][e], cfg.act),
                     return_hidden=True)
        rows = torch.from_numpy(pm["inv_perm"][ps].astype(np.int64)).to(DEV)
        hg = O.decode(raw(h[rows]), cfg.act)
        yg = O.decode(raw(y_perm[rows]), cfg.act)
        herr, hmax = max(herr, np.abs(hg - hr).max()), max(hmax, np.abs(hr).max())
        yerr, ymax = max(yerr, np.abs(yg - yr).max()), max(ymax, np.abs(yr).max())
        n += ps.size
    t = tol_of(cfg)
    assert herr <= t * hmax, (herr, hmax)
    assert yerr <= t * ymax, (yerr, ymax)
    return n


def _products(cfg, inp, ov):
    p = problem(cfg)
    tm = M.moe_tile_m(p)
    assert tm == BM
    idx, _ = oracle_select(cfg, oracle_logits(cfg, ov), ov)
    pm = O.permute(idx, cfg.E, tm)
    cap = M.moe_rows_capacity(p)
    x_perm = act_from_raw(host_x_perm(cfg, ov["x"], pm, cap), cfg.act)
    counts = torch.from_numpy(pm["counts"]).to(DEV)
    offsets = torch.from_numpy(pm["offsets"]).to(DEV)
    none = torch.empty(1, dtype=torch.uint8, device=DEV)
    h = M.moe_expert_up(p, x_perm, counts, offsets, inp["W1"], inp["b1"], inp["w1_scale"])
    h2 = M.moe_expert_up(p, x_perm, counts, offsets, inp["W1"], inp["b1"], inp["w1_scale"])
    h0 = M.moe_expert_up(p, x_perm, counts, offsets, inp["W1"], inp["b1"], inp["w1_scale"], ws=none)
    y = M.moe_expert_down(p, h, counts, offsets, inp["W2"], inp["b2"], inp["w2_scale"])
    y2 = M.moe_expert_down(p, h, counts, offsets, inp["W2"], inp["b2"], inp["w2_scale"])
    y0 = M.moe_expert_down(p, h, counts, offsets, inp["W2"], inp["b2"], inp["w2_scale"], ws=none)
    sync()
    rows = valid_rows(pm["counts"], pm["offsets"])
    vi = torch.from_numpy(rows).to(DEV)
    # deterministic on the valid rows (padding rows are never written)
    assert torch.equal(h[vi], h2[vi]) and torch.equal(y[vi], y2[vi])
    _split_vs_plain(h, h0, rows)
    _split_vs_plain(y, y0, rows)
    return idx, pm, h, y, split_tails(cfg, pm["offsets"], cap)


def test_dsv3_w8a16_split_tail_experts_every_row():
    """DeepSeek shape, fp8 weights and bf16 activations (S=4096, d=7168,
    d_ff=2048, E=256, K=8): both expert products with the split tail (the
    default workspace) against the unsplit launch on every valid row, and
    every routed row of every expert (the split tiles' owners among them)
    against the oracle."""
    cfg = D.CONFIGS["dsv3_fp8"]
    inp = gpu_inputs("dsv3_fp8")
    ov = oracle_view(inp)
    print("dsv3 W8A16 products, split vs unsplit", flush=True)
    idx, pm, h, y, (up_tails, down_tails) = _products(cfg, inp, ov)
    tails = up_tails + down_tails
    assert up_tails, "the DeepSeek shape's up product has split tail tiles"
    owners = sorted(set(e for _, _, e in tails))
    print(f"split tiles {len(tails)}, owned by experts {owners}", flush=True)
    n = _oracle_rows(cfg, ov, pm, idx, range(cfg.E), h, y)
    print(f"compared {n} routed rows of {cfg.E} experts", flush=True)
    assert n == cfg.S * cfg.K


@pytest.mark.parametrize("w", ["bf16", "fp8"])
def test_mid_regime_split_tail_all_rows(w):
    """128-row tiles with k = 2048 (32 k-tiles of 64) at a size the oracle
    covers whole, with split tail tiles in both products: every valid row of
    both products against the oracle, and split against unsplit."""
    cfg = D.MoEConfig(f"mid_{w}", S=1700, d=2048, d_ff=2048, E=16, K=2, w=w, router_offset="normal",
                      offset_beta=0.3, seed=11)
    inp = D.make_inputs(cfg, DEV)
    ov = oracle_view(inp)
    print(f"mid regime {w}: split vs unsplit, all rows", flush=True)
    idx, pm, h, y, (up_tails, down_tails) = _products(cfg, inp, ov)
    assert up_tails and down_tails, "this shape has split tail tiles in both products"
    n = _oracle_rows(cfg, ov, pm, idx, range(cfg.E), h, y)
    assert n == cfg.S * cfg.K


def _w8a8_layer(cfg, inp, tokens):
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, 1.0, 0, 1)
    logits = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.S, cfg.K), dtype=torch.float32, device=DEV)
    counts = torch.empty(cfg.E, dtype=torch.int32, device=DEV)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"],
                            topk_idx_out=idx, topk_gate_out=gate, logits_out=logits, expert_counts_out=counts)
    sync()
    return p, y, idx.cpu().numpy(), gate.cpu().numpy(), logits.cpu().numpy(), counts.cpu().numpy()


def _w8a8_check(cfg, inp, tokens, y, idx, gate, lg):
    ov = oracle_view(inp)
    ref = O.layer_forward(ov["x"], ov["W_r"], ov["W1"], ov["b1"], ov["W2"], ov["b2"], K=cfg.K, act=cfg.act,
                          w=cfg.w, select_bias=ov["select_bias"], n_groups=cfg.n_groups,
                          topk_groups=cfg.topk_groups, renormalize=cfg.renormalize, w1_scale=ov["w1_scale"],
                          w2_scale=ov["w2_scale"], logits_in=lg, tokens=tokens, act_quant=True,
                          return_parts=True)
    assert np.array_equal(idx[tokens], ref["idx"])
    np.testing.assert_allclose(gate[tokens], ref["gates"], rtol=0, atol=GATE_TOL)
    yg = O.decode(raw(y[torch.from_numpy(np.asarray(tokens)).to(DEV)]), cfg.act)
    err = np.abs(yg - ref["y"]).max() / np.abs(ref["y"]).max()
    print(f"w8a8 {cfg.name}: {len(tokens)} tokens, rel err {err:.3e}", flush=True)
    assert err <= TOL["fp8"], err


def test_w8a8_mid_regime_split_tail_all_tokens():
    """fp8 activations on 128-row tiles with BK = 128 and k = 2048 (16
    k-tiles) in both products, so both run the split tail: every token of the
    layer against the oracle's W8A8 layer on the GPU's own scores."""
    base = D.CONFIGS["dsv3_fp8"]
    cfg = dataclasses.replace(base, name="w8a8_mid", S=1700, d=2048, d_ff=2048, E=16, K=2, n_groups=1,
                              topk_groups=1, select_bias_var=0.0, router_offset="normal", offset_beta=0.3,
                              seed=11)
    inp = D.make_inputs(cfg, device=DEV)
    p, y, idx, gate, lg, counts = _w8a8_layer(cfg, inp, None)
    assert M.moe_tile_m(p) == BM
    offs = np.concatenate([[0], np.cumsum(-(-counts // BM) * BM)])
    up_tails, down_tails = split_tails(cfg, offs, M.moe_rows_capacity(p), a8=True)
    assert up_tails, "split tail tiles in the up product"
    assert down_tails, "split tail tiles in the down product"
    _w8a8_check(cfg, inp, np.arange(cfg.S), y, idx, gate, lg)


def test_w8a8_dsv3_split_tail_tokens():
    """DeepSeek shape with fp8 activations: 64 tokens, 40 of them routed to
    experts that own a split tail tile, the rest spread over the batch,
    against the oracle's W8A8 layer on the GPU's own scores."""
    cfg = D.CONFIGS["dsv3_fp8"]
    inp = gpu_inputs("dsv3_fp8")
    p, y, idx, gate, lg, counts = _w8a8_layer(cfg, inp, None)
    offs = np.concatenate([[0], np.cumsum(-(-counts // BM) * BM)])
    up_tails, down_tails = split_tails(cfg, offs, M.moe_rows_capacity(p), a8=True)
    tails = up_tails + down_tails
    assert tails
    owners = sorted(set(e for _, _, e in tails))
    rng = np.random.default_rng(5)
    hit = np.flatnonzero(np.isin(idx, owners).any(axis=1))
    picked = rng.choice(hit, min(40, hit.size), replace=False)
    rest = np.setdiff1d(np.linspace(0, cfg.S - 1, 24).astype(np.int64), picked)
    tokens = np.unique(np.concatenate([picked, rest, [cfg.S - 1]]))
    print(f"w8a8 dsv3: split tiles {len(tails)} owned by {len(owners)} experts; {tokens.size} tokens", flush=True)
    _w8a8_check(cfg, inp, tokens, y, idx, gate, lg)


def test_dsv3_w8a8_products_split_tail_experts_every_row():
    """The W8A8 stage entry points at the DeepSeek shape: x_perm quantised
    per row, the up product with the split tail against the unsplit launch on
    every valid row, h quantised per row, the same for the down product; and
    every routed row of every expert (the split tiles' owners among them)
    against the oracle's W8A8 expert FFN."""
    cfg = D.CONFIGS["dsv3_fp8"]
    inp = gpu_inputs("dsv3_fp8")
    ov = oracle_view(inp)
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, 1.0, 0, 1)
    assert M.moe_tile_m(p) == BM
    idx, _ = oracle_select(cfg, oracle_logits(cfg, ov), ov)
    pm = O.permute(idx, cfg.E, BM)
    cap = M.moe_rows_capacity(p)
    x_perm = act_from_raw(host_x_perm(cfg, ov["x"], pm, cap), cfg.act)
    counts = torch.from_numpy(pm["counts"]).to(DEV)
    offsets = torch.from_numpy(pm["offsets"]).to(DEV)
    none = torch.empty(1, dtype=torch.uint8, device=DEV)
    print("dsv3 W8A8 products, split vs unsplit", flush=True)
    x8, xs = M.moe_quantize_rows(x_perm)
    hz = lambda: torch.zeros((cap, cfg.d_ff), dtype=torch.bfloat16, device=DEV)   # padding rows stay 0
    up = lambda ws=None: M.moe_expert_up_a8(p, x8, xs, counts, offsets, inp["W1"], inp["b1"], inp["w1_scale"],
                                            h=hz(), ws=ws)
    h, h2, h0 = up(), up(), up(none)
    h8, hs = M.moe_quantize_rows(h)
    down = lambda ws=None: M.moe_expert_down_a8(p, h8, hs, counts, offsets, inp["W2"], inp["b2"],
                                                inp["w2_scale"], ws=ws)
    y, y2, y0 = down(), down(), down(none)
    sync()
    rows = valid_rows(pm["counts"], pm["offsets"])
    vi = torch.from_numpy(rows).to(DEV)
    assert torch.equal(h[vi], h2[vi]) and torch.equal(y[vi], y2[vi])
    _split_vs_plain(h, h0, rows)
    _split_vs_plain(y, y0, rows)
    up_tails, down_tails = split_tails(cfg, pm["offsets"], cap, a8=True)
    assert up_tails
    owners = sorted(set(e for _, _, e in up_tails + down_tails))
    print(f"split tiles {len(up_tails)} + {len(down_tails)}, owned by experts {owners}", flush=True)
    n = _oracle_rows(cfg, ov, pm, idx, range(cfg.E), h, y, ffn=O.expert_ffn_w8a8)
    print(f"compared {n} routed rows of {cfg.E} experts", flush=True)
    assert n == cfg.S * cfg.K
