"""GPU parity of the fp8-activation (W8A8) path through the C ABI: the row
quantiser bit-exact against the oracle's, and the whole layer with e4m3
activations against the oracle's W8A8 layer on the GPU's own scores."""
import dataclasses

import numpy as np
import pytest
import torch

import datagen as D
import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, GATE_TOL, TOL, gpu_inputs, oracle_view, sample_tokens

pytestmark = pytest.mark.gpu


def sync():
    torch.cuda.synchronize()


def _bf16(a):
    """float32 numpy -> (bf16 device tensor, the bf16 values as float32)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.to(DEV), t.float().numpy()


# Row lengths on both sides of each register-block size of the quantiser
# (1024, 2048, 4096 and 8192 values held in registers; longer rows are read
# twice): 8-136 and 1024, 1032-2048, 4096, 7168-8192, then 8200 and 14336.
@pytest.mark.parametrize("rows,n,seed", [(1, 8, 0), (37, 64, 1), (300, 2048, 2), (64, 7168, 3), (16, 14336, 4),
                                         (1000, 136, 5), (12, 1024, 6), (9, 1032, 7), (40, 4096, 8),
                                         (5, 8192, 9), (3, 8200, 10)])
def test_quantize_rows_bit_exact(rows, n, seed):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal((rows, n)) * np.exp(rng.uniform(-20, 20, (rows, 1)))
    if rows > 3:
        v[1] = 0.0                          # zero row
        v[2, :] = -0.0
        v[3, ::3] = 0.0                     # zeros inside a row
        v[3, 1::3] *= -1
    src, vals = _bf16(v)
    print(f"quantize rows={rows} n={n}", flush=True)
    codes, scales = M.moe_quantize_rows(src)
    sync()
    o_codes, o_scales = O.quantize_rows_e4m3(vals)
    np.testing.assert_array_equal(scales.cpu().numpy(), o_scales)
    np.testing.assert_array_equal(codes.cpu().numpy(), o_codes)


def test_quantize_rows_ties_and_subnormals():
    """Rows whose products v * (448 / amax) land exactly on e4m3 midpoints
    and in the subnormal range: amax = 448 makes the factor 1."""
    mags = np.sort(O.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8)))
    mids = (mags[1:] + mags[:-1]) / 2
    vals = np.concatenate([mids, -mids, mags, -mags])
    vals = vals[np.abs(vals.astype(np.float32).astype(np.float64) - vals) == 0]   # exact in bf16 below
    n = 256
    rows = []
    for i in range(0, len(vals), n - 1):
        chunk = vals[i:i + n - 1]
        row = np.zeros(n)
        row[0] = 448.0
        row[1:1 + len(chunk)] = chunk
        rows.append(row)
    v = np.array(rows)
    src, bv = _bf16(v)
    keep = np.all(bv.astype(np.float64) == v, axis=1)          # rows that bf16 holds exactly
    codes, scales = M.moe_quantize_rows(src)
    sync()
    o_codes, o_scales = O.quantize_rows_e4m3(bv)
    assert keep.sum() >= 1
    np.testing.assert_array_equal(codes.cpu().numpy(), o_codes)
    np.testing.assert_array_equal(scales.cpu().numpy(), o_scales)


def test_quantize_rows_tiny_rows():
    """Rows whose 448 / amax overflows float32 (amax below about 1.3e-36,
    down to bf16 subnormals) against the oracle, codes and scales bit for
    bit: both scale such rows up by 2^64 first."""
    rng = np.random.default_rng(21)
    rows, n = 48, 264
    v = rng.standard_normal((rows, n)) * np.exp2(-rng.integers(112, 142, (rows, 1)).astype(np.float64))
    v[0] = 0.0
    v[1, :] = 2.0 ** -133 * np.arange(n)                    # bf16 subnormals and a zero
    v[2, ::2] = 0.0
    src, vals = _bf16(v)
    amax = np.abs(vals).max(axis=1)
    with np.errstate(divide="ignore", over="ignore"):
        assert np.sum(np.isinf(np.float32(448) / amax[1:])) >= 20   # most rows take the scaled-up path
    codes, scales = M.moe_quantize_rows(src)
    sync()
    o_codes, o_scales = O.quantize_rows_e4m3(vals)
    np.testing.assert_array_equal(scales.cpu().numpy(), o_scales)
    np.testing.assert_array_equal(codes.cpu().numpy(), o_codes)


def _layer_w8a8(cfg, inp, tokens, cap=0):
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, 1.0, cap, 1)
    logits = torch.empty((cfg.S, cfg.E), dtype=torch.float32, device=DEV)
    idx = torch.empty((cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    gate = torch.empty((cfg.S, cfg.K), dtype=torch.float32, device=DEV)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"],
                            topk_idx_out=idx, topk_gate_out=gate, logits_out=logits)
    sync()
    ov = oracle_view(inp)
    lg = logits.cpu().numpy()
    o_idx = O.select_experts(lg, cfg.K, ov["select_bias"], cfg.n_groups, cfg.topk_groups)
    if not cap:
        assert np.array_equal(idx.cpu().numpy(), o_idx)
    ref = O.layer_forward(ov["x"], ov["W_r"], ov["W1"], ov["b1"], ov["W2"], ov["b2"], K=cfg.K, act=cfg.act,
                          w=cfg.w, select_bias=ov["select_bias"], n_groups=cfg.n_groups,
                          topk_groups=cfg.topk_groups, renormalize=cfg.renormalize, w1_scale=ov["w1_scale"],
                          w2_scale=ov["w2_scale"], logits_in=lg, tokens=tokens, capacity=cap, act_quant=True,
                          return_parts=True)
    # routing from the GPU's own scores: indices exact, gates to GATE_TOL
    assert np.array_equal(idx.cpu().numpy()[tokens], ref["idx"])
    np.testing.assert_allclose(gate.cpu().numpy()[tokens], ref["gates"], rtol=0, atol=GATE_TOL)
    ref = ref["y"]
    yg = O.decode(raw(y[torch.from_numpy(np.asarray(tokens)).to(DEV)]), cfg.act)
    err = np.abs(yg - ref).max() / np.abs(ref).max()
    print(f"w8a8 {cfg.name} S={cfg.S} rel err {err:.3e}", flush=True)
    assert err <= TOL["fp8"], err
    return y


@pytest.mark.parametrize("S,E,K,seed,d,d_ff", [(2048, 8, 2, 0, 512, 768),    # 512 rows per expert: 128-row tiles
                                               (640, 16, 2, 1, 512, 768),    # 80 rows per expert
                                               (24, 8, 2, 2, 512, 768),      # decode: 16-row tiles, k % 256 == 0
                                               (333, 8, 3, 3, 512, 768),     # ragged groups
                                               (400, 8, 2, 4, 640, 384),     # 128-wide channel tiles
                                               (20, 8, 2, 5, 640, 384)])     # decode with k % 256 != 0
def test_layer_w8a8_small(S, E, K, seed, d, d_ff):
    base = D.CONFIGS["dsv3_fp8"]
    cfg = dataclasses.replace(base, name=f"w8a8_{S}_{E}", S=S, d=d, d_ff=d_ff, E=E, K=K, n_groups=1,
                              topk_groups=1, select_bias_var=0.0, seed=seed)
    inp = D.make_inputs(cfg, device=DEV)
    sync()
    _layer_w8a8(cfg, inp, np.arange(S) if S <= 400 else sample_tokens(S, 96, seed))


def test_layer_w8a8_dsv3_full_size():
    cfg = D.CONFIGS["dsv3_fp8"]
    inp = gpu_inputs("dsv3_fp8")
    y8 = _layer_w8a8(cfg, inp, sample_tokens(cfg.S, 8, seed=4))
    # and it stays close to the bf16-activation layer on the same inputs
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize)
    y16 = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                              inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"])
    sync()
    a, b = y8.float(), y16.float()
    assert float((a - b).abs().max()) <= TOL["fp8"] * float(b.abs().max())


@pytest.mark.parametrize("S,E,K,seed", [(2048, 8, 2, 0), (640, 16, 2, 1), (24, 8, 2, 2)])
def test_layer_w8a8_equals_its_stages(S, E, K, seed):
    """The W8A8 layer quantises each token's row once and its up product
    reads those codes in place; the stage entry points gather x per (token,
    slot) pair and quantise the gathered rows.  Both compute the same codes
    and the same products, so the outputs agree bit for bit (prefill, mid
    and decode tiles)."""
    base = D.CONFIGS["dsv3_fp8"]
    cfg = dataclasses.replace(base, name=f"w8a8_st_{S}", S=S, d=512, d_ff=768, E=E, K=K, n_groups=1,
                              topk_groups=1, select_bias_var=0.0, router_offset="normal", offset_beta=0.5, seed=seed)
    inp = D.make_inputs(cfg, device=DEV)
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, 1.0, 0, 1)
    # routing, dispatch and combine of the stage path on the same problem
    # with bf16 activations (moe_permute refuses act_quant = 1)
    p0 = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                        cfg.renormalize)
    assert M.moe_tile_m(p0) == M.moe_tile_m(p)
    y = M.moe_layer_forward(p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"],
                            inp["router_bias"], inp["select_bias"], inp["w1_scale"], inp["w2_scale"])
    idx, gate = M.moe_route(p0, inp["x"], inp["W_r"], inp["router_bias"], inp["select_bias"])
    counts, offsets, perm, inv, x_perm = M.moe_permute(p0, idx, inp["x"])
    x8, xs = M.moe_quantize_rows(x_perm)
    h = M.moe_expert_up_a8(p, x8, xs, counts, offsets, inp["W1"], inp["b1"], inp["w1_scale"])
    h8, hs = M.moe_quantize_rows(h)
    y_perm = M.moe_expert_down_a8(p, h8, hs, counts, offsets, inp["W2"], inp["b2"], inp["w2_scale"])
    y2 = M.moe_combine(p0, y_perm, inv, gate)
    sync()
    print(f"w8a8 layer vs stages S={S}: regime tile {M.moe_tile_m(p)}", flush=True)
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


def test_layer_w8a8_deterministic():
    cfg = D.CONFIGS["dsv3_fp8"]
    inp = gpu_inputs("dsv3_fp8")
    p = M.make_problem(cfg.S, cfg.d, cfg.d_ff, cfg.E, cfg.K, cfg.act, cfg.w, cfg.n_groups, cfg.topk_groups,
                       cfg.renormalize, 1.0, 0, 1)
    args = (p, inp["x"], inp["W_r"], inp["W1"], inp["b1"], inp["W2"], inp["b2"], inp["router_bias"],
            inp["select_bias"], inp["w1_scale"], inp["w2_scale"])
    y1 = M.moe_layer_forward(*args)
    y2 = M.moe_layer_forward(*args)
    sync()
    assert torch.equal(y1, y2)


def test_layer_w8a8_with_capacity():
    """fp8 activations and a per-expert capacity together: the capacity
    decides the routing, the W8A8 products run on the kept pairs."""
    base = D.CONFIGS["dsv3_fp8"]
    cfg = dataclasses.replace(base, name="w8a8_cap", S=640, d=512, d_ff=768, E=16, K=2, n_groups=1, topk_groups=1,
                              select_bias_var=0.0, router_offset="normal", offset_beta=1.0, seed=7)
    inp = D.make_inputs(cfg, device=DEV)
    sync()
    _layer_w8a8(cfg, inp, np.arange(0, cfg.S, 3), cap=60)
