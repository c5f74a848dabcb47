"""Pins of the oracle's fp8 activation path (W8A8).

FP8 E4M3 is the production format the pages name for experts ("MoE 推理工程
深层实战" section 3.3); with fp8 activations both operands of each expert
product are e4m3.  The encoder is pinned against torch's float8_e4m3fn
conversion (a library routine the oracle does not use) and the format's own
round trip; the per-row quantiser by closed forms (the row maximum lands on
448, power-of-two scaling, the half-spacing error bound); the W8A8 expert by
the special case where quantisation is exact.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _torch_codes(v):
    return torch.from_numpy(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encoder_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = O.decode_e4m3fn(codes).astype(np.float32)
    np.testing.assert_array_equal(O.encode_e4m3fn(vals), codes)


def test_encoder_matches_torch_on_grid_and_every_tie():
    grid = np.linspace(-448.0, 448.0, 400001).astype(np.float32)
    np.testing.assert_array_equal(O.encode_e4m3fn(grid), _torch_codes(grid))
    mags = np.sort(O.decode_e4m3fn(np.arange(0x7F, dtype=np.uint8)))
    mids = ((mags[1:] + mags[:-1]) / 2).astype(np.float32)       # exact in float32
    assert np.all(mids.astype(np.float64) == (mags[1:] + mags[:-1]) / 2)
    for v in (mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))):
        v = np.clip(v, -448, 448).astype(np.float32)
        np.testing.assert_array_equal(O.encode_e4m3fn(v), _torch_codes(v))
    tiny = np.array([0.0, -0.0, 2.0 ** -10, -2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11, 2.0 ** -9], np.float32)
    np.testing.assert_array_equal(O.encode_e4m3fn(tiny), _torch_codes(tiny))


def test_encoder_hand_values():
    # 1.0 = 0 0111 000; 448 = 0 1111 110; 2^-9 = smallest subnormal 0 0000 001;
    # 1.0625 is the tie between 1.0 (even mantissa 000) and 1.125 -> 1.0;
    # 1.1875 is the tie between 1.125 (001) and 1.25 (010) -> 1.25
    v = np.array([1.0, 448.0, 2.0 ** -9, 1.0625, 1.1875, -2.0, -0.0], np.float32)
    np.testing.assert_array_equal(O.encode_e4m3fn(v), [0x38, 0x7E, 0x01, 0x38, 0x3A, 0xC0, 0x80])
    with pytest.raises(ValueError):
        O.encode_e4m3fn(np.array([449.0], np.float32))


def test_quantize_rows_closed_forms():
    rng = np.random.default_rng(3)
    v = (rng.standard_normal((50, 300)) * np.exp(rng.uniform(-8, 8, (50, 1)))).astype(np.float32)
    v[7] = 0.0
    q, s = O.quantize_rows_e4m3(v)
    amax = np.abs(v).max(axis=1)
    # the scale is the float32 quotient amax / 448; a zero row has scale 0, codes 0
    np.testing.assert_array_equal(s, (amax / np.float32(448)).astype(np.float32))
    assert s[7] == 0 and np.all(q[7] == 0)
    # the row maximum lands on 448 (code 0x7E, or 0xFE when negative)
    for r in range(50):
        if r == 7:
            continue
        j = int(np.argmax(np.abs(v[r])))
        assert q[r, j] & 0x7F == 0x7E
    # error bound: half the spacing of the e4m3 grid, relative 2^-4 for
    # normals and 2^-10 * s in the subnormal range (plus the float32 quotient)
    deq = O.dequantize_rows_e4m3(q, s)
    err = np.abs(deq - v.astype(np.float64))
    bound = (2.0 ** -4 * np.abs(v) + 2.0 ** -10 * s[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # power-of-two scaling changes the scale and nothing else
    q2, s2 = O.quantize_rows_e4m3((v * np.float32(2.0 ** 5)).astype(np.float32))
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, (s * np.float32(32)).astype(np.float32))


def test_quantize_rows_tiny_rows_are_power_of_two_copies():
    """Rows whose 448 / amax overflows float32 (amax below about 1.3e-36)
    get the codes of the same row scaled up by a power of two, and the
    scale amax / 448 (subnormal here) as one float32 quotient.  Elements
    are bf16 values (8 significant bits) in [2^-8, 1], so every scaled value
    down to 2^-133 is still exact in float32 (subnormal spacing 2^-149)."""
    rng = np.random.default_rng(11)
    v = (np.sign(rng.standard_normal((6, 40))) * np.exp2(rng.uniform(-8, 0, (6, 40)))).astype(np.float32)
    v = (v.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)   # truncate to bf16 values
    v[:, 0] = 1.0                                  # amax = 1 in every row
    q, _ = O.quantize_rows_e4m3(v)
    for k in (118, 119, 120, 125):                 # 448 * 2^119 < FLT_MAX < 448 * 2^120
        vs = (v * np.float32(2.0 ** -k)).astype(np.float32)
        assert np.all(vs.astype(np.float64) == v.astype(np.float64) * 2.0 ** -k)
        with np.errstate(over="ignore"):
            assert np.isinf(np.float32(448) / np.float32(2.0 ** -k)) == (k >= 120)
        qs, ss = O.quantize_rows_e4m3(vs)
        np.testing.assert_array_equal(qs, q)
        np.testing.assert_array_equal(ss, np.full(6, np.float32(2.0 ** -k) / np.float32(448), np.float32))
    # float32 subnormal inputs: the largest lands on 448 (0x7E), half of it
    # on -224 (0xF6), a zero stays 0, and 3/32 of it, 42, is the tie
    # between 40 (0x62) and 44 (0x63) that goes to the even code
    sub = np.array([[2.0 ** -140, -(2.0 ** -141), 0.0, 3 * 2.0 ** -145]], np.float32)
    qs, ss = O.quantize_rows_e4m3(sub)
    np.testing.assert_array_equal(qs[0], [0x7E, 0xF6, 0x00, 0x62])
    assert ss[0] == np.float32(np.float32(2.0 ** -140) / np.float32(448))


def test_quantize_rows_against_torch_conversion():
    rng = np.random.default_rng(5)
    v = rng.standard_normal((20, 64)).astype(np.float32)
    q, s = O.quantize_rows_e4m3(v)
    t = torch.from_numpy(v)
    st = t.abs().amax(dim=1) / 448.0
    rt = 448.0 / t.abs().amax(dim=1)
    qt = (t * rt[:, None]).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(s, st.numpy())
    np.testing.assert_array_equal(q, qt)


def test_w8a8_expert_exact_when_activations_are_on_the_grid():
    """x rows made of e4m3 values times 2^j with the row maximum 448 * 2^j
    quantise exactly, so the first product equals the unquantised one."""
    rng = np.random.default_rng(8)
    d, d_ff, n = 32, 48, 6
    codes = rng.integers(0, 0x7F, size=(n, d)).astype(np.uint8) | (rng.integers(0, 2, (n, d)) * 0x80).astype(np.uint8)
    codes[:, 0] = 0x7E
    x = (O.decode_e4m3fn(codes) * (2.0 ** rng.integers(-6, 6, (n, 1)))).astype(np.float32)
    w1 = rng.standard_normal((d_ff, d)) / 5
    b1 = rng.standard_normal(d_ff) / 10
    w2 = rng.standard_normal((d, d_ff)) / 7
    b2 = rng.standard_normal(d) / 10
    h8, _ = O.expert_ffn_w8a8(x.astype(np.float64), w1, b1, w2, b2, return_hidden=True)
    h, _ = O.expert_ffn(x.astype(np.float64), w1, b1, w2, b2, return_hidden=True)
    np.testing.assert_array_equal(h8, h)


def test_w8a8_expert_against_loops_with_torch_quantiser():
    """A per-element loop (math.erf, fsum) over activations quantised with
    torch's e4m3 conversion."""
    rng = np.random.default_rng(9)
    d, d_ff, n = 8, 12, 3
    x = rng.standard_normal((n, d)).astype(np.float32)
    w1 = rng.standard_normal((d_ff, d)) / 3
    b1 = rng.standard_normal(d_ff) / 10
    w2 = rng.standard_normal((d, d_ff)) / 3
    b2 = rng.standard_normal(d) / 10

    def tq(row):
        t = torch.from_numpy(np.asarray(row, np.float32))
        sc = t.abs().max() / 448.0
        q = (t * (448.0 / t.abs().max())).clamp(-448, 448).to(torch.float8_e4m3fn).to(torch.float64)
        return (q * sc.double()).numpy()

    y = O.expert_ffn_w8a8(x.astype(np.float64), w1, b1, w2, b2)
    for r in range(n):
        xq = tq(x[r])
        h = [0.0] * d_ff
        for j in range(d_ff):
            a = math.fsum(xq[k] * w1[j, k] for k in range(d)) + b1[j]
            h[j] = 0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0)))
        hq = tq(np.array(h, np.float32))
        for i in range(d):
            ref = math.fsum(hq[j] * w2[i, j] for j in range(d_ff)) + b2[i]
            assert abs(y[r, i] - ref) <= 1e-12 * (1 + abs(ref))


def test_w8a8_layer_close_to_w8a16_layer():
    """fp8 activations move the tiny layer by a few per cent of max|y| at
    most (each activation moves by at most 2^-4 of itself)."""
    rng = np.random.default_rng(10)
    S, d, d_ff, E, K = 16, 64, 96, 4, 2
    x = rng.standard_normal((S, d)).astype(np.float32)
    wr = rng.standard_normal((E, d)).astype(np.float32)
    w1 = (rng.standard_normal((E, d_ff, d)) / 8).astype(np.float32)
    b1 = (rng.standard_normal((E, d_ff)) / 10).astype(np.float32)
    w2 = (rng.standard_normal((E, d, d_ff)) / 10).astype(np.float32)
    b2 = (rng.standard_normal((E, d)) / 10).astype(np.float32)
    y = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32")
    y8 = O.layer_forward(x, wr, w1, b1, w2, b2, K=K, act="f32", w="f32", act_quant=True)
    rel = np.abs(y8 - y).max() / np.abs(y).max()
    assert 0 < rel < 6e-2
