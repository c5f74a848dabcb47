"""The 256 x 256 bf16 prefill tiles at every fill level of their wave rows.

An expert's rows are dealt to its row tiles in 32-row fragments (balanced
row tiles), and each of a tile's two wave rows of 128 rows holds 0-4 valid
fragments; the kernel runs one copy of its k loop for 4, 2 and 1 valid
fragments (3 runs the copy for 4, 0 the copy for 1).  The expert sizes here
put the wave rows on every count and on both sides of each 32-row edge
(31, 32, 33, ..., 255, 256, 257), with empty experts between, and enough
rows per expert on average for the 256-row regime.  Every valid row of h
and y_perm is compared with the oracle's expert FFN (P2 §11.1.2 expert
formula), with the split-K workspace (the down product has 16 k-tiles, so
its partly filled last round is split) and without it; the padding rows of
both outputs must keep the sentinel they were filled with."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_ffn_layer_amd as M
from tests._util import raw
from tests.gpu_common import DEV, act_from_raw

pytestmark = pytest.mark.gpu

COUNTS = [1, 31, 32, 33, 0, 64, 65, 96, 97, 100, 128, 129, 160, 161, 192, 193, 224, 225, 255, 256, 257, 300,
          0, 600, 1000, 3000]
D_MODEL, D_FF = 512, 1024
SENTINEL = 0x7FC0  # a bf16 NaN: never a result of the products


def _bf16_bits(rng, shape, scale):
    """Seeded normal values cut to bf16 (the top 16 bits of their float32)."""
    v = (rng.standard_normal(shape) * scale).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


def _filled(rows, cols):
    return torch.full((rows, cols), SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)


@pytest.mark.parametrize("split", [True, False])
def test_prefill_tiles_every_fill_level(split):
    E, S = len(COUNTS), sum(COUNTS)
    p = M.make_problem(S, D_MODEL, D_FF, E, 1, "bf16", "bf16")
    tile = M.moe_tile_m(p)
    assert tile == 256, tile  # the 256-row regime (rows per expert >= 256 on average)
    cap = M.moe_rows_capacity(p)
    offs = np.zeros(E + 1, dtype=np.int64)
    for e, c in enumerate(COUNTS):
        offs[e + 1] = offs[e] + -(-c // tile) * tile
    assert offs[-1] <= cap
    rng = np.random.default_rng(20260)
    xb = _bf16_bits(rng, (cap, D_MODEL), 1.0)  # rows past an expert's count are never read
    W1 = _bf16_bits(rng, (E, D_FF, D_MODEL), D_MODEL ** -0.5)
    b1 = _bf16_bits(rng, (E, D_FF), 0.1)
    W2 = _bf16_bits(rng, (E, D_MODEL, D_FF), D_FF ** -0.5)
    b2 = _bf16_bits(rng, (E, D_MODEL), 0.1)
    counts_t = torch.tensor(COUNTS, dtype=torch.int32, device=DEV)
    offs_t = torch.from_numpy(offs.astype(np.int32)).to(DEV)
    ws = None if split else torch.empty(1, dtype=torch.uint8, device=DEV)
    h = _filled(cap, D_FF)
    y = _filled(cap, D_MODEL)
    print(f"prefill tile fill levels: S={S} E={E} split={split} cap={cap}", flush=True)
    M.moe_expert_up(p, act_from_raw(xb, "bf16"), counts_t, offs_t, act_from_raw(W1, "bf16"),
                    act_from_raw(b1, "bf16"), None, h=h, ws=ws)
    M.moe_expert_down(p, h, counts_t, offs_t, act_from_raw(W2, "bf16"), act_from_raw(b2, "bf16"), None,
                      y_perm=y, ws=ws)
    torch.cuda.synchronize()
    hb, yb = raw(h), raw(y)

    valid = np.zeros(cap, dtype=bool)
    for e, c in enumerate(COUNTS):
        valid[offs[e]:offs[e] + c] = True
    assert np.all(hb[~valid] == SENTINEL) and np.all(yb[~valid] == SENTINEL)

    hmax = ymax = herr = yerr = 0.0
    for e, c in enumerate(COUNTS):
        if c == 0:
            continue
        r = slice(offs[e], offs[e] + c)
        hr, yr = O.expert_ffn(O.decode(xb[r], "bf16"), O.expert_matrix(W1[e], "bf16"), O.decode(b1[e], "bf16"),
                              O.expert_matrix(W2[e], "bf16"), O.decode(b2[e], "bf16"), return_hidden=True)
        hg, yg = O.decode(hb[r], "bf16"), O.decode(yb[r], "bf16")
        # h: one bf16 rounding (half a spacing, 2^-8 relative) of a float32
        # sum over 512 products, whose error stays far below 2e-4 max|h|
        hm = np.abs(hr).max()
        assert np.all(np.abs(hg - hr) <= 2.0 ** -8 * np.abs(hr) + 2e-4 * hm), (e, c)
        herr, hmax = max(herr, np.abs(hg - hr).max()), max(hmax, hm)
        yerr, ymax = max(yerr, np.abs(yg - yr).max()), max(ymax, np.abs(yr).max())
    # y: its products read the bf16 h, the oracle's the exact one
    assert yerr <= 6e-3 * ymax, (yerr, ymax)
    assert herr <= 2.0 ** -8 * hmax + 2e-4 * hmax, (herr, hmax)
