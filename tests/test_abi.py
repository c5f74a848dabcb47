"""The C-ABI library without a GPU: it loads, exports every symbol declared in
include/moe.h, matches the header's struct layout, and rejects invalid
arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

import sparse_ffn_layer_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH), reason="library not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 17, names
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", M.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(l.split()[-1] for l in nm.splitlines() if " T " in l)
    assert set(names) <= exported


def test_struct_layout_matches_header():
    code = r'''
#include <stddef.h>
#include <stdio.h>
#include "moe.h"
int main(void) {
  printf("%zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu %zu\n", sizeof(moe_problem),
    offsetof(moe_problem, S), offsetof(moe_problem, d), offsetof(moe_problem, d_ff),
    offsetof(moe_problem, E), offsetof(moe_problem, K), offsetof(moe_problem, n_groups),
    offsetof(moe_problem, topk_groups), offsetof(moe_problem, renormalize),
    offsetof(moe_problem, act_dtype), offsetof(moe_problem, w_dtype), offsetof(moe_problem, gate_temperature),
    offsetof(moe_problem, capacity), offsetof(moe_problem, act_quant));
  return 0;
}'''
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "t.c"), os.path.join(d, "t")
        open(c, "w").write(code)
        subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), c, "-o", exe], check=True)
        vals = [int(v) for v in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    P = M.moe_problem
    mine = [ctypes.sizeof(P)] + [getattr(P, f).offset for f, _ in P._fields_]
    assert vals == mine


def prob(**kw):
    base = dict(S=64, d=128, d_ff=256, E=8, K=2, act="bf16", w="bf16")
    base.update(kw)
    return M.make_problem(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(K=9), M.MOE_ERR_INVALID_ARG),
    (dict(K=0), M.MOE_ERR_INVALID_ARG),
    (dict(E=0), M.MOE_ERR_INVALID_ARG),
    (dict(S=-1), M.MOE_ERR_INVALID_ARG),
    (dict(renormalize=2), M.MOE_ERR_INVALID_ARG),
    (dict(capacity=-1), M.MOE_ERR_INVALID_ARG),
    (dict(act_quant=2), M.MOE_ERR_INVALID_ARG),
    (dict(act_quant=1), M.MOE_ERR_UNSUPPORTED),                       # bf16 weights
    (dict(act_quant=1, w="fp8", d=192), M.MOE_ERR_UNSUPPORTED),       # d not a multiple of 128
    (dict(act_quant=1, act="f32", w="f32"), M.MOE_ERR_UNSUPPORTED),
    (dict(E=12, n_groups=4, topk_groups=2), M.MOE_ERR_INVALID_ARG),   # group of 3: not a power of 2
    (dict(E=16, n_groups=3, topk_groups=1), M.MOE_ERR_INVALID_ARG),   # 16 % 3
    (dict(E=16, n_groups=4, topk_groups=0), M.MOE_ERR_INVALID_ARG),
    (dict(E=16, n_groups=4, topk_groups=5), M.MOE_ERR_INVALID_ARG),
    (dict(E=16, n_groups=4, topk_groups=1, K=5), M.MOE_ERR_INVALID_ARG),  # K > 1 group of 4
    (dict(act="f32", w="bf16"), M.MOE_ERR_UNSUPPORTED),
    (dict(act="bf16", w="f32"), M.MOE_ERR_UNSUPPORTED),
    (dict(act="f32", w="fp8"), M.MOE_ERR_UNSUPPORTED),
    (dict(d=100), M.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=96), M.MOE_ERR_UNSUPPORTED),
    (dict(E=1024, K=2), M.MOE_ERR_UNSUPPORTED),
    (dict(E=128, K=65), M.MOE_ERR_UNSUPPORTED),
    (dict(E=256, n_groups=128, topk_groups=2), M.MOE_ERR_UNSUPPORTED),
])
def test_invalid_problems_rejected(kw, status):
    p = prob(**kw)
    lib = M.lib()
    assert lib.moe_tile_m(ctypes.byref(p)) == -1
    assert lib.moe_rows_capacity(ctypes.byref(p)) == -1
    assert lib.moe_workspace_bytes(ctypes.byref(p), M.STAGE_LAYER) == 0
    fake = ctypes.c_void_p(1 << 20)
    args15 = [fake] * 15
    assert lib.moe_layer_forward(ctypes.byref(p), *args15, fake, 1 << 40, None) == status
    assert lib.moe_route(ctypes.byref(p), *([fake] * 8), fake, 1 << 40, None) == status
    assert lib.moe_permute(ctypes.byref(p), *([fake] * 7), fake, 1 << 40, None) == status
    assert lib.moe_expert_ffn(ctypes.byref(p), *([fake] * 11), fake, 1 << 40, None) == status
    assert lib.moe_combine(ctypes.byref(p), *([fake] * 4), None) == status
    assert lib.moe_expert_up(ctypes.byref(p), *([fake] * 7), None, 0, None) == status
    assert lib.moe_expert_down(ctypes.byref(p), *([fake] * 7), None, 0, None) == status
    assert lib.moe_apply_capacity(ctypes.byref(p), *([fake] * 5), fake, 1 << 40, None) == status
    assert lib.moe_layer_forward_noalloc(ctypes.byref(p), *args15, None) == status


@pytest.mark.parametrize("S,K,ok", [((1 << 24) - 1, 2, True), (1 << 24, 2, False), ((1 << 24) - 1, 4, True),
                                    ((1 << 24) - 1, 8, False), ((1 << 23), 8, False), ((1 << 23) - 1, 8, True),
                                    ((1 << 20), 64, False), ((1 << 20) - 1, 64, True)])
def test_token_and_pair_limits(S, K, ok):
    """S < 2^24 and S * K < 2^26: every kernel launch stays below 2^32
    work-items (256 threads per token in the combine, 64 per pair in the row
    gather and quantiser)."""
    p = prob(S=S, K=K, E=64)
    lib = M.lib()
    assert (lib.moe_tile_m(ctypes.byref(p)) > 0) == ok
    assert (lib.moe_rows_capacity(ctypes.byref(p)) > 0) == ok
    if not ok:
        fake = ctypes.c_void_p(1 << 20)
        assert lib.moe_layer_forward(ctypes.byref(p), *([fake] * 15), fake, 1 << 62, None) == M.MOE_ERR_UNSUPPORTED
    q = lib.moe_quantize_rows
    fake = ctypes.c_void_p(1 << 20)
    assert q(fake, 1 << 26, 64, fake, fake, None) == M.MOE_ERR_UNSUPPORTED


def test_noalloc_rejects_problems_past_its_scratch():
    """moe_layer_forward_noalloc checks the layer's workspace against its
    scratch array on the host, before any HIP call: a problem that needs more
    returns MOE_ERR_TOO_LARGE; pointer checks come first; S == 0 is a no-op."""
    lib = M.lib()
    a = ctypes.c_void_p(1 << 20)
    base = [a, a, None, None, a, a, a, a, None, None, a, None, None, None, None]
    big = prob(S=4096, d=4096, d_ff=14336, E=8, K=2)
    assert M.moe_workspace_bytes(big, M.STAGE_LAYER) > M.MOE_NOALLOC_SCRATCH_BYTES
    assert lib.moe_layer_forward_noalloc(ctypes.byref(big), *base, None) == M.MOE_ERR_TOO_LARGE
    assert "no-alloc" in M.moe_status_string(M.MOE_ERR_TOO_LARGE)
    bad = list(base); bad[0] = None
    assert lib.moe_layer_forward_noalloc(ctypes.byref(big), *bad, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_layer_forward_noalloc(ctypes.byref(prob(S=0)), *([None] * 15), None) == M.MOE_OK
    # decode-sized problems fit: the shapes the header names
    for kw in (dict(S=255, d=4096, d_ff=14336, E=8, K=2),
               dict(S=16, d=7168, d_ff=2048, E=256, K=8, w="fp8", n_groups=8, topk_groups=2),
               dict(S=16, d=7168, d_ff=2048, E=256, K=8, w="fp8", n_groups=8, topk_groups=2, act_quant=1)):
        assert 0 < M.moe_workspace_bytes(prob(**kw), M.STAGE_LAYER) <= M.MOE_NOALLOC_SCRATCH_BYTES, kw


@pytest.mark.parametrize("tau,ok", [(0.0, True), (1.0, True), (0.25, True), (-1.0, False),
                                    (float("nan"), False), (float("inf"), False)])
def test_gate_temperature_validation(tau, ok):
    """0 means 1; a temperature must otherwise be positive and finite."""
    p = prob(temperature=tau)
    lib = M.lib()
    assert (lib.moe_tile_m(ctypes.byref(p)) > 0) == ok
    if not ok:
        assert lib.moe_route(ctypes.byref(p), *([ctypes.c_void_p(1 << 20)] * 8), None, 0, None) == M.MOE_ERR_INVALID_ARG


def test_load_stats_argument_checks():
    lib = M.lib()
    p = prob()
    a = ctypes.c_void_p(1 << 20)
    assert lib.moe_load_stats(ctypes.byref(p), None, None, None, 1.0, a, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(ctypes.byref(p), a, None, None, 1.0, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(ctypes.byref(p), a, None, None, float("nan"), a, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(ctypes.byref(p), ctypes.c_void_p((1 << 20) + 4), None, None, 1.0, a, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_load_stats(ctypes.byref(prob(S=0)), None, None, None, 1.0, None, None) == M.MOE_OK


def test_null_problem_and_status_strings():
    lib = M.lib()
    assert lib.moe_tile_m(None) == -1
    assert lib.moe_route(None, *([None] * 8), None, 0, None) == M.MOE_ERR_INVALID_ARG
    for s, txt in ((0, "ok"), (-1, "invalid"), (-2, "unsupported"), (-3, "workspace"), (-4, "HIP"),
                   (-5, "scratch")):
        assert txt in M.moe_status_string(s)


def test_pointer_and_workspace_checks_precede_launch():
    lib = M.lib()
    p = prob()
    a = ctypes.c_void_p(1 << 20)          # aligned, never dereferenced
    odd = ctypes.c_void_p((1 << 20) + 4)  # misaligned
    ws_need = M.moe_workspace_bytes(p, M.STAGE_LAYER)
    assert ws_need > 0
    base = [a, a, None, None, a, a, a, a, None, None, a, None, None, None, None]
    # missing required pointer
    bad = list(base); bad[0] = None
    assert lib.moe_layer_forward(ctypes.byref(p), *bad, a, ws_need, None) == M.MOE_ERR_INVALID_ARG
    # misaligned pointer
    bad = list(base); bad[4] = odd
    assert lib.moe_layer_forward(ctypes.byref(p), *bad, a, ws_need, None) == M.MOE_ERR_INVALID_ARG
    # workspace too small / missing
    assert lib.moe_layer_forward(ctypes.byref(p), *base, a, ws_need - 1, None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_layer_forward(ctypes.byref(p), *base, None, ws_need, None) == M.MOE_ERR_WORKSPACE
    # fp8 weights without scales
    p8 = prob(w="fp8")
    assert lib.moe_layer_forward(ctypes.byref(p8), *base, a, 1 << 40, None) == M.MOE_ERR_INVALID_ARG
    # route: logits_in lets x / W_r be NULL, but outputs are required
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, a, None, None, a, None, 0, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(p), None, None, None, None, None, None, a, a, None, 0, None) == M.MOE_ERR_INVALID_ARG
    pw = prob(E=64, K=4)   # router product on the MFMA path needs a logits workspace
    assert M.moe_workspace_bytes(pw, M.STAGE_ROUTE) == 64 * 64 * 4
    assert lib.moe_route(ctypes.byref(pw), a, a, None, None, None, None, a, a, None, 0, None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_permute(ctypes.byref(p), a, a, a, a, a, a, a, None, 0, None) == M.MOE_ERR_WORKSPACE


def test_empty_batch_is_a_noop_without_device():
    lib = M.lib()
    p = prob(S=0)
    assert lib.moe_layer_forward(ctypes.byref(p), *([None] * 15), None, 0, None) == M.MOE_OK
    assert lib.moe_route(ctypes.byref(p), *([None] * 8), None, 0, None) == M.MOE_OK
    assert lib.moe_permute(ctypes.byref(p), *([None] * 7), None, 0, None) == M.MOE_OK
    assert lib.moe_expert_ffn(ctypes.byref(p), *([None] * 11), None, 0, None) == M.MOE_OK
    assert lib.moe_combine(ctypes.byref(p), *([None] * 4), None) == M.MOE_OK
    assert lib.moe_expert_up(ctypes.byref(p), *([None] * 7), None, 0, None) == M.MOE_OK
    assert lib.moe_expert_down(ctypes.byref(p), *([None] * 7), None, 0, None) == M.MOE_OK


@pytest.mark.parametrize("S,E,K", [(4096, 8, 2), (16, 8, 2), (8192, 64, 4), (4096, 256, 8), (1, 8, 2), (3, 512, 64)])
def test_capacity_formula(S, E, K):
    p = prob(S=S, E=E, K=K, d=4096, d_ff=14336)
    tm = M.moe_tile_m(p)
    assert tm in (16, 128, 256)
    pairs = S * K
    assert M.moe_rows_capacity(p) == pairs + min(E, pairs) * (tm - 1)
    cap = M.moe_rows_capacity(p)
    ws = M.moe_workspace_bytes(p, M.STAGE_LAYER)
    assert ws >= cap * (4096 + 14336) * 2   # h and y_perm (x_perm only when rows are not read in place)


def test_apply_capacity_argument_checks():
    lib = M.lib()
    p = prob(capacity=5)
    a = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    need = M.moe_workspace_bytes(p, M.STAGE_CAPACITY)
    assert need == ((64 * 2 + 4 + 8) * 4 + 255) // 256 * 256   # pair list, 4 state ints, run[E]
    call = lambda *args: lib.moe_apply_capacity(ctypes.byref(p), *args)
    # logits, topk_idx, topk_gate are required; select_bias and dropped are optional
    assert call(None, None, a, a, None, a, need, None) == M.MOE_ERR_INVALID_ARG
    assert call(a, None, None, a, None, a, need, None) == M.MOE_ERR_INVALID_ARG
    assert call(a, None, a, None, None, a, need, None) == M.MOE_ERR_INVALID_ARG
    assert call(a, odd, a, a, None, a, need, None) == M.MOE_ERR_INVALID_ARG
    assert call(a, None, a, a, odd, a, need, None) == M.MOE_ERR_INVALID_ARG
    assert call(a, None, a, a, None, a, need - 1, None) == M.MOE_ERR_WORKSPACE
    assert call(a, None, a, a, None, None, need, None) == M.MOE_ERR_WORKSPACE
    # a layer with a capacity needs room for the pair list on top
    assert M.moe_workspace_bytes(p, M.STAGE_LAYER) == M.moe_workspace_bytes(prob(), M.STAGE_LAYER) + need
    assert lib.moe_apply_capacity(ctypes.byref(prob(S=0)), *([None] * 5), None, 0, None) == M.MOE_OK


def test_fp8_activation_checks():
    lib = M.lib()
    a = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 4)
    p = prob(w="fp8", act_quant=1)
    assert lib.moe_tile_m(ctypes.byref(p)) > 0
    # the layer needs room for the h codes and the row scales on top
    plain = M.moe_workspace_bytes(prob(w="fp8"), M.STAGE_LAYER)
    assert M.moe_workspace_bytes(p, M.STAGE_LAYER) > plain
    # the stage entry points take bf16 activations only
    assert lib.moe_permute(ctypes.byref(p), *([a] * 7), a, 1 << 30, None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_ffn(ctypes.byref(p), *([a] * 11), a, 1 << 30, None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_up(ctypes.byref(p), *([a] * 7), None, 0, None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_down(ctypes.byref(p), *([a] * 7), None, 0, None) == M.MOE_ERR_UNSUPPORTED
    # the W8A8 stage products: they need act_quant = 1 and every pointer
    assert lib.moe_expert_up_a8(ctypes.byref(prob(w="fp8")), *([a] * 8), None, 0, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_down_a8(ctypes.byref(prob(w="fp8")), *([a] * 8), None, 0, None) == M.MOE_ERR_INVALID_ARG
    for i in range(8):
        args = [a] * 8
        args[i] = None
        assert lib.moe_expert_up_a8(ctypes.byref(p), *args, None, 0, None) == M.MOE_ERR_INVALID_ARG
        args[i] = odd
        assert lib.moe_expert_down_a8(ctypes.byref(p), *args, None, 0, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_up_a8(ctypes.byref(prob(w="fp8", act_quant=1, S=0)), *([None] * 8), None, 0, None) == 0
    # the row quantiser
    q = lib.moe_quantize_rows
    assert q(a, -1, 64, a, a, None) == M.MOE_ERR_INVALID_ARG
    assert q(a, 4, 60, a, a, None) == M.MOE_ERR_INVALID_ARG
    assert q(a, 4, 0, a, a, None) == M.MOE_ERR_INVALID_ARG
    assert q(None, 4, 64, a, a, None) == M.MOE_ERR_INVALID_ARG
    assert q(a, 4, 64, odd, a, None) == M.MOE_ERR_INVALID_ARG
    assert q(a, 4, 64, a, None, None) == M.MOE_ERR_INVALID_ARG
    assert q(None, 0, 64, None, None, None) == M.MOE_OK
