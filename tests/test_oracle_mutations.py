"""Planted mistakes in the numpy oracle: each must fail one of its pins.

Every mutation below is a plausible slip in oracle/moe_oracle.py (a dropped
term, a wrong sign or index, a transposed operand, a different order or
constant).  For each one, a copy of the oracle with that single change runs
the pin suites (printed worked example, special cases, closed forms,
brute force, exhaustive decoders, invariants) in a separate process; the
test passes only if every mutant fails at least one pin and the unchanged
copy passes them all.  CPU only."""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "moe_oracle.py")
PIN_FILES = ["test_oracle_pins.py", "test_oracle_fp8act.py", "test_oracle_capacity.py", "test_oracle_stats.py"]

# (name, exact text in the oracle, replacement)
MUTATIONS = [
    ("drop b1", "a = x_rows @ w1.T + b1[None, :]", "a = x_rows @ w1.T"),
    ("drop b2", "o = h @ w2.T + b2[None, :]", "o = h @ w2.T"),
    ("erf argument", "_erf(a / math.sqrt(2.0))", "_erf(a / 2.0)"),
    ("ties to the higher index", 'order = np.argsort(-key, axis=1, kind="stable")',
     'order = key.shape[1] - 1 - np.argsort(-key[:, ::-1], axis=1, kind="stable")'),
    ("renormalise flag inverted", "    if renormalize:\n        return softmax(chosen, temperature)",
     "    if not renormalize:\n        return softmax(chosen, temperature)"),
    ("groups kept by lowest score",
     '        g_order = np.argsort(-gs, axis=1, kind="stable")[:, :topk_groups]\n'
     '        keep = np.zeros((S, n_groups), dtype=bool)\n'
     '        np.put_along_axis(keep, g_order, True, axis=1)\n        keep_e',
     '        g_order = np.argsort(gs, axis=1, kind="stable")[:, :topk_groups]\n'
     '        keep = np.zeros((S, n_groups), dtype=bool)\n'
     '        np.put_along_axis(keep, g_order, True, axis=1)\n        keep_e'),
    ("group sum by adjacent pairs", "v[:, :, :w] = v[:, :, :w] + v[:, :, w:2 * w]",
     "v[:, :, :w] = v[:, :, 0:2 * w:2] + v[:, :, 1:2 * w:2]"),
    ("e4m3 exponent bias", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    ("e4m3 subnormal scale", "m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    ("fp8 scale on the input axis",
     "    if scale is not None:\n        v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]",
     "    if scale is not None:\n        v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[None, :]"),
    ("tokens in reverse order inside an expert", "    for p in range(S * K):", "    for p in reversed(range(S * K)):"),
    ("unpadded rows", "inv = padded[flat] + rank", "inv = dense[flat] + rank"),
    ("combine gates reversed", 'return np.einsum("sk,skd->sd", gates, outputs)',
     'return np.einsum("sk,skd->sd", gates[:, ::-1], outputs)'),
    ("selection bias subtracted",
     "        key = (key + np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)\n"
     "    S, E = key.shape\n    if not 1 <= K <= E:",
     "        key = (key - np.asarray(select_bias, dtype=np.float32)[None, :]).astype(np.float32)\n"
     "    S, E = key.shape\n    if not 1 <= K <= E:"),
    ("router bias subtracted", "acc = acc + np.asarray(router_bias", "acc = acc - np.asarray(router_bias"),
    ("temperature multiplies", "z = np.asarray(logits, dtype=np.float64) / float(temperature)",
     "z = np.asarray(logits, dtype=np.float64) * float(temperature)"),
    ("e4m3 maximum of the fnuz format", "E4M3_MAX = 448.0", "E4M3_MAX = 240.0"),
    ("capacity off by one", "if load[e] < capacity:", "if load[e] <= capacity:"),
    ("rerouting ignores held experts", "int(e) not in held and load[e] < capacity",
     "load[e] < capacity"),
    ("sample standard deviation", '"std": float(np.sqrt(((c - mean) ** 2).sum() / E))',
     '"std": float(np.sqrt(((c - mean) ** 2).sum() / (E - 1)))'),
    ("balance loss without the share", "f = c / c.sum()", "f = c"),
    ("quantiser ties away from zero", "pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))",
     "pick_hi = (d_hi <= d_lo)"),
    ("W8A8 hidden row left unquantised",
     "    qh, sh = quantize_rows_e4m3(h.astype(np.float32))\n"
     "    o = dequantize_rows_e4m3(qh, sh) @ w2.T + b2[None, :]",
     "    o = h @ w2.T + b2[None, :]"),
]


def _tree(tmp, source):
    """A copy of what the pin suites import, with the oracle replaced."""
    for d in ("datagen",):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(tmp, d),
                        ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(tmp, "oracle"))
    shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(tmp, "oracle"))
    open(os.path.join(tmp, "oracle", "moe_oracle.py"), "w").write(source)
    os.makedirs(os.path.join(tmp, "tests"))
    for f in ["conftest.py", "_util.py"] + PIN_FILES:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tmp, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tmp, "tests", "golden"))


def _run(source):
    with tempfile.TemporaryDirectory() as tmp:
        _tree(tmp, source)
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="2")
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"]
                           + [os.path.join("tests", f) for f in PIN_FILES],
                           cwd=tmp, env=env, capture_output=True, text=True, timeout=600)
        return r.returncode, r.stdout[-600:]


def test_mutations_apply_once():
    src = open(ORACLE).read()
    for name, old, new in MUTATIONS:
        assert src.count(old) == 1, name
        assert old != new


@pytest.mark.slow
def test_every_planted_mistake_fails_a_pin():
    src = open(ORACLE).read()
    jobs = [("unchanged", src)] + [(name, src.replace(old, new)) for name, old, new in MUTATIONS]
    with cf.ThreadPoolExecutor(max(1, min(4, (os.cpu_count() or 2) // 2))) as ex:
        results = dict(zip([n for n, _ in jobs], ex.map(lambda j: _run(j[1]), jobs)))
    rc, out = results.pop("unchanged")
    assert rc == 0, out                                  # the real oracle passes its pins
    survivors = [n for n, (rc, _) in results.items() if rc != 1]
    assert not survivors, {n: results[n][1] for n in survivors}
