"""The oracle's pins catch plausible mistakes in the oracle.

Each mutation below plants one plausible mistake in a copy of
oracle/fia_oracle.py (a wrong head map, sign, bias, index, bound, decode
constant, layout order ...); the pins of test_oracle_pins.py then run in a
child process against that copy, and at least one pin must fail.  A mutation
that every pin accepts would mean part of the oracle is not pinned."""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "fia_oracle.py")

# (name, text in the oracle, replacement)
MUTATIONS = [
    ("gqa head map", "g = h // G", "g = h % num_kv_heads"),
    ("alibi sign", "s = s + slopes[h] * (jpos - ipos)", "s = s + slopes[h] * (ipos - jpos)"),
    ("alibi scaled", "s = s + slopes[h] * (jpos - ipos)", "s = s + scale * slopes[h] * (jpos - ipos)"),
    ("mode 3 delta sign", "return j <= i + delta", "return j <= i - delta"),
    ("mode 2 strict", "        return j <= i\n", "        return j < i\n"),
    ("band lower edge", "(j >= i + delta - pre)", "(j >= i + delta - pre + 1)"),
    ("band upper edge", "(j <= i + delta + nxt)", "(j < i + delta + nxt)"),
    ("e4m3 exponent bias", "np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    ("e4m3 subnormal scale", "sub = (m / 8.0) * 2.0 ** -6", "sub = (m / 8.0) * 2.0 ** -7"),
    ("e4m3 nan code", "np.where((e == 15) & (m == 7), np.nan, val)", "np.where((e == 15) & (m == 6), np.nan, val)"),
    ("bf16 shift", "astype(np.uint32) << np.uint32(16)", "astype(np.uint32) << np.uint32(15)"),
    ("fp16 exponent bias", "np.exp2(e.astype(np.float64) - 15.0)", "np.exp2(e.astype(np.float64) - 14.0)"),
    ("fp16 subnormal scale", "sub = (m / 1024.0) * 2.0 ** -14", "sub = (m / 1024.0) * 2.0 ** -15"),
    ("lse log base", "lse[rows] = m[rows] + np.log(l)", "lse[rows] = m[rows] + np.log2(l)"),
    ("empty lse sign", 'POS_INF = float("inf")', 'POS_INF = float("-inf")'),
    ("sink not in normaliser", "l = l + np.exp(extra_logit - m[rows])", "l = l + 0.0 * np.exp(extra_logit - m[rows])"),
    ("sink scaled", "extra_logit=float(sinks[h]))", "extra_logit=float(sinks[h]) * case.softmax_scale)"),
    ("window off by one", "lo, hi = max(0, p - win_left), min(Lk - 1, p + win_right)",
     "lo, hi = max(0, p - win_left + 1), min(Lk - 1, p + win_right)"),
    ("compressed bound", "comp = [int(c) for c in idx_row if 0 <= int(c) < n_cmp]",
     "comp = [int(c) for c in idx_row if 0 <= int(c) <= n_cmp]"),
    ("multi-token causality", "n_cmp = max(0, Lk // cmp_ratio - (S1 - 1 - t))", "n_cmp = max(0, Lk // cmp_ratio)"),
    ("token position", "    p = Lk - S1 + t\n    lo, hi", "    p = Lk - 1 - t\n    lo, hi"),
    ("packed scale order", "nope = codes * np.repeat(scales, TILE)", "nope = codes * np.tile(scales, TILE)"),
    ("packed field order", "return np.concatenate([rope, nope])", "return np.concatenate([nope, rope])"),
    ("padded rows computed", "live = idx[idx < Lq]", "live = idx[idx < Lq + 1]"),
    ("paged slot", "return pool[blocks, j % bs]", "return pool[blocks, (j + 1) % bs]"),
    ("bnnbsd order", "return pool[blocks, :, j % bs]", "return pool[blocks, j % bs]"),
    ("length broadcast", "        return arr * B\n", "        return arr + [0] * (B - 1)\n"),
    ("tnd kv length", "kv_len = [kv_off[b + 1] - kv_off[b] for b in range(B)]", "kv_len = [kv_off[b + 1] for b in range(B)]"),
    ("mask polarity", "vis = (m2[:Lq, :Lk] == 0)[live]", "vis = (m2[:Lq, :Lk] != 0)[live]"),
    ("bias row broadcast", "(pb[np.zeros_like(live)] if pb.shape[0] == 1 else pb[live])",
     "(pb[np.zeros_like(live)] if pb.shape[0] == 1 else pb[np.zeros_like(live)])"),
    ("dequant offset sign", "return s * (c + o)", "return s * (c - o)"),
    ("per-token scale batch", "s = sc2[b, :Lk][:, None, None]", "s = sc2[0, :Lk][:, None, None]"),
    ("sfmla tnd kv offset", "return kv[int(cu[b]) + r, 0]", "return kv[r, 0]"),
    ("sfmla lse without sink", "extra_logit=None if sinks is None else float(sinks[h]))",
     "extra_logit=None)"),
]

DRIVER = """
import sys
sys.path.insert(0, sys.argv[1])
import oracle.fia_oracle
assert oracle.fia_oracle.__file__.startswith(sys.argv[1]), oracle.fia_oracle.__file__
import pytest
sys.exit(pytest.main([sys.argv[2], "-x", "-q", "-p", "no:cacheprovider"]))
"""


def _run_pins(tmpdir):
    r = subprocess.run([sys.executable, "-c", DRIVER, tmpdir,
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-400:]


def _mutant(name, old, new):
    src = open(ORACLE).read()
    assert src.count(old) >= 1, f"{name}: text not found in the oracle"
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    try:
        os.makedirs(os.path.join(d, "oracle"))
        shutil.copy(os.path.join(ROOT, "oracle", "__init__.py"), os.path.join(d, "oracle"))
        with open(os.path.join(d, "oracle", "fia_oracle.py"), "w") as f:
            f.write(src.replace(old, new))
        return _run_pins(d)
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_unmutated_copy_passes_the_pins():
    d = tempfile.mkdtemp(prefix="oracle_copy_")
    try:
        shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(d, "oracle"),
                        ignore=shutil.ignore_patterns("__pycache__"))
        rc, tail = _run_pins(d)
        assert rc == 0, tail
    finally:
        shutil.rmtree(d, ignore_errors=True)


def test_every_mutation_fails_a_pin():
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        results = list(ex.map(lambda m: (m[0],) + _mutant(*m), MUTATIONS))
    survivors = [(name, tail) for name, rc, tail in results if rc == 0]
    assert not survivors, "mutations no pin catches: " + "; ".join(n for n, _ in survivors)
    # a crash is not a caught mistake: every mutant must reach the pins and fail one
    crashed = [name for name, rc, tail in results if rc not in (1,)]
    assert not crashed, "mutants that did not run the pins to a failure: " + ", ".join(crashed)
