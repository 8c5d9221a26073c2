"""Pins for the blockwise feed-forward oracle: checks that tie it to something other than itself.

Every check takes the implementation as an argument (an object exposing ``gelu``, ``relu``, ``ffn_rows``,
``ffn_blockwise`` and ``block_bounds``) so that copies of the oracle with a planted mistake can be run
through the same checks, each of which must then fail at least one.

What pins what:
  * hand-worked cases (tests/golden/ffn_hand_worked.txt): a rational ReLU case and a GELU case built on
    printed values of the standard normal CDF;
  * closed forms of GELU: GELU(0) = 0, GELU(x) = x Phi(x) at x = 1, 2, 3 from normal tables, the
    identity GELU(x) - GELU(-x) = x, and the limits x and 0 far from zero;
  * a pure-Python brute force with math.erf (the C library's erf, not the oracle's) on tiny shapes;
  * special cases: identity weights give act(x) elementwise; W2 = 0 gives b2 on every row;
  * invariants: the blockwise form equals the row-wise one for every block size, the block bounds tile
    the rows exactly, permuting rows permutes the output, and the output is linear in W2 when b2 = 0.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ffn_hand_worked.txt")
PHI = {1: 0.8413447460685429, 2: 0.9772498680518208, 3: 0.9986501019683699}   # standard normal CDF, tables


def _mat(text: str) -> np.ndarray:
    return np.array([[float(Fraction(t)) for t in row.split()] for row in text.split("|")], dtype=np.float64)


def _vec(text: str) -> np.ndarray:
    return np.array([float(Fraction(t.strip())) for t in text.split("|")], dtype=np.float64)


def load_golden():
    cases, cur = [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            if key == "case":
                cur = {"name": val.strip()}
                cases.append(cur)
            else:
                cur[key] = val.strip()
    return cases


def _close(a, b, tol=1e-13, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b) / np.maximum(1.0, np.abs(b))) if a.size else 0.0
    assert err <= tol, f"{what}: error {err:.3e} > {tol:.1e}"


def _rand(rng, n, d, d_ff):
    x = rng.standard_normal((n, d))
    w1 = rng.standard_normal((d_ff, d)) / math.sqrt(d)
    w2 = rng.standard_normal((d, d_ff)) / math.sqrt(d_ff)
    return x, w1, 0.3 * rng.standard_normal(d_ff), w2, 0.3 * rng.standard_normal(d)


def check_golden(impl):
    for c in load_golden():
        args = (_mat(c["x"]), _mat(c["w1"]), _vec(c["b1"]), _mat(c["w2"]), _vec(c["b2"]), c["act"])
        want = _mat(c["y"])
        _close(impl.ffn_rows(*args), want, 1e-15, c["name"])
        _close(impl.ffn_blockwise(*args, block=1), want, 1e-15, c["name"] + " blockwise")


def check_gelu_values(impl):
    _close(impl.gelu(np.array([0.0])), np.array([0.0]), 0.0, "gelu(0)")
    for x, phi in PHI.items():
        _close(impl.gelu(np.array([float(x)])), np.array([x * phi]), 1e-15, f"gelu({x})")
        _close(impl.gelu(np.array([-float(x)])), np.array([-x * (1.0 - phi)]), 1e-15, f"gelu(-{x})")
    xs = np.random.default_rng(21).standard_normal(200) * 3
    _close(impl.gelu(xs) - impl.gelu(-xs), xs, 1e-14, "gelu(x) - gelu(-x) = x")
    big = np.array([9.0, 12.0, 40.0])
    _close(impl.gelu(big), big, 1e-15, "gelu -> x")
    assert np.all(np.abs(impl.gelu(-big)) < 1e-15), "gelu -> 0"
    _close(impl.relu(np.array([-2.0, 0.0, 3.5])), np.array([0.0, 0.0, 3.5]), 0.0, "relu")


def _brute(x, w1, b1, w2, b2, act):
    n, d = x.shape
    d_ff = w1.shape[0]
    out = []
    for i in range(n):
        h = []
        for f in range(d_ff):
            s = b1[f]
            for c in range(d):
                s += x[i][c] * w1[f][c]
            h.append(s * 0.5 * (1.0 + math.erf(s / math.sqrt(2.0))) if act == "gelu" else max(s, 0.0))
        row = []
        for c in range(w2.shape[0]):
            s = b2[c]
            for f in range(d_ff):
                s += h[f] * w2[c][f]
            row.append(s)
        out.append(row)
    return np.array(out)


def check_bruteforce(impl, seed=22):
    rng = np.random.default_rng(seed)
    for n, d, d_ff in ((1, 1, 1), (3, 2, 5), (5, 4, 3), (4, 3, 8)):
        x, w1, b1, w2, b2 = _rand(rng, n, d, d_ff)
        for act in ("gelu", "relu"):
            _close(impl.ffn_rows(x, w1, b1, w2, b2, act), _brute(x, w1, b1, w2, b2, act), 1e-13, f"brute {act}")


def check_special_weights(impl, seed=23):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((6, 5)) * 2
    eye = np.eye(5)
    for act in ("gelu", "relu"):
        _close(impl.ffn_rows(x, eye, None, eye, None, act), impl.ACTS[act](x), 1e-15, f"identity {act}")
    _close(impl.ffn_rows(x, eye, None, eye, None, "none"), x, 1e-15, "identity weights, no activation")
    _close(impl.ffn_rows(x, 2 * eye, None, eye / 4, None, "none"), x / 2, 1e-15, "linear layers compose")
    _, w1, b1, _, b2 = _rand(rng, 6, 5, 7)
    _close(impl.ffn_rows(x, w1, b1, np.zeros((5, 7)), b2, "gelu"), np.tile(b2, (6, 1)), 0.0, "W2 = 0")


def check_blockwise(impl, seed=24):
    rng = np.random.default_rng(seed)
    x, w1, b1, w2, b2 = _rand(rng, 13, 6, 10)
    full = impl.ffn_rows(x, w1, b1, w2, b2, "gelu")
    for block in (1, 2, 3, 7, 13, 20):
        _close(impl.ffn_blockwise(x, w1, b1, w2, b2, "gelu", block), full, 1e-13, f"block {block}")
    assert impl.block_bounds(10, 4) == [0, 4, 8, 10]
    assert impl.block_bounds(8, 4) == [0, 4, 8]
    assert impl.block_bounds(3, 5) == [0, 3]


def check_invariants(impl, seed=25):
    rng = np.random.default_rng(seed)
    x, w1, b1, w2, _ = _rand(rng, 9, 4, 6)
    perm = rng.permutation(9)
    y = impl.ffn_rows(x, w1, b1, w2, None, "gelu")
    _close(impl.ffn_rows(x[perm], w1, b1, w2, None, "gelu"), y[perm], 1e-14, "row permutation")
    w2b = rng.standard_normal(w2.shape)
    _close(impl.ffn_rows(x, w1, b1, w2 + w2b, None, "gelu"),
           y + impl.ffn_rows(x, w1, b1, w2b, None, "gelu"), 1e-13, "linear in W2")


ALL_CHECKS = [check_golden, check_gelu_values, check_bruteforce, check_special_weights, check_blockwise,
              check_invariants]
