"""Pins for the CPU oracle: checks that tie it to something other than itself.

Every check takes the oracle implementation as an argument (an object exposing ``naive_head``,
``blockwise_head``, ``merge``, ``chunked_head``) so that the same checks can be run against copies of the
oracle with a planted mistake, which must fail at least one of them.

What pins what:
  * hand-worked cases (tests/golden/hand_worked.txt): exact rational answers from the definition;
  * independent library routines: torch's fp64 CPU scaled_dot_product_attention for O, scipy's
    softmax/logsumexp on an explicit logit matrix for the weights and lse;
  * a pure-Python brute force (math.exp loops) on tiny shapes;
  * closed forms: Q = 0 gives the mean of the visible V rows and lse = ln(#visible); one key gives its V
    row; two keys give logistic weights; a dominant key selects its V row; constant V is reproduced;
    V = I returns the weights themselves, which are >= 0 and sum to one per row;
  * invariants: blockwise = naive for every block size (deferred vs progressive normalisation are the
    same result), chunked = single pass for every chunk count, merge is commutative and associative
    with identity (0, -inf), and permuting K and V rows together changes nothing when not causal.
"""
from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.txt")
TIGHT = 1e-12


# ----------------------------------------------------------------------------------------------- helpers
def _tok(t: str) -> float:
    if t == "-inf":
        return -math.inf
    if t.startswith("ln"):
        return math.log(int(t[2:]))
    return float(Fraction(t))


def _mat(text: str) -> np.ndarray:
    return np.array([[_tok(t) for t in row.split()] for row in text.split("|")], dtype=np.float64)


def _vec(text: str) -> np.ndarray:
    return np.array([_tok(t.strip()) for t in text.split("|")], dtype=np.float64)


def load_golden():
    cases, merges, cur = [], [], None
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, val = line.partition(":")
            val = val.strip()
            if key in ("case", "merge"):
                cur = {"name": val}
                (cases if key == "case" else merges).append(cur)
            else:
                cur[key] = val
    return cases, merges


def _close(a, b, tol=TIGHT, what=""):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    inf_a, inf_b = np.isinf(a), np.isinf(b)
    assert np.array_equal(inf_a, inf_b) and np.array_equal(a[inf_a], b[inf_b]), f"{what}: infinities differ"
    fin = ~inf_a
    err = np.max(np.abs(a[fin] - b[fin]) / np.maximum(1.0, np.abs(b[fin]))) if fin.any() else 0.0
    assert err <= tol, f"{what}: error {err:.3e} > {tol:.1e}"


def _rand(rng, n, n_kv, d, dv=None, std=1.0):
    dv = d if dv is None else dv
    return (rng.standard_normal((n, d)) * std, rng.standard_normal((n_kv, d)), rng.standard_normal((n_kv, dv)))


# ------------------------------------------------------------------------------------------------ checks
def check_golden_attention(impl):
    cases, _ = load_golden()
    for c in cases:
        q, k, v = _mat(c["q"]), _mat(c["k"]), _mat(c["v"])
        scale, causal, off = float(c["scale"]), bool(int(c["causal"])), int(c["offset"])
        o_ref, lse_ref = _mat(c["o"]), _vec(c["lse"])
        o, lse = impl.naive_head(q, k, v, scale, causal, off)
        _close(o, o_ref, 1e-14, c["name"] + " naive O")
        _close(lse, lse_ref, 1e-14, c["name"] + " naive lse")
        if off == k.shape[0] - q.shape[0]:      # the default offset is the bottom-right alignment
            for f in (impl.naive_head, impl.blockwise_head, impl.chunked_head):
                o, lse = f(q, k, v, scale, causal)
                _close(o, o_ref, 1e-14, c["name"] + " default offset O")
                _close(lse, lse_ref, 1e-14, c["name"] + " default offset lse")
        for blk in (1, 2, 3):
            o, lse = impl.blockwise_head(q, k, v, scale, causal, off, None, blk)
            _close(o, o_ref, 1e-14, f"{c['name']} blockwise({blk}) O")
            _close(lse, lse_ref, 1e-14, f"{c['name']} blockwise({blk}) lse")
        for p in range(1, k.shape[0] + 2):
            o, lse = impl.chunked_head(q, k, v, scale, causal, off, None, p)
            _close(o, o_ref, 1e-14, f"{c['name']} chunked({p}) O")
            _close(lse, lse_ref, 1e-14, f"{c['name']} chunked({p}) lse")


def check_golden_merge(impl):
    _, merges = load_golden()
    for c in merges:
        o, lse = impl.merge(_mat(c["o_a"]), _vec(c["lse_a"]), _mat(c["o_b"]), _vec(c["lse_b"]))
        _close(o, _mat(c["o"]), 1e-14, c["name"] + " O")
        _close(lse, _vec(c["lse"]), 1e-14, c["name"] + " lse")


def check_torch_sdpa(impl, seed=11):
    """O against torch's own fp64 CPU attention, with an explicit bottom-right mask."""
    import torch
    import torch.nn.functional as F

    rng = np.random.default_rng(seed)
    for n, n_kv, d, dv, causal, scale in [(5, 5, 4, 4, False, 0.5), (7, 7, 3, 5, True, 1.3),
                                          (4, 9, 6, 2, True, 0.7), (9, 4, 2, 3, True, 0.9),
                                          (6, 11, 5, 5, False, 2.0)]:
        q, k, v = _rand(rng, n, n_kv, d, dv)
        off = n_kv - n
        mask = np.ones((n, n_kv), bool) if not causal else (np.arange(n_kv)[None, :] <= np.arange(n)[:, None] + off)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q)[None], torch.from_numpy(k)[None],
                                             torch.from_numpy(v)[None], attn_mask=torch.from_numpy(mask)[None],
                                             scale=scale)[0].numpy()
        o, _ = impl.naive_head(q, k, v, scale, causal, off)
        live = mask.any(axis=1)
        _close(o[live], ref[live], 1e-12, f"sdpa n={n} n_kv={n_kv} causal={causal}")


def check_scipy_softmax(impl, seed=12):
    """V = I returns the softmax weights; lse matches scipy's logsumexp of the explicit logits."""
    from scipy.special import logsumexp, softmax

    rng = np.random.default_rng(seed)
    for n, n_kv, d, causal, scale in [(6, 6, 3, False, 0.8), (5, 8, 4, True, 1.1), (8, 5, 2, True, 0.6)]:
        q, k = rng.standard_normal((n, d)), rng.standard_normal((n_kv, d))
        off = n_kv - n
        logits = np.einsum("ic,jc->ij", q, k) * scale
        mask = np.ones((n, n_kv), bool) if not causal else (np.arange(n_kv)[None, :] <= np.arange(n)[:, None] + off)
        for form in ("naive", "blockwise"):
            f = impl.naive_head if form == "naive" else (lambda *a: impl.blockwise_head(*a, None, 3))
            w, lse = f(q, k, np.eye(n_kv), scale, causal, off)
            for i in range(n):
                if not mask[i].any():
                    assert np.all(w[i] == 0) and lse[i] == -np.inf, "empty row must be (0, -inf)"
                    continue
                ref_w = np.zeros(n_kv)
                ref_w[mask[i]] = softmax(logits[i, mask[i]])
                _close(w[i], ref_w, 1e-13, f"{form} weights row {i}")
                _close(lse[i], logsumexp(logits[i, mask[i]]), 1e-13, f"{form} lse row {i}")
                assert np.all(w[i] >= 0) and abs(w[i].sum() - 1.0) < 1e-13, "weights must be >= 0 and sum to 1"


def _brute(q, k, v, scale, causal, off):
    n, n_kv, dv = len(q), len(k), len(v[0])
    o, lse = [], []
    for i in range(n):
        keys = [j for j in range(n_kv) if (not causal) or j <= i + off]
        if not keys:
            o.append([0.0] * dv)
            lse.append(-math.inf)
            continue
        logit = {j: scale * math.fsum(q[i][c] * k[j][c] for c in range(len(q[i]))) for j in keys}
        top = max(logit.values())
        wsum = math.fsum(math.exp(logit[j] - top) for j in keys)
        o.append([math.fsum(math.exp(logit[j] - top) * v[j][c] for j in keys) / wsum for c in range(dv)])
        lse.append(top + math.log(wsum))
    return np.array(o), np.array(lse)


def check_bruteforce(impl, seed=13):
    rng = np.random.default_rng(seed)
    for _ in range(12):
        n, n_kv = int(rng.integers(1, 7)), int(rng.integers(1, 7))
        d, dv = int(rng.integers(1, 5)), int(rng.integers(1, 4))
        causal = bool(rng.integers(0, 2))
        scale = float(rng.uniform(0.2, 2.0))
        q, k, v = _rand(rng, n, n_kv, d, dv, std=1.5)
        off = n_kv - n
        o_ref, lse_ref = _brute(q.tolist(), k.tolist(), v.tolist(), scale, causal, off)
        for name, (o, lse) in {
            "naive": impl.naive_head(q, k, v, scale, causal, off),
            "blockwise": impl.blockwise_head(q, k, v, scale, causal, off, None, 2),
            "chunked": impl.chunked_head(q, k, v, scale, causal, off, None, 3),
        }.items():
            _close(o, o_ref, 1e-12, f"brute {name} O n={n} n_kv={n_kv} causal={causal}")
            _close(lse, lse_ref, 1e-12, f"brute {name} lse")


def check_closed_forms(impl, seed=14):
    rng = np.random.default_rng(seed)
    n, n_kv, d = 6, 9, 5
    _, k, v = _rand(rng, n, n_kv, d)
    zero_q = np.zeros((n, d))
    # Q = 0: every visible key has logit 0 -> the mean of the visible V rows, lse = ln(count)
    for causal in (False, True):
        off = n_kv - n
        for f in (lambda *a: impl.naive_head(*a), lambda *a: impl.blockwise_head(*a, None, 4),
                  lambda *a: impl.chunked_head(*a, None, 4)):
            o, lse = f(zero_q, k, v, 0.7, causal, off)
            for i in range(n):
                cnt = n_kv if not causal else i + off + 1
                _close(o[i], v[:cnt].mean(axis=0), 1e-13, f"Q=0 mean row {i} causal={causal}")
                _close(lse[i], math.log(cnt), 1e-13, f"Q=0 lse row {i}")
    # one key: O = V_0, lse = s * q.k_0
    q1, k1, v1 = _rand(rng, 4, 1, 3)
    o, lse = impl.naive_head(q1, k1, v1, 0.9)
    _close(o, np.repeat(v1, 4, axis=0), 1e-14, "one key O")
    _close(lse, 0.9 * (q1 @ k1[0]), 1e-14, "one key lse")
    # two keys: weight of key 0 is the logistic function of the logit gap
    q2, k2, v2 = _rand(rng, 5, 2, 3)
    o, lse = impl.naive_head(q2, k2, v2, 1.2)
    s0, s1 = 1.2 * (q2 @ k2[0]), 1.2 * (q2 @ k2[1])
    w0 = 1.0 / (1.0 + np.exp(s1 - s0))
    _close(o, w0[:, None] * v2[0] + (1 - w0)[:, None] * v2[1], 1e-13, "two keys O")
    _close(lse, np.logaddexp(s0, s1), 1e-13, "two keys lse")
    # a dominant key (logit gap >= 60) selects its V row
    kd = rng.standard_normal((n_kv, d)) * 0.01
    qd = np.zeros((3, d))
    qd[:, 0] = 1.0
    kd[4, 0] = 80.0
    o, _ = impl.naive_head(qd, kd, v, 1.0)
    _close(o, np.repeat(v[4:5], 3, axis=0), 1e-20 + 1e-14, "dominant key")
    o, _ = impl.blockwise_head(qd, kd, v, 1.0, False, None, None, 3)
    _close(o, np.repeat(v[4:5], 3, axis=0), 1e-14, "dominant key blockwise")
    # constant V is reproduced exactly by any convex combination
    q3, k3, _ = _rand(rng, 5, 7, 4)
    o, _ = impl.blockwise_head(q3, k3, np.full((7, 3), 2.5), 1.0, True, 2, None, 2)
    _close(o, np.full((5, 3), 2.5), 1e-14, "constant V")


def check_empty_rows(impl):
    rng = np.random.default_rng(15)
    q, k, v = _rand(rng, 6, 3, 2)
    # offset -3: queries 0..2 see no key
    for f in (lambda *a: impl.naive_head(*a), lambda *a: impl.blockwise_head(*a, None, 2),
              lambda *a: impl.chunked_head(*a, None, 2)):
        o, lse = f(q, k, v, 1.0, True, -3)
        assert np.all(o[:3] == 0) and np.all(lse[:3] == -np.inf), "rows without keys must be (0, -inf)"
        assert np.all(np.isfinite(o[3:])) and np.all(np.isfinite(lse[3:]))


def check_blockwise_vs_naive(impl, seed=16):
    rng = np.random.default_rng(seed)
    n, n_kv, d = 13, 21, 6
    for std in (1.0, 10.0, 30.0, 1000.0):
        q, k, v = _rand(rng, n, n_kv, d, std=std)
        for sort_keys in (None, "up", "down"):
            kk = k.copy()
            if sort_keys:   # "up": the running max of query 0 rises on every block; "down": it never does,
                # and with std 1000 any exponent not taken against the running max overflows
                order = np.argsort(kk @ q[0])
                kk = kk[order if sort_keys == "up" else order[::-1]]
            for causal in (False, True):
                o_ref, lse_ref = impl.naive_head(q, kk, v, 0.4, causal, n_kv - n)
                for blk in (1, 2, 3, 5, 7, 16, n_kv):
                    o, lse = impl.blockwise_head(q, kk, v, 0.4, causal, n_kv - n, None, blk)
                    _close(o, o_ref, 1e-12, f"blockwise({blk}) std={std} sorted={sort_keys} causal={causal}")
                    _close(lse, lse_ref, 1e-12, f"blockwise({blk}) lse")


def check_merge_algebra(impl, seed=17):
    rng = np.random.default_rng(seed)
    r, d = 7, 4
    parts = [(rng.standard_normal((r, d)), rng.standard_normal(r) * 3) for _ in range(3)]
    (oa, la), (ob, lb), (oc, lc) = parts
    x = impl.merge(oa, la, ob, lb)
    y = impl.merge(ob, lb, oa, la)
    _close(x[0], y[0], 1e-14, "commutative O")
    _close(x[1], y[1], 1e-14, "commutative lse")
    left = impl.merge(*impl.merge(oa, la, ob, lb), oc, lc)
    right = impl.merge(oa, la, *impl.merge(ob, lb, oc, lc))
    _close(left[0], right[0], 1e-13, "associative O")
    _close(left[1], right[1], 1e-13, "associative lse")
    ident = impl.merge(oa, la, np.zeros((r, d)), np.full(r, -np.inf))
    _close(ident[0], oa, 1e-15, "identity O")
    _close(ident[1], la, 1e-15, "identity lse")
    eq = impl.merge(oa, la, ob, la)
    _close(eq[0], (oa + ob) / 2, 1e-14, "equal lse O")
    _close(eq[1], la + math.log(2), 1e-14, "equal lse lse")
    both = impl.merge(oa, np.full(r, -np.inf), ob, np.full(r, -np.inf))
    assert np.all(both[0] == 0) and np.all(both[1] == -np.inf), "two empty partials stay empty"
    # two-way split of the keys = single pass
    q, k, v = _rand(rng, 5, 9, 3)
    full = impl.naive_head(q, k, v, 0.8)
    a = impl.naive_head(q, k[:4], v[:4], 0.8, False, 4)
    b = impl.naive_head(q, k[4:], v[4:], 0.8, False, 0)
    m = impl.merge(*a, *b)
    _close(m[0], full[0], 1e-13, "split O")
    _close(m[1], full[1], 1e-13, "split lse")


def check_chunked_every_p(impl, seed=18):
    rng = np.random.default_rng(seed)
    for n, n_kv in [(6, 10), (10, 6), (8, 8)]:
        q, k, v = _rand(rng, n, n_kv, 3)
        for causal in (False, True):
            o_ref, lse_ref = impl.naive_head(q, k, v, 0.9, causal, n_kv - n)
            for p in range(1, n_kv + 3):
                o, lse = impl.chunked_head(q, k, v, 0.9, causal, n_kv - n, None, p)
                _close(o, o_ref, 1e-13, f"chunked P={p} n={n} n_kv={n_kv} causal={causal}")
                _close(lse, lse_ref, 1e-13, f"chunked P={p} lse")


def check_permutation(impl, seed=19):
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 7, 12, 4)
    perm = rng.permutation(12)
    a = impl.naive_head(q, k, v, 0.6)
    b = impl.blockwise_head(q, k[perm], v[perm], 0.6, False, None, None, 5)
    _close(a[0], b[0], 1e-13, "permutation O")
    _close(a[1], b[1], 1e-13, "permutation lse")


def check_row_positions(impl, seed=20):
    """Queries evaluated at explicit positions equal the same rows of the full evaluation."""
    rng = np.random.default_rng(seed)
    q, k, v = _rand(rng, 12, 15, 3)
    rows = np.array([0, 3, 7, 11])
    for causal in (False, True):
        full = impl.naive_head(q, k, v, 0.5, causal, 3)
        for f in (lambda *a: impl.naive_head(*a), lambda *a: impl.blockwise_head(*a, 4)):
            part = f(q[rows], k, v, 0.5, causal, 3, rows)
            _close(part[0], full[0][rows], 1e-14, "row positions O")
            _close(part[1], full[1][rows], 1e-14, "row positions lse")


def check_batched_front_end(impl, seed=21):
    """The batched front end over [B=2, H=3] heads (each head drawn with its own scale of values, so a head
    mix-up shows) against the pure-Python brute force of every head on its own, for both forms, one and
    three chunks, causal with N_q < N_kv, N_q > N_kv and an explicit offset, and non-causal."""
    rng = np.random.default_rng(seed)
    B, H = 2, 3
    for n, n_kv, causal, off in [(5, 8, True, None), (8, 5, True, None), (6, 7, True, 2), (4, 6, False, None)]:
        d, dv = 3, 2
        scale_h = np.arange(1, B * H + 1, dtype=np.float64).reshape(B, H, 1, 1)
        q = rng.standard_normal((B, H, n, d))
        k = rng.standard_normal((B, H, n_kv, d))
        v = rng.standard_normal((B, H, n_kv, dv)) * scale_h + 10.0 * scale_h
        eff = n_kv - n if off is None else off
        ref_o = np.zeros((B, H, n, dv))
        ref_l = np.zeros((B, H, n))
        for b in range(B):
            for h in range(H):
                o_bh, l_bh = _brute(q[b, h].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.7, causal, eff)
                ref_o[b, h], ref_l[b, h] = o_bh, l_bh
        for form in ("naive", "blockwise"):
            for chunks in (1, 3):
                o, lse = impl.attention(q, k, v, 0.7, causal, off, form=form, block=2, chunks=chunks)
                what = f"batched {form} chunks={chunks} n={n} n_kv={n_kv} causal={causal} offset={off}"
                _close(o, ref_o, 1e-12, what + " O")
                _close(lse, ref_l, 1e-12, what + " lse")


ALL_CHECKS = [check_golden_attention, check_golden_merge, check_torch_sdpa, check_scipy_softmax,
              check_bruteforce, check_closed_forms, check_empty_rows, check_blockwise_vs_naive,
              check_merge_algebra, check_chunked_every_p, check_permutation, check_row_positions,
              check_batched_front_end]
