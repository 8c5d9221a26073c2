"""GPU parity: the HIP path (called through the C ABI) against the fp64 CPU oracle, element by element.

Small shapes are compared in full; they span several query and key tiles and end in ragged tails.  The five
measured workloads run at full size in the launch configuration the bench times, and are compared on
seeded query rows that the oracle evaluates one by one (64 per head).  Invariants that hold at any size
(determinism, NaN-poisoned outputs overwritten, chunked = single pass) are checked on the GPU as well.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import oracle
import workloads as W
from parity import assert_parity, errors, out_to_f64, storage_to_f64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


def make(w: W.Workload):
    """Seeded storage arrays and device tensors for a workload."""
    st = [W.tensor_storage(w, t) for t in (W.Q_T, W.K_T, W.V_T)]
    return st, [to_device(s) for s in st]


def oracle_full(st, w, chunks=1):
    q, k, v = (storage_to_f64(s) for s in st)
    return oracle.attention(q, k, v, w.scale, w.causal, w.offset, chunks=chunks)


def rows_for(w: W.Workload, b: int, h: int, n: int = 64) -> np.ndarray:
    if w.sample_rows:
        return W.sample_rows(w, b, h)
    rng = np.random.default_rng((w.seed, 77, b, h))
    r = rng.choice(w.N_q, size=min(n, w.N_q), replace=False)
    return np.unique(np.concatenate([r, [0, w.N_q - 1]]))


def check_sampled(w, st, o_dev, lse_dev, heads=None, what=""):
    """Compare sampled rows of every head (or the given heads) against the oracle's row-by-row result."""
    o_all, l_all = [], []
    ref_o, ref_l = [], []
    for b in range(w.B):
        for h in range(w.H):
            if heads is not None and (b, h) not in heads:
                continue
            rows = rows_for(w, b, h)
            q = storage_to_f64(st[0][b, h][rows])
            k = storage_to_f64(st[1][b, h])
            v = storage_to_f64(st[2][b, h])
            o_r, l_r = oracle.naive_head(q, k, v, w.scale, w.causal, w.offset, rows)
            idx = torch.from_numpy(rows).cuda()
            o_all.append(out_to_f64(o_dev[b, h].index_select(0, idx)))
            l_all.append(out_to_f64(lse_dev[b, h].index_select(0, idx)))
            ref_o.append(o_r)
            ref_l.append(l_r)
    err = errors(np.concatenate(o_all), np.concatenate(l_all), np.concatenate(ref_o), np.concatenate(ref_l))
    print(f"{what} {err}", flush=True)
    assert_parity(err, w.dtype, what)
    return err


def oracle_every_row(w, st, rb: int = 256, kb: int = 1024):
    """The oracle's result for every row of every head: its blockwise form (key blocks of ``kb``), over row
    blocks of ``rb`` queries on a thread pool of this host's cores (one BLAS thread each).  A causal row block
    is given only the keys up to its last visible one: key blocks past it are wholly masked for every row
    of the block and leave the running max, denominator and output unchanged, so this is the same result."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    o = np.empty((w.B, w.H, w.N_q, st[2].shape[-1]))
    lse = np.empty((w.B, w.H, w.N_q))
    with threadpool_limits(limits=1, user_api="blas"), ThreadPoolExecutor(workers) as ex:
        for b in range(w.B):
            for h in range(w.H):
                q, k, v = (storage_to_f64(s[b, h]) for s in st)

                def job(r0):
                    rows = np.arange(r0, min(r0 + rb, w.N_q))
                    end = w.N_kv if not w.causal else max(0, min(w.N_kv, int(rows[-1]) + w.offset + 1))
                    o[b, h, rows], lse[b, h, rows] = oracle.blockwise_head(q[rows], k[:end], v[:end], w.scale,
                                                                           w.causal, w.offset, rows, kb)

                list(ex.map(job, range(0, w.N_q, rb)))
    return o, lse


def check_every_row(w, o_ref, l_ref, o_dev, lse_dev, what=""):
    err = errors(out_to_f64(o_dev), out_to_f64(lse_dev), o_ref, l_ref)
    print(f"{what} {err}", flush=True)
    assert_parity(err, w.dtype, what)
    return err


# ------------------------------------------------------------------------------ small shapes, full compare
SMALL = [
    # B, H, N_q, N_kv, d, causal, dtype
    (1, 2, 300, 777, 128, False, "bf16"),
    (1, 2, 300, 777, 128, True, "bf16"),
    (2, 1, 333, 333, 128, True, "bf16"),
    (1, 2, 257, 1000, 64, True, "bf16"),
    (1, 2, 1000, 257, 64, True, "bf16"),    # N_q > N_kv: the first rows see no key
    (1, 1, 1, 1, 128, False, "bf16"),
    (1, 3, 5, 3, 64, False, "bf16"),
    (1, 1, 129, 65, 64, False, "bf16"),
    (1, 1, 640, 640, 128, True, "bf16"),
    (1, 2, 200, 300, 64, False, "f32"),
    (1, 2, 130, 70, 37, True, "f32"),
    (1, 1, 64, 64, 256, True, "f32"),
    (1, 1, 1, 5, 1, False, "f32"),
    (2, 2, 100, 100, 128, True, "f32"),
]


def small_workload(i, case, q_std=1.0):
    B, H, N_q, N_kv, d, causal, dt = case
    return W.Workload(f"small{i}", B, H, N_q, N_kv, d, dt, causal, 1, seed=1000 + i, q_std=q_std)


@pytest.mark.parametrize("i", range(len(SMALL)), ids=lambda i: "x".join(map(str, SMALL[i][:5])) +
                         ("c" if SMALL[i][5] else "n") + SMALL[i][6])
def test_small_full(i):
    w = small_workload(i, SMALL[i])
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    o, lse = A.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
    print(w, err, flush=True)
    assert_parity(err, w.dtype, w.name)
    for P in sorted({2, 3, 7, w.N_kv + 2}):
        o, lse = A.fwd_chunked(q, k, v, P, causal=w.causal, scale=w.scale)
        torch.cuda.synchronize()
        err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
        assert_parity(err, w.dtype, f"{w.name} chunks={P}")


# The bf16 kernel runs as four-wave (128-row) or eight-wave (256-row) workgroups, chosen by the launch size;
# ATTN_BF16_D128_WAVES and ATTN_BF16_D64_WAVES force one.  Every shape below runs through both at both head
# dimensions, against the oracle, and the two must agree bit for bit (each row sees the same tiles in the
# same order either way).
WG_SHAPES = [
    # B, H, N_q, N_kv, causal
    (1, 2, 300, 777, False),
    (1, 2, 300, 777, True),
    (2, 1, 333, 333, True),
    (1, 1, 1000, 257, True),     # the first rows see no key
    (1, 1, 257, 1000, True),
    (1, 1, 700, 700, False),     # three 256-row workgroups, the last one ragged
    (1, 2, 513, 1500, True),
    (1, 1, 1, 64, False),
    (1, 1, 64, 1, True),
    (1, 1, 256, 4100, False),    # many tiles, then a ragged one
]


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("case", WG_SHAPES, ids=lambda c: "x".join(map(str, c[:4])) + ("c" if c[4] else "n"))
def test_bf16_both_workgroup_sizes(case, d, monkeypatch):
    B, H, N_q, N_kv, causal = case
    w = W.Workload(f"d{d}wg", B, H, N_q, N_kv, d, "bf16", causal, 1, seed=3000 + N_q + N_kv + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    outs = {}
    for waves in ("4", "8"):
        monkeypatch.setenv(f"ATTN_BF16_D{d}_WAVES", waves)
        o, lse = A.fwd(q, k, v, causal=causal, scale=w.scale)
        o32, l32 = A.fwd_ex(q, k, v, causal=causal, scale=w.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
        print(w, waves, err, flush=True)
        assert_parity(err, "bf16", f"{w.name} waves={waves}")
        outs[waves] = (o.cpu(), lse.cpu(), o32.cpu(), l32.cpu())
    for a_, b_ in zip(outs["4"], outs["8"]):
        assert torch.equal(a_, b_), "four- and eight-wave workgroups disagree"


# The fp32 kernel shares a query row among 4, 8 or 16 lanes, chosen by the launch size (16 only at d > 32);
# ATTN_F32_LANES_PER_ROW forces one.  Every shape runs through each, chunked (folded partials) and not,
# against the oracle; the head dimensions cover every template (d <= 32, 64, 128, 256) and both load paths
# (float4 rows at d % 4 == 0, element loads otherwise).
F32_SHAPES = [
    # B, H, N_q, N_kv, d, causal
    (1, 2, 200, 300, 64, False),
    (1, 2, 130, 70, 37, True),
    (1, 1, 64, 64, 256, True),
    (1, 1, 100, 333, 200, False),
    (1, 1, 1, 5, 1, False),
    (2, 2, 100, 100, 128, True),
    (1, 1, 77, 129, 30, True),
]


@pytest.mark.parametrize("lanes", ["4", "8", "16"])
@pytest.mark.parametrize("case", F32_SHAPES, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else "n"))
def test_f32_lanes_per_row(case, lanes, monkeypatch):
    B, H, N_q, N_kv, d, causal = case
    monkeypatch.setenv("ATTN_F32_LANES_PER_ROW", lanes)
    w = W.Workload("f32lanes", B, H, N_q, N_kv, d, "f32", causal, 1, seed=3400 + N_q + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    o, lse = A.fwd(q, k, v, causal=causal, scale=w.scale)
    oc, lc = A.fwd_chunked(q, k, v, 3, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), "f32", f"{w} lanes={lanes}")
    assert_parity(errors(out_to_f64(oc), out_to_f64(lc), o_ref, l_ref), "f32", f"{w} lanes={lanes} 3 chunks")


# Long rows with peaky logits (std 6) in fp32: the weighted rows are summed per key tile before they join the running
# sums, so the rounding grows with the number of tiles, not of keys (summed key by key, the second and third shapes
# reached max-abs 2.1e-5 and 1.6e-5 against the 1e-5 bar, at every lanes-per-row choice).
F32_PEAKY = [
    # B, H, N_q, N_kv, d
    (2, 1, 78, 2187, 8),
    (1, 2, 200, 4000, 64),
    (1, 1, 130, 3000, 128),
]


@pytest.mark.parametrize("lanes", ["4", "8", "16"])
@pytest.mark.parametrize("case", F32_PEAKY, ids=lambda c: "x".join(map(str, c)))
def test_f32_long_peaky_rows(case, lanes, monkeypatch):
    B, H, N_q, N_kv, d = case
    monkeypatch.setenv("ATTN_F32_LANES_PER_ROW", lanes)
    w = W.Workload("f32peaky", B, H, N_q, N_kv, d, "f32", False, 1, seed=5100 + d, q_std=6.0)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    o, lse = A.fwd(q, k, v, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
    print(w.name, case, lanes, err, flush=True)
    assert_parity(err, "f32", f"{case} lanes={lanes}")


def test_f32_large_launch():
    """An fp32 launch large enough for four lanes per row on its own (1024 workgroups of 64 rows), with
    tiles in flight across many steps: sampled rows against the oracle."""
    w = W.Workload("f32big", 1, 16, 4096, 2048, 64, "f32", True, 1, seed=3500)
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    check_sampled(w, st, o, lse, what="fp32 16 heads x 4096 rows")


@pytest.mark.parametrize("case", [(7, 73, 40, 70, 128, "bf16"), (7, 73, 40, 70, 64, "bf16"),
                                  (5, 61, 33, 20, 48, "f32")],
                         ids=lambda c: "x".join(map(str, c[:5])) + c[5])
def test_many_heads(case):
    """Hundreds of (b, h) pairs with short rows: the head indexing and the XCD-aware workgroup order at a
    workgroup count that is not a multiple of 8, causal with N_q < N_kv, chunked as well."""
    B, H, N_q, N_kv, d, dt = case
    w = W.Workload("heads", B, H, N_q, N_kv, d, dt, True, 1, seed=3600 + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    o, lse = A.fwd(q, k, v, causal=True, scale=w.scale)
    oc, lc = A.fwd_chunked(q, k, v, 3, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), dt, f"{w}")
    assert_parity(errors(out_to_f64(oc), out_to_f64(lc), o_ref, l_ref), dt, f"{w} 3 chunks")


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.5])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_unusual_scales(scale, dt):
    w = W.Workload("scales", 1, 2, 190, 260, 128 if dt == "bf16" else 64, dt, True, 1, seed=2000)
    st, (q, k, v) = make(w)
    qq, kk, vv = (storage_to_f64(s) for s in st)
    o_ref, l_ref = oracle.attention(qq, kk, vv, scale, True, w.offset)
    o, lse = A.fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), dt, f"scale={scale}")


@pytest.mark.parametrize("d", [64, 128])
def test_peaky_sorted_keys_rescale_every_tile(d):
    """Keys sorted by ascending logit for query 0: its running max rises on every key tile."""
    w = W.Workload("sorted", 1, 1, 256, 2048, d, "bf16", False, 1, seed=2100, q_std=4.0)
    st, _ = make(w)
    q64 = storage_to_f64(st[0][0, 0])
    order = np.argsort(storage_to_f64(st[1][0, 0]) @ q64[0])
    st[1] = st[1][:, :, order].copy()
    st[2] = st[2][:, :, order].copy()
    q, k, v = (to_device(s) for s in st)
    o_ref, l_ref = oracle_full(st, w)
    o, lse = A.fwd(q, k, v, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), "bf16", "sorted keys")


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("d", [64, 128])
def test_stale_reference_envelope(d, waves, monkeypatch):
    """The exponent reference stays at the row max of the first key tile here: every later tile holds one key about
    63 exp2-units above it, just under the 2^64 weight-sum bound that would move it, and that key's V entries are
    near 2^58.  The fp32 accumulators then reach ~2^125.5, near the edge of the envelope the bf16 kernel states for
    its stale reference (at most 2^64 per tile x tiles x max|V|, below 2^128).  The result still matches the oracle
    (which keeps the running max), compared in units of 2^58."""
    monkeypatch.setenv(f"ATTN_BF16_D{d}_WAVES", waves)
    B, H, nq, nkv = 1, 2, 64, 1024
    scale = 1.0 / math.sqrt(d)
    c = scale * math.log2(math.e)
    rng = np.random.default_rng(2300 + d)
    q = np.zeros((B, H, nq, d), np.float32)
    q[..., 0] = 1.0
    q[..., 1] = rng.choice([-0.5, 0.5], (B, H, nq))
    k = np.zeros((B, H, nkv, d), np.float32)
    k[..., 1] = rng.choice([-1.0, 1.0], (B, H, nkv))
    big = 64 * np.arange(1, nkv // 64) + rng.integers(0, 64, nkv // 64 - 1)   # one key in every tile after the first
    k[:, :, big, 0] = np.float32(round(63.0 / c))
    v = rng.standard_normal((B, H, nkv, d)).astype(np.float32)
    v[:, :, big, :] = np.float32(2.0 ** 58) * rng.choice([0.75, 1.0, 1.25, 1.5], (B, H, len(big), d)).astype(np.float32)
    st = [W.f32_to_bf16_bits(x) for x in (q, k, v)]
    qq, kk, vv = (storage_to_f64(x) for x in st)
    top = (kk[0, 0, big, 0] - 0.5) * c   # the big keys' exponents against the first tile's max (0.5)
    assert top.max() < 64.0 and top.min() > 62.0, "the test keys sit just under the bound that moves the reference"
    o_ref, l_ref = oracle.attention(qq, kk, vv, scale, False, nkv - nq)
    o, lse = A.fwd(*(to_device(x) for x in st), causal=False, scale=scale)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o) / 2.0 ** 58, out_to_f64(lse), o_ref / 2.0 ** 58, l_ref)
    print(f"d={d} waves={waves}", err, flush=True)
    assert_parity(err, "bf16", f"envelope d={d} waves={waves}")


def test_key_range_and_offset_partials():
    """attn_fwd_ex over two key ranges (fp32 partials with explicit offsets) merged = the whole."""
    w = W.Workload("ranges", 1, 2, 384, 1000, 128, "bf16", True, 1, seed=2200)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    cut = 437
    off = w.N_kv - w.N_q
    oa, la = A.fwd_ex(q, k, v, True, w.scale, causal_offset=off, key_range=(0, cut), out_dtype=torch.float32)
    ob, lb = A.fwd_ex(q, k, v, True, w.scale, causal_offset=off - cut, key_range=(cut, w.N_kv),
                      out_dtype=torch.float32)
    o, lse = A.merge(oa, la, ob, lb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), "bf16", "two ranges merged")
    # the fp32 partials themselves against the oracle's partials
    qq, kk, vv = (storage_to_f64(s) for s in st)
    pa = oracle.attention(qq, kk[:, :, :cut], vv[:, :, :cut], w.scale, True, off)
    err = errors(out_to_f64(oa), out_to_f64(la), *pa)
    assert_parity(err, "bf16", "partial a")


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f32", 64)])
def test_merge_grouping_does_not_matter(dt, d):
    """Partials over five ragged key ranges (fp32, explicit causal offsets) combined with attn_merge in four
    groupings: left fold, right fold, a balanced tree and a shuffled order.  The merge is associative and
    commutative ("ATTENTION2D" explainer, section 2), so each equals the oracle's whole within tolerance,
    the property the 2-D and ring schemes rely on when partials arrive in any order."""
    w = W.Workload("groupings", 1, 2, 300, 1111, d, dt, True, 1, seed=2300 + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    cuts = [0, 97, 410, 411, 800, w.N_kv]          # one range of a single key
    off = w.N_kv - w.N_q
    parts = [A.fwd_ex(q, k, v, True, w.scale, causal_offset=off - lo, key_range=(lo, hi), out_dtype=torch.float32)
             for lo, hi in zip(cuts[:-1], cuts[1:])]
    m = lambda a, b: A.merge(a[0], a[1], b[0], b[1])
    left = parts[0]
    for p_ in parts[1:]:
        left = m(left, p_)
    right = parts[-1]
    for p_ in reversed(parts[:-1]):
        right = m(p_, right)
    tree = m(m(parts[0], parts[1]), m(parts[2], m(parts[3], parts[4])))
    shuffled = m(m(parts[3], parts[0]), m(m(parts[4], parts[2]), parts[1]))
    torch.cuda.synchronize()
    results = {"left fold": left, "right fold": right, "tree": tree, "shuffled": shuffled}
    for name, (o, lse) in results.items():
        err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
        print(f"{dt} d{d} {name}: {err}", flush=True)
        assert_parity(err, "f32" if dt == "f32" else "bf16", f"merge grouping {name}")
        if dt == "f32":   # fp32 partials from fp32 inputs: the groupings differ only in rounding
            assert float((o - left[0]).abs().max()) <= 1e-6


# ------------------------------------------------------------------------- fused fold of a key range (acc)
@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 37)])
@pytest.mark.parametrize("causal", [False, True])
def test_fwd_acc_vs_oracle(dt, d, causal):
    """attn_fwd_acc folds key ranges into a running fp32 partial in the kernel epilogue: three ranges
    (the middle one folded in place, the last one written in the input dtype) equal the whole; the causal
    case has query rows that see nothing in the later ranges and rows that see nothing in the first."""
    w = W.Workload("acc", 1, 2, 300, 700, d, dt, causal, 1, seed=2300 + d + 7 * causal)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    off = w.N_kv - w.N_q if causal else 0
    a, b = 250, 520
    oa, la = A.fwd_ex(q, k, v, causal, w.scale, causal_offset=off, key_range=(0, a), out_dtype=torch.float32)
    res = A.fwd_acc(q, k, v, oa, la, causal, w.scale, causal_offset=off - a, key_range=(a, b),
                    out_dtype=torch.float32, out=oa, lse=la)
    assert res[0].data_ptr() == oa.data_ptr()
    o, lse = A.fwd_acc(q, k, v, oa, la, causal, w.scale, causal_offset=off - b, key_range=(b, w.N_kv))
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
    print(w, err, flush=True)
    assert_parity(err, dt, f"three ranges folded, {dt} d{d}")
    # the same fold against the separate merge kernel: equal up to rounding
    ob, lb = A.fwd_ex(q, k, v, causal, w.scale, causal_offset=off - b, key_range=(b, w.N_kv),
                      out_dtype=torch.float32)
    om, lm = A.merge(oa, la, ob, lb, out_dtype=q.dtype)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), out_to_f64(om), out_to_f64(lm)), dt, "fold vs merge")


def test_fwd_acc_empty_partial_is_identity():
    """A partial of all-empty rows (lse = -inf, O = 0) folded with a range gives that range's result."""
    w = W.Workload("acc0", 1, 2, 200, 300, 128, "bf16", False, 1, seed=2400)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    oa = torch.zeros((1, 2, 200, 128), dtype=torch.float32, device="cuda")
    la = torch.full((1, 2, 200), -math.inf, dtype=torch.float32, device="cuda")
    o, lse = A.fwd_acc(q, k, v, oa, la, False, w.scale)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), "bf16", "identity partial")


# ------------------------------------------------------------------------------------------------- merge
MERGE_CASES = [("f32", "f32", 128), ("f32", "bf16", 128), ("bf16", "bf16", 64), ("bf16", "f32", 128),
               ("f32", "f32", 4), ("f32", "f32", 96), ("f32", "f32", 256), ("f32", "f32", 260),
               ("f32", "f32", 37), ("bf16", "f32", 5)]


def merge_inputs(rng, rows, d, din):
    oa, ob = rng.standard_normal((rows, d)).astype(np.float32), rng.standard_normal((rows, d)).astype(np.float32)
    la, lb = (rng.standard_normal(rows) * 5).astype(np.float32), (rng.standard_normal(rows) * 5).astype(np.float32)
    la[::7] = -np.inf
    lb[::11] = -np.inf
    oa[::7] = 0
    ob[::11] = 0
    if din == "bf16":
        oa, ob = W.f32_to_bf16_bits(oa), W.f32_to_bf16_bits(ob)
    return oa, la, ob, lb


@pytest.mark.parametrize("din,dout,d", MERGE_CASES)
def test_merge_vs_oracle(din, dout, d):
    """Row-per-wave kernel (d a multiple of 4 up to 256: lane groups of 1 to 64 lanes per row, idle lanes
    at d = 96) and the whole-row workgroup kernel (d = 260, 37, 5); 3001 rows leave a ragged last group."""
    rng = np.random.default_rng(3000 + d)
    rows = 3001
    oa, la, ob, lb = merge_inputs(rng, rows, d, din)
    ref_o, ref_l = oracle.merge(storage_to_f64(oa), la.astype(np.float64), storage_to_f64(ob), lb.astype(np.float64))
    tdt = torch.bfloat16 if dout == "bf16" else torch.float32
    o, lse = A.merge(to_device(oa), to_device(la), to_device(ob), to_device(lb), out_dtype=tdt)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), ref_o, ref_l)
    tol = 2e-2 if dout == "bf16" else 1e-5
    assert not err["nan"] and err["lse_inf_match"]
    assert err["max_abs"] <= tol and err["lse_abs"] <= 1e-5, err
    if dout == "bf16":   # the bf16 tolerance pair: rounding the merged rows to bf16 costs ~2^-9/sqrt(3) rel-RMS
        assert err["rel_rms"] <= 5e-3, err


@pytest.mark.parametrize("din,dout,d", [("f32", "f32", 128), ("bf16", "f32", 64)])
def test_merge_misaligned_buffers(din, dout, d):
    """Buffers aligned to their element size only: the launch falls back from vector loads."""
    rng = np.random.default_rng(3050 + d)
    rows = 1025
    oa, la, ob, lb = merge_inputs(rng, rows, d, din)
    ref_o, ref_l = oracle.merge(storage_to_f64(oa), la.astype(np.float64), storage_to_f64(ob), lb.astype(np.float64))

    def shifted(x):   # the same values one element past a 256-byte boundary
        t = to_device(x)
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        buf[1:].copy_(t.reshape(-1))
        return buf[1:].view(t.shape)

    tdt = torch.bfloat16 if dout == "bf16" else torch.float32
    out = torch.empty(rows * d + 1, dtype=tdt, device="cuda")[1:].view(rows, d)
    o, lse = A.merge(shifted(oa), to_device(la), shifted(ob), to_device(lb), out=out)
    torch.cuda.synchronize()
    assert o.data_ptr() % 16 != 0
    err = errors(out_to_f64(o), out_to_f64(lse), ref_o, ref_l)
    assert not err["nan"] and err["lse_inf_match"]
    assert err["max_abs"] <= 1e-5 and err["lse_abs"] <= 1e-5, err


@pytest.mark.parametrize("dout", ["f32", "bf16"])
def test_merge_large_streaming(dout):
    """A merge larger than twice the Infinity Cache takes the non-temporal path (two row groups in flight
    per lane): in place for fp32 out, fp32 -> bf16 out of place; 524,287 rows leave a ragged last group."""
    rng = np.random.default_rng(3070)
    rows, d = 524287, 128
    oa, la, ob, lb = merge_inputs(rng, rows, d, "f32")
    ref_o, ref_l = oracle.merge(oa.astype(np.float64), la.astype(np.float64), ob.astype(np.float64),
                                lb.astype(np.float64))
    ta, tla = to_device(oa), to_device(la)
    if dout == "f32":
        o, lse = A.merge(ta, tla, to_device(ob), to_device(lb), out=ta, lse=tla)
        assert o.data_ptr() == ta.data_ptr()
    else:
        o, lse = A.merge(ta, tla, to_device(ob), to_device(lb), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), ref_o, ref_l)
    assert not err["nan"] and err["lse_inf_match"]
    assert err["max_abs"] <= (2e-2 if dout == "bf16" else 1e-5) and err["lse_abs"] <= 1e-5, err


def test_binding_checks_caller_buffers():
    """The binding passes raw pointers on, so it refuses caller tensors whose shape, dtype or device differs
    from what the call reads or writes; a given output tensor decides the output dtype."""
    w = W.Workload("bind", 1, 2, 64, 96, 128, "bf16", False, 1, seed=3200)
    st, (q, k, v) = make(w)
    bad = [
        lambda: A.fwd(q, k, v, out=torch.empty(q.shape, dtype=torch.float32, device="cuda")),
        lambda: A.fwd(q, k, v, lse=torch.empty((1, 2, 63), dtype=torch.float32, device="cuda")),
        lambda: A.fwd(q, k, v[:, :, :95].contiguous()),
        lambda: A.fwd(q, k[:, :1].contiguous(), v[:, :1].contiguous()),
        lambda: A.fwd_ex(q, k, v, out=torch.empty(q.shape, dtype=torch.float32, device="cuda"),
                         out_dtype=torch.bfloat16),
        lambda: A.fwd_chunked(q, k, v, 2, workspace=torch.empty(1 << 20, dtype=torch.uint8)),
    ]
    oa = torch.zeros((10, 128), dtype=torch.float32, device="cuda")
    la = torch.zeros(10, dtype=torch.float32, device="cuda")
    bad += [
        lambda: A.merge(oa, la, oa.to(torch.bfloat16), la),
        lambda: A.merge(oa, la, oa[:9].contiguous(), la),
        lambda: A.merge(oa, la, oa, la, out=torch.empty((10, 64), device="cuda")),
        lambda: A.merge(oa, la, oa, la.to(torch.float64)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises((ValueError, TypeError)):
            call()
            pytest.fail(f"case {i} accepted")
    # bf16 inputs with an fp32 output tensor and no out_dtype: written as fp32
    o32 = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    o, _ = A.fwd_ex(q, k, v, out=o32)
    ref, _ = A.fwd_ex(q, k, v, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert o.data_ptr() == o32.data_ptr() and torch.equal(o32, ref)


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_graph_capture_and_replay(dt, d):
    """The chunked forward (three folded chunks, causal) and a merge captured into one HIP graph: nothing in
    them allocates, clears memory or synchronises, so replays equal the eager calls bit for bit.  Each replay
    runs on fresh inputs copied in by eager work, with synchronisations between replays."""
    w = W.Workload("graph", 1, 2, 200, 700, d, dt, True, 3, seed=3300 + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    ws = torch.empty(max(A.workspace_bytes(1, 2, 200, d, 3), 1), dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty((1, 2, 200), dtype=torch.float32, device="cuda")
    om = torch.empty((1, 2, 200, d), dtype=torch.float32, device="cuda")
    lm = torch.empty_like(lse)
    o32 = torch.empty((1, 2, 200, d), dtype=torch.float32, device="cuda")

    def work():
        A.fwd_chunked(q, k, v, 3, causal=True, scale=w.scale, out=o, lse=lse, workspace=ws)
        o32.copy_(o)
        A.merge(o32, lse, o32, lse, out=om, lse=lm)   # a row merged with itself: same O, lse + ln 2

    work()   # eager, also sets the kernels' LDS attributes before capture
    torch.cuda.synchronize()
    eager = [t.clone() for t in (o, lse, om, lm)]
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), dt, "eager chunked")
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            work()
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in (o, lse, om, lm):
            t.fill_(float("nan"))               # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((o, lse, om, lm), eager):
            assert torch.equal(got, want), f"replay {rep} differs from the eager result"


def test_merge_in_place():
    rng = np.random.default_rng(3100)
    rows, d = 4096, 128
    oa, ob = rng.standard_normal((rows, d)).astype(np.float32), rng.standard_normal((rows, d)).astype(np.float32)
    la, lb = rng.standard_normal(rows).astype(np.float32), rng.standard_normal(rows).astype(np.float32)
    ref_o, ref_l = oracle.merge(oa, la, ob, lb)
    ta, tla = to_device(oa), to_device(la)
    o, lse = A.merge(ta, tla, to_device(ob), to_device(lb), out=ta, lse=tla)
    torch.cuda.synchronize()
    assert o.data_ptr() == ta.data_ptr()
    err = errors(out_to_f64(ta), out_to_f64(tla), ref_o, ref_l)
    assert err["max_abs"] <= 1e-5 and err["lse_abs"] <= 1e-5, err


# --------------------------------------------------------------------------- invariants on the GPU itself
def test_determinism_and_poisoned_outputs():
    w = W.Workload("det", 2, 4, 1500, 1500, 128, "bf16", True, 1, seed=4000)
    st, (q, k, v) = make(w)
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((2, 4, 1500), float("nan"), device="cuda")
    A.fwd(q, k, v, causal=True, out=o1, lse=l1)
    o2, l2 = A.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_constant_v_gives_constant_output():
    w = W.Workload("ones", 1, 2, 700, 900, 128, "bf16", True, 1, seed=4100)
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, torch.ones_like(v), causal=True)
    torch.cuda.synchronize()
    assert (o.float() - 1).abs().max().item() <= 2e-2


# -------------------------------------------------------------------------- the measured workloads, full size
def test_tiny_fp32_full_and_4_chunks():
    w = W.WORKLOADS["tiny_fp32"]
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    o, lse = A.fwd(q, k, v, causal=w.causal, scale=w.scale)
    oc, lc = A.fwd_chunked(q, k, v, w.chunks, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert_parity(errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref), "f32", "tiny single pass")
    assert_parity(errors(out_to_f64(oc), out_to_f64(lc), o_ref, l_ref), "f32", "tiny 4 chunks")


def test_causal_prefill_4k():
    """Every row of every head against the oracle's blockwise form, and seeded rows against its plain form."""
    w = W.WORKLOADS["causal_prefill_4k"]
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    check_sampled(w, st, o, lse, what="causal_prefill_4k sampled")
    o_ref, l_ref = oracle_every_row(w, st)
    check_every_row(w, o_ref, l_ref, o, lse, what="causal_prefill_4k every row")


def test_peaky_16k():
    """Every row of every head against the oracle's blockwise form, and seeded rows against its plain form."""
    w = W.WORKLOADS["peaky_16k"]
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, v, causal=False, scale=w.scale)
    torch.cuda.synchronize()
    check_sampled(w, st, o, lse, what="peaky_16k sampled")
    o_ref, l_ref = oracle_every_row(w, st)
    check_every_row(w, o_ref, l_ref, o, lse, what="peaky_16k every row")


def test_causal_d64_prefill_every_row():
    """The d = 64 kernel on long causal rows (B4 H16, 4096 queries and keys, logits with std 4, so that single keys
    dominate rows and the denominator of the rounded weights matters): every row of every head against the
    oracle's blockwise form, and seeded rows against its plain form."""
    w = W.Workload("causal_d64_4k", 4, 16, 4096, 4096, 64, "bf16", True, 1, seed=4100, q_std=4.0)
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    check_sampled(w, st, o, lse, what="causal_d64_4k sampled")
    o_ref, l_ref = oracle_every_row(w, st)
    check_every_row(w, o_ref, l_ref, o, lse, what="causal_d64_4k every row")


def test_ring_share_128k_chunked():
    """The chunked step the bench times (8 chunks folded in the forward epilogues) and the single pass, each
    compared on every row of every head against the oracle's single-pass blockwise result."""
    w = W.WORKLOADS["ring_share_128k"]
    st, (q, k, v) = make(w)
    o, lse = A.fwd_chunked(q, k, v, w.chunks, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    check_sampled(w, st, o, lse, what="ring_share_128k 8 chunks sampled")
    o1, l1 = A.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_every_row(w, st)
    check_every_row(w, o_ref, l_ref, o, lse, what="ring_share_128k 8 chunks every row")
    check_every_row(w, o_ref, l_ref, o1, l1, what="ring_share_128k single pass every row")


def test_max_keys_per_launch():
    """The largest key count one bf16 d128 launch accepts (2^31-1 bytes of K and of V per head: 8,388,607
    keys, a ragged last tile), causal with 200 query rows: sampled rows against the oracle."""
    w = W.Workload("max_keys", 1, 1, 200, 8388607, 128, "bf16", True, 1, seed=4500)
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    del q, k, v
    check_sampled(w, st, o, lse, what="8,388,607 keys")


def test_ulysses_share_256k():
    w = W.WORKLOADS["ulysses_share_256k"]
    st, (q, k, v) = make(w)
    o, lse = A.fwd(q, k, v, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    check_sampled(w, st, o, lse, what="ulysses_share_256k seeded rows")


# ------------------------------------------------------------- K and V streamed from host memory (NEXT-2)
STREAMED = [
    # B, H, N_q, N_kv, d, causal, dtype, chunk counts
    (1, 2, 300, 777, 128, True, "bf16", (1, 3, 8)),
    (1, 2, 1000, 257, 64, True, "bf16", (2, 7)),      # N_q > N_kv: future chunks skipped, empty rows
    (1, 3, 5, 3, 64, False, "bf16", (5,)),           # more chunks than keys: empty chunks skipped
    (1, 2, 130, 70, 37, True, "f32", (1, 4)),
    (2, 1, 200, 300, 64, False, "f32", (3,)),
]


@pytest.mark.parametrize("case", STREAMED, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else "n") + c[6])
def test_streamed_equals_chunked(case):
    """attn_fwd_streamed (K, V in pinned host memory) gives exactly attn_fwd_chunked's result, and the oracle's."""
    B, H, N_q, N_kv, d, causal, dt, chunk_counts = case
    w = W.Workload("streamed", B, H, N_q, N_kv, d, dt, causal, 1, seed=4000 + N_q + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle_full(st, w)
    kh = k.cpu().pin_memory()
    vh = v.cpu().pin_memory()
    for P in chunk_counts:
        oc, lc = A.fwd_chunked(q, k, v, P, causal=causal, scale=w.scale)
        o, lse = A.fwd_streamed(q, kh, vh, P, causal=causal, scale=w.scale)
        torch.cuda.synchronize()
        err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
        print(w, P, err, flush=True)
        assert_parity(err, dt, f"streamed P={P}")
        assert torch.equal(o, oc) and torch.equal(lse, lc), f"streamed != chunked at P={P}"


def test_streamed_pageable_and_repeated_calls():
    """Pageable host memory gives the same result (serialised copies); back-to-back calls of different sizes
    reuse the library's synchronisation events without interfering."""
    w = W.Workload("streamed2", 1, 2, 256, 1500, 128, "bf16", True, 1, seed=4100)
    st, (q, k, v) = make(w)
    kh, vh = k.cpu(), v.cpu()
    kp, vp = kh.pin_memory(), vh.pin_memory()
    oc, lc = A.fwd_chunked(q, k, v, 6, causal=True, scale=w.scale)
    w2 = W.Workload("streamed3", 1, 1, 64, 200, 128, "bf16", False, 1, seed=4101)
    st2, (q2, k2, v2) = make(w2)
    oc2, lc2 = A.fwd_chunked(q2, k2, v2, 3, causal=False, scale=w2.scale)
    k2h, v2h = k2.cpu().pin_memory(), v2.cpu().pin_memory()
    outs = []
    for _ in range(2):
        outs.append(A.fwd_streamed(q, kp, vp, 6, causal=True, scale=w.scale))
        outs.append(A.fwd_streamed(q2, k2h, v2h, 3, causal=False, scale=w2.scale))
    outs.append(A.fwd_streamed(q, kh, vh, 6, causal=True, scale=w.scale))
    torch.cuda.synchronize()
    for i, (o, lse) in enumerate(outs):
        ref = (oc, lc) if i % 2 == 0 else (oc2, lc2)
        assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1]), f"call {i} differs from the chunked result"


def test_streamed_back_to_back_shared_workspace():
    """Two calls in a row with different host K/V, one explicit workspace and one non-blocking copy stream:
    the second call's first copies wait for the first call's last kernels (which still read the staging
    slots), so each result equals attn_fwd_chunked's bit for bit.  Many query rows against few keys make
    every chunk's kernel longer than its copy, the case where an unordered copy would overwrite a slot in use."""
    w1 = W.Workload("streamed_b2b_1", 1, 8, 65536, 4096, 128, "bf16", False, 1, seed=4300)
    w2 = W.Workload("streamed_b2b_2", 1, 8, 65536, 4096, 128, "bf16", False, 1, seed=4301)
    _, (q, k1, v1) = make(w1)
    _, (_, k2, v2) = make(w2)
    P = 8
    oc1, lc1 = A.fwd_chunked(q, k1, v1, P, scale=w1.scale)
    oc2, lc2 = A.fwd_chunked(q, k2, v2, P, scale=w1.scale)
    k1h, v1h, k2h, v2h = (t.cpu().pin_memory() for t in (k1, v1, k2, v2))
    ws = torch.empty(A.streamed_workspace_bytes(1, 8, 65536, 4096, 128, P, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    cs = torch.cuda.Stream()
    torch.cuda.synchronize()
    for _ in range(2):
        o1, l1 = A.fwd_streamed(q, k1h, v1h, P, scale=w1.scale, workspace=ws, copy_stream=cs)
        o2, l2 = A.fwd_streamed(q, k2h, v2h, P, scale=w1.scale, workspace=ws, copy_stream=cs)
        torch.cuda.synchronize()
        assert torch.equal(o1, oc1) and torch.equal(l1, lc1), "first call differs from the chunked result"
        assert torch.equal(o2, oc2) and torch.equal(l2, lc2), "second call differs from the chunked result"


def test_streamed_ring_share_full_size():
    """The ring-share workload (1 GiB of K and V in pinned host memory, 8 chunks) streamed equals the
    device-resident chunked path bit for bit."""
    w = W.WORKLOADS["ring_share_128k"]
    st, (q, k, v) = make(w)
    kh, vh = k.cpu().pin_memory(), v.cpu().pin_memory()
    oc, lc = A.fwd_chunked(q, k, v, w.chunks, causal=w.causal, scale=w.scale)
    o, lse = A.fwd_streamed(q, kh, vh, w.chunks, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    check_sampled(w, st, o, lse, heads=[(0, 0), (0, 31)], what="ring_share_128k streamed")
