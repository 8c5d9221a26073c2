"""Properties of exact attention that hold at any size, checked on the GPU at long key counts without the
oracle (the pages define attention as a row softmax of the scores times V: "FlashAttention by hand",
paragraph on the three standard steps, and the single final division):

  * zero queries make every score 0, so each row's weights are uniform over its visible keys: O_i is the
    mean of the visible V rows (a prefix mean under the causal mask) and LSE_i = ln(number of visible keys);
  * a permutation of the key/value rows, applied to K and V together, leaves a non-causal result unchanged
    (only the order of the sums differs).

The expected means are exact fp64 prefix sums of the values the GPU reads, so a wrong tile bound, a dropped
or doubled tile, a wrong causal offset or a chunk merged twice shows up at sizes the oracle cannot reach.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import workloads as W
from parity import assert_parity, errors, out_to_f64, storage_to_f64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


CASES = [
    # B, H, N_q, N_kv, d, dtype, causal, chunks
    (1, 2, 3000, 70001, 128, "bf16", True, 1),
    (1, 2, 3000, 70001, 128, "bf16", True, 8),
    (1, 2, 2048, 65600, 64, "bf16", False, 5),
    (2, 1, 5000, 33333, 64, "bf16", True, 3),
    (1, 2, 700, 20000, 64, "f32", True, 4),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])) + c[5] + ("c" if c[6] else "n")
                         + f"P{c[7]}")
def test_zero_queries_give_prefix_means(case):
    B, H, N_q, N_kv, d, dt, causal, chunks = case
    w = W.Workload("zeroq", B, H, N_q, N_kv, d, dt, causal, chunks, seed=8000 + N_kv)
    v_st = W.tensor_storage(w, W.V_T)
    k = to_device(W.tensor_storage(w, W.K_T))
    v = to_device(v_st)
    q = torch.zeros((B, H, N_q, d), dtype=k.dtype, device="cuda")
    o, lse = A.fwd_chunked(q, k, v, chunks, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    delta = N_kv - N_q
    # visible keys of row i: min(i + delta + 1, N_kv) under the mask, all N_kv without it
    count = np.minimum(np.arange(N_q) + delta + 1, N_kv) if causal else np.full(N_q, N_kv)
    assert count.min() >= 1
    for b in range(B):
        for h in range(H):
            vv = storage_to_f64(v_st[b, h])
            mean = np.cumsum(vv, axis=0)[count - 1] / count[:, None]
            err = errors(out_to_f64(o[b, h]), out_to_f64(lse[b, h]), mean, np.log(count))
            print(f"{case} b{b} h{h}: {err}", flush=True)
            assert_parity(err, dt, f"zero queries {case} b{b} h{h}")


@pytest.mark.parametrize("d,dt", [(128, "bf16"), (64, "bf16"), (64, "f32")])
def test_key_permutation_leaves_the_result(d, dt):
    w = W.Workload("perm", 1, 2, 1024, 50000, d, dt, False, 1, seed=8100 + d)
    q, k, v = (to_device(W.tensor_storage(w, t)) for t in (W.Q_T, W.K_T, W.V_T))
    perm = torch.from_numpy(np.random.default_rng(8101).permutation(w.N_kv)).cuda()
    o1, l1 = A.fwd(q, k, v, scale=w.scale)
    o2, l2 = A.fwd(q, k.index_select(2, perm).contiguous(), v.index_select(2, perm).contiguous(), scale=w.scale)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o2), out_to_f64(l2), out_to_f64(o1), out_to_f64(l1))
    print(f"d{d} {dt}: {err}", flush=True)
    assert_parity(err, dt, f"key permutation d{d} {dt}")


PLANT = [
    # B, H, N_q, N_kv, d, dtype, causal, chunks
    (1, 2, 4096, 131072, 128, "bf16", True, 1),
    (1, 2, 4096, 131072, 128, "bf16", True, 8),
    (1, 2, 4096, 100000, 64, "bf16", False, 3),
    (1, 2, 512, 20000, 64, "f32", True, 4),
]


@pytest.mark.parametrize("case", PLANT, ids=lambda c: "x".join(map(str, c[:5])) + c[5] + ("c" if c[6] else "n")
                         + f"P{c[7]}")
def test_one_planted_key_per_row_selects_its_value(case):
    """256 query rows per head each get one visible key j_i = a_i q_i whose score is SCORE (fp64; 120 at
    d = 128, 170 at d = 64).  The
    row's score against the other planted keys is about N(0, SCORE^2/d) and against the random keys O(1),
    and the test requires every one of them to stay more than 50 below SCORE: beyond the 2^64 (e^44.4) weight
    range that the kernels let a row's exponent reference lag behind its max, so the reference is the planted
    score and every other key weighs less than e^-50.  O_i is then V[j_i]: bit for bit in bf16, within 1e-5
    in fp32; LSE_i is the planted score.  Single pass and chunked, so the merges must also pick the right
    part."""
    B, H, N_q, N_kv, d, dt, causal, chunks = case
    SCORE, ROWS = (120.0 if d >= 128 else 170.0), 256   # other scores spread as SCORE/sqrt(d)
    w = W.Workload("plant", B, H, N_q, N_kv, d, dt, causal, chunks, seed=8200 + N_kv + d)
    q_st, k_st, v_st = (W.tensor_storage(w, t) for t in (W.Q_T, W.K_T, W.V_T))
    k_st = k_st.copy()
    rng = np.random.default_rng(8201)
    visible_to_all = N_kv - N_q + 1 if causal else N_kv   # keys 0 .. N_kv - N_q are visible to every row
    planted = {}
    for b in range(B):
        for h in range(H):
            rows = np.sort(rng.choice(N_q, size=ROWS, replace=False))
            j = rng.choice(visible_to_all, size=ROWS, replace=False)
            q = storage_to_f64(q_st[b, h][rows])
            kp = (SCORE / (w.scale * (q * q).sum(axis=1)))[:, None] * q
            k_st[b, h][j] = W.f32_to_bf16_bits(kp.astype(np.float32)) if dt == "bf16" else kp.astype(np.float32)
            s_all = w.scale * q @ storage_to_f64(k_st[b, h]).T     # every score of the planted rows
            s = s_all[np.arange(ROWS), j]
            s_all[np.arange(ROWS), j] = -np.inf
            margin = (s - s_all.max(axis=1)).min()
            assert np.abs(s - SCORE).max() < 1 and margin > 50, f"the planted keys do not dominate ({margin})"
            planted[(b, h)] = (rows, j, s)
    q, k, v = (to_device(x) for x in (q_st, k_st, v_st))
    o, lse = A.fwd_chunked(q, k, v, chunks, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    for b in range(B):
        for h in range(H):
            rows, j, s = planted[(b, h)]
            idx = torch.from_numpy(rows).cuda()
            want = v_st[b, h][j]
            lse_err = float(np.abs(out_to_f64(lse[b, h].index_select(0, idx)) - s).max())
            if dt == "bf16":
                got = o[b, h].index_select(0, idx).view(torch.int16).cpu().numpy().view(np.uint16)
                mismatch = int((got != want).any(axis=1).sum())
                print(f"{case} b{b} h{h}: rows differing from V[j_i]: {mismatch} of {ROWS}, lse {lse_err:.2e}",
                      flush=True)
                assert mismatch == 0
            else:
                err = float(np.abs(out_to_f64(o[b, h].index_select(0, idx)) - want.astype(np.float64)).max())
                print(f"{case} b{b} h{h}: max-abs {err:.2e}, lse {lse_err:.2e}", flush=True)
                assert err <= 1e-5
            assert lse_err <= 1e-4
