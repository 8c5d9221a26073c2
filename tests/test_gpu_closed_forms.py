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
