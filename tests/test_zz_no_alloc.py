"""attn_fwd_chunked_noalloc on the GPU, through the C ABI: the running partial in the library's fixed per-device
scratch gives attn_fwd_chunked's result bit for bit (and the oracle's within tolerance) on two calls in a row,
the second one smaller, and the calls change neither the device's free memory nor torch's allocator state."""
from __future__ import annotations

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


CASES = [
    # B, H, N_q, N_kv, d, causal, dtype, chunks: the first fills most of the 64 MiB scratch, the second is smaller
    (1, 8, 16000, 20000, 128, True, "bf16", 5),
    (1, 2, 700, 900, 64, False, "bf16", 3),
    (1, 3, 130, 270, 37, True, "f32", 4),
]


def test_noalloc_equals_chunked_two_calls_in_a_row():
    runs = []
    for i, (B, H, N_q, N_kv, d, causal, dt, P) in enumerate(CASES):
        w = W.Workload(f"noalloc{i}", B, H, N_q, N_kv, d, dt, causal, 1, seed=5400 + i)
        assert A.workspace_bytes(B, H, N_q, d, P) <= A.NOALLOC_SCRATCH_BYTES
        st = [W.tensor_storage(w, t) for t in (W.Q_T, W.K_T, W.V_T)]
        q, k, v = (to_device(s) for s in st)
        ref_o, ref_l = A.fwd_chunked(q, k, v, P, causal=causal, scale=w.scale)
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, N_q), float("nan"), device="cuda")
        runs.append((w, st, q, k, v, P, ref_o, ref_l, o, lse))
    torch.cuda.synchronize()
    # the first call on this device looks the scratch up (and loads the code that holds it); after it, the
    # calls allocate nothing
    w, st, q, k, v, P, ref_o, ref_l, o, lse = runs[0]
    A.fwd_chunked_noalloc(q, k, v, P, causal=w.causal, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for w, st, q, k, v, P, ref_o, ref_l, o, lse in runs:   # big, then smaller, then smallest, back to back
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        A.fwd_chunked_noalloc(q, k, v, P, causal=w.causal, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0, "device free memory changed during the calls"
    assert torch.cuda.memory_allocated() == alloc0
    for w, st, q, k, v, P, ref_o, ref_l, o, lse in runs:
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"{w.name}: differs from attn_fwd_chunked"
        if w.B * w.H * w.N_q * w.N_kv <= 5e7:   # the whole result
            o_ref, l_ref = oracle.attention(*(storage_to_f64(s) for s in st), w.scale, w.causal, w.offset)
            err = errors(out_to_f64(o), out_to_f64(lse), o_ref, l_ref)
        else:                                     # 64 seeded rows of every head, row by row
            rng = np.random.default_rng(w.seed)
            got_o, got_l, want_o, want_l = [], [], [], []
            for b in range(w.B):
                for h in range(w.H):
                    rows = np.unique(np.concatenate([rng.choice(w.N_q, 64, replace=False), [0, w.N_q - 1]]))
                    o_r, l_r = oracle.naive_head(storage_to_f64(st[0][b, h][rows]), storage_to_f64(st[1][b, h]),
                                                 storage_to_f64(st[2][b, h]), w.scale, w.causal, w.offset, rows)
                    idx = torch.from_numpy(rows).cuda()
                    got_o.append(out_to_f64(o[b, h].index_select(0, idx)))
                    got_l.append(out_to_f64(lse[b, h].index_select(0, idx)))
                    want_o.append(o_r)
                    want_l.append(l_r)
            err = errors(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(want_o), np.concatenate(want_l))
        print(w.name, P, err, flush=True)
        assert_parity(err, w.dtype, f"{w.name} noalloc")


def test_noalloc_rejects_a_partial_larger_than_the_scratch():
    w = W.Workload("noalloc_big", 1, 1, 130056, 64, 128, "bf16", False, 1, seed=5450)
    q = torch.zeros((1, 1, 130056, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((1, 1, 64, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(A.AttnError, match="WORKSPACE_TOO_SMALL"):
        A.fwd_chunked_noalloc(q, k, k, 2, scale=w.scale)
    # one chunk needs no partial at all
    o, lse = A.fwd_chunked_noalloc(q, k, k, 1, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o, torch.zeros_like(o)) and torch.allclose(lse, torch.full_like(lse, 4.1588830833596715))
