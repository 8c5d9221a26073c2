"""GPU checks of the library's memory and fold contracts, through the C ABI.

  * Guard canaries: every output and the workspace are carved out of larger buffers whose surrounding bytes
    hold a fixed pattern; at ragged shapes (query and key counts that end inside a tile) every call leaves
    those bytes untouched and still matches the oracle.
  * No allocation: with every output and workspace supplied by the caller, no call changes the device's free
    memory or torch's allocation count, and the workspace size does not depend on the key count, so no
    score matrix of N_q x N_kv entries is ever stored ("FlashAttention by hand", paragraph on why the fused
    kernel helps: the score matrix never reaches memory).
  * Resume: a chunked fold stopped after some chunks, its running partial (O_acc, lse_acc) saved to host
    memory and restored into fresh device buffers, and then continued, equals the uninterrupted
    attn_fwd_chunked bit for bit.
  * Duplicate: folding one chunk twice is not the result; the merge is not idempotent (merging a partial
    with itself adds ln 2 to its lse), so the partials of the "ATTENTION2D" explainer (sections 2 and 3)
    must cover disjoint key sets, each exactly once.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import oracle
import workloads as W
from parity import assert_parity, errors, out_to_f64, storage_to_f64, to_device

pytestmark = pytest.mark.gpu

GUARD = 4096          # bytes of pattern before and after every guarded array (a multiple of 256)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


def make(w):
    st = [W.tensor_storage(w, t) for t in (W.Q_T, W.K_T, W.V_T)]
    return st, [to_device(s) for s in st]


class Guarded:
    """A device array of `shape` and `dtype` inside a byte buffer with GUARD pattern bytes on each side."""

    def __init__(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
        self.n = n
        self.buf = torch.full((GUARD + ((n + 255) // 256) * 256 + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(shape)

    def intact(self) -> bool:
        before = self.buf[:GUARD]
        after = self.buf[GUARD + self.n:]
        return bool((before == PATTERN).all().item()) and bool((after == PATTERN).all().item())


CANARY_CASES = [
    # B, H, N_q, N_kv, d, causal, dtype, chunks
    (1, 3, 333, 1001, 128, True, "bf16", 3),
    (2, 2, 517, 389, 128, False, "bf16", 4),
    (1, 2, 1000, 257, 64, True, "bf16", 2),
    (1, 3, 130, 70, 37, True, "f32", 3),
    (1, 2, 67, 300, 64, False, "f32", 5),
]


@pytest.mark.parametrize("case", CANARY_CASES, ids=lambda c: "x".join(map(str, c[:5])) + ("c" if c[5] else "n") + c[6])
def test_guard_canaries(case):
    B, H, N_q, N_kv, d, causal, dt, P = case
    w = W.Workload("canary", B, H, N_q, N_kv, d, dt, causal, 1, seed=5000 + N_q + d)
    st, (q, k, v) = make(w)
    o_ref, l_ref = oracle.attention(*(storage_to_f64(s) for s in st), w.scale, w.causal, w.offset)
    tdt = q.dtype
    # single pass
    o = Guarded(q.shape, tdt)
    lse = Guarded((B, H, N_q), torch.float32)
    A.fwd(q, k, v, causal=causal, scale=w.scale, out=o.t, lse=lse.t)
    torch.cuda.synchronize()
    assert o.intact() and lse.intact(), "attn_fwd wrote outside O or LSE"
    assert_parity(errors(out_to_f64(o.t), out_to_f64(lse.t), o_ref, l_ref), dt, "guarded fwd")
    # chunked, with a guarded workspace
    o2 = Guarded(q.shape, tdt)
    lse2 = Guarded((B, H, N_q), torch.float32)
    ws = Guarded((A.workspace_bytes(B, H, N_q, d, P),), torch.uint8)
    A.fwd_chunked(q, k, v, P, causal=causal, scale=w.scale, out=o2.t, lse=lse2.t, workspace=ws.t)
    torch.cuda.synchronize()
    assert o2.intact() and lse2.intact() and ws.intact(), "attn_fwd_chunked wrote outside O, LSE or its workspace"
    assert_parity(errors(out_to_f64(o2.t), out_to_f64(lse2.t), o_ref, l_ref), dt, "guarded chunked")
    # fold of the second half of the keys into a partial over the first half (fp32 partial, output in dtype)
    half = N_kv // 2
    off = N_kv - N_q
    acc_o = Guarded(q.shape, torch.float32)
    acc_l = Guarded((B, H, N_q), torch.float32)
    A.fwd_ex(q, k, v, causal, w.scale, causal_offset=off, key_range=(0, half), out_dtype=torch.float32,
             out=acc_o.t, lse=acc_l.t)
    o3 = Guarded(q.shape, tdt)
    lse3 = Guarded((B, H, N_q), torch.float32)
    A.fwd_acc(q, k, v, acc_o.t, acc_l.t, causal, w.scale, causal_offset=off - half, key_range=(half, N_kv),
              out=o3.t, lse=lse3.t)
    torch.cuda.synchronize()
    assert acc_o.intact() and acc_l.intact() and o3.intact() and lse3.intact(), "attn_fwd_ex/acc wrote outside"
    assert_parity(errors(out_to_f64(o3.t), out_to_f64(lse3.t), o_ref, l_ref), dt, "guarded fold")
    # merge of two guarded partials into a guarded result
    pb_o = Guarded(q.shape, torch.float32)
    pb_l = Guarded((B, H, N_q), torch.float32)
    A.fwd_ex(q, k, v, causal, w.scale, causal_offset=off - half, key_range=(half, N_kv), out_dtype=torch.float32,
             out=pb_o.t, lse=pb_l.t)
    mo = Guarded(q.shape, tdt)
    ml = Guarded((B, H, N_q), torch.float32)
    A.merge(acc_o.t, acc_l.t, pb_o.t, pb_l.t, out=mo.t, lse=ml.t)
    torch.cuda.synchronize()
    assert pb_o.intact() and pb_l.intact() and mo.intact() and ml.intact(), "attn_merge wrote outside"
    assert_parity(errors(out_to_f64(mo.t), out_to_f64(ml.t), o_ref, l_ref), dt, "guarded merge")


def test_no_device_allocation_and_no_score_matrix():
    """Calls with caller-supplied outputs and workspace change neither the device's free memory nor torch's
    allocator state; the chunked workspace is O(N_q d), whatever the key count."""
    w = W.Workload("noalloc", 1, 4, 700, 9000, 128, "bf16", True, 1, seed=5100)
    st, (q, k, v) = make(w)
    P = 5
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 700), dtype=torch.float32, device="cuda")
    ws = torch.empty(A.workspace_bytes(1, 4, 700, 128, P), dtype=torch.uint8, device="cuda")
    acc_o = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    acc_l = torch.empty_like(lse)
    m_o = torch.empty_like(acc_o)
    m_l = torch.empty_like(lse)

    def calls():
        A.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
        A.fwd_chunked(q, k, v, P, causal=True, scale=w.scale, out=o, lse=lse, workspace=ws)
        A.fwd_ex(q, k, v, True, w.scale, causal_offset=9000 - 700, key_range=(0, 4000), out_dtype=torch.float32,
                 out=acc_o, lse=acc_l)
        A.fwd_acc(q, k, v, acc_o, acc_l, True, w.scale, causal_offset=5000 - 700, key_range=(4000, 9000),
                  out_dtype=torch.float32, out=acc_o, lse=acc_l)
        A.merge(acc_o, acc_l, acc_o, acc_l, out=m_o, lse=m_l)

    calls()   # first launches load the kernels' code
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    for _ in range(3):
        calls()
    torch.cuda.synchronize()
    free1, total = torch.cuda.mem_get_info()
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes during the calls"
    assert torch.cuda.memory_allocated() == alloc0
    # the workspace does not grow with the key count; a stored fp32 score matrix of the Ulysses head share
    # (8 heads of 262144 x 262144) would need more than the whole device
    sizes = {A.workspace_bytes(1, 8, 262144, 128, P) for P in (2, 8, 64)}
    assert sizes == {A.workspace_bytes(1, 8, 262144, 128, 2)}
    assert 8 * 262144 * 262144 * 4 > total
    assert A.workspace_bytes(1, 8, 262144, 128, 8) < 8 * 262144 * 129 * 4 + 4096


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_fold_resumed_from_saved_partial(dt, d):
    """Chunks 0..2 of 7 folded, the running partial copied to host memory and the device buffers freed; the
    fold resumed from the restored copy over chunks 3..6 equals attn_fwd_chunked bit for bit."""
    w = W.Workload("resume", 1, 3, 600, 2100, d, dt, True, 1, seed=5200 + d)
    st, (q, k, v) = make(w)
    P = 7
    o_ref_dev, l_ref_dev = A.fwd_chunked(q, k, v, P, causal=True, scale=w.scale)
    cuts = oracle.chunk_bounds(w.N_kv, P)
    off = w.N_kv - w.N_q
    acc_o, acc_l = A.fwd_ex(q, k, v, True, w.scale, causal_offset=off - cuts[0], key_range=(cuts[0], cuts[1]),
                            out_dtype=torch.float32)
    for p in (1, 2):
        A.fwd_acc(q, k, v, acc_o, acc_l, True, w.scale, causal_offset=off - cuts[p], key_range=(cuts[p], cuts[p + 1]),
                  out_dtype=torch.float32, out=acc_o, lse=acc_l)
    torch.cuda.synchronize()
    saved_o, saved_l = acc_o.cpu(), acc_l.cpu()
    del acc_o, acc_l
    torch.cuda.synchronize()
    acc_o, acc_l = saved_o.cuda(), saved_l.cuda()
    for p in range(3, P):
        last = p == P - 1
        out_o, out_l = A.fwd_acc(q, k, v, acc_o, acc_l, True, w.scale, causal_offset=off - cuts[p],
                                 key_range=(cuts[p], cuts[p + 1]), out_dtype=q.dtype if last else torch.float32,
                                 out=None if last else acc_o, lse=None if last else acc_l)
    torch.cuda.synchronize()
    assert torch.equal(out_o, o_ref_dev) and torch.equal(out_l, l_ref_dev), "resumed fold differs"
    o_ref, l_ref = oracle.attention(*(storage_to_f64(s) for s in st), w.scale, True, off)
    assert_parity(errors(out_to_f64(out_o), out_to_f64(out_l), o_ref, l_ref), dt, "resumed fold")


def test_duplicated_chunk_breaks_the_fold():
    """The same 7-chunk fold with chunk 3 folded twice: rows that see chunk 3's keys move far outside the
    tolerance (their lse by up to ln 2), while the fold with every chunk once is within it."""
    w = W.Workload("dup", 1, 2, 500, 2100, 128, "bf16", False, 1, seed=5300)
    st, (q, k, v) = make(w)
    P = 7
    cuts = oracle.chunk_bounds(w.N_kv, P)
    o_ref, l_ref = oracle.attention(*(storage_to_f64(s) for s in st), w.scale, False)

    def fold(order):
        acc_o, acc_l = A.fwd_ex(q, k, v, False, w.scale, key_range=(cuts[order[0]], cuts[order[0] + 1]),
                                out_dtype=torch.float32)
        for p in order[1:]:
            A.fwd_acc(q, k, v, acc_o, acc_l, False, w.scale, key_range=(cuts[p], cuts[p + 1]),
                      out_dtype=torch.float32, out=acc_o, lse=acc_l)
        torch.cuda.synchronize()
        return errors(out_to_f64(acc_o), out_to_f64(acc_l), o_ref, l_ref)

    good = fold(list(range(P)))
    assert_parity(good, "bf16", "each chunk once")
    bad = fold([0, 1, 2, 3, 3, 4, 5, 6])
    print("each chunk once", good, "chunk 3 twice", bad, flush=True)
    assert bad["lse_abs"] > 0.05, bad   # the rows' lse gain up to ln 2 where chunk 3 carries their weight
    with pytest.raises(AssertionError):
        assert_parity(bad, "bf16", "chunk 3 folded twice")
    # the oracle's own merge is not idempotent either: (O, L) merged with itself gives (O, L + ln 2)
    o1, l1 = oracle.merge(o_ref, l_ref, o_ref, l_ref)
    assert np.allclose(o1, o_ref) and np.allclose(l1, l_ref + np.log(2.0))
