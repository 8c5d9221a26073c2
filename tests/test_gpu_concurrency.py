"""Concurrent calls through the C ABI: several host threads, each with its own HIP stream, call the entry
points at the same time, and every result equals bit for bit the same call made alone on one stream.

The library keeps no per-call state.  What it shares between calls is per-device launch settings written
once, the timing log (off here), and the pool of synchronisation events of the host-streamed mode, which
the streamed case below exercises from several threads at once.  ctypes releases the interpreter lock for
the duration of each foreign call, so the threads' calls into the library do overlap.
"""
from __future__ import annotations

import threading

import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import workloads as W
from parity import to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


def qkv(name, B, H, N_q, N_kv, d, dt, causal, seed):
    w = W.Workload(name, B, H, N_q, N_kv, d, dt, causal, 1, seed=seed)
    return w, [to_device(W.tensor_storage(w, t)) for t in (W.Q_T, W.K_T, W.V_T)]


def build_calls():
    """(name, call) pairs; each call allocates its outputs on the calling thread's current stream."""
    calls = []
    w, (q, k, v) = qkv("conc_d128", 1, 4, 700, 900, 128, "bf16", True, 6000)
    calls.append(("fwd bf16 d128 causal", lambda: A.fwd(q, k, v, causal=True, scale=w.scale)))
    w2, (q2, k2, v2) = qkv("conc_d64", 2, 2, 333, 1000, 64, "bf16", False, 6001)
    calls.append(("fwd_chunked bf16 d64, 3 chunks", lambda: A.fwd_chunked(q2, k2, v2, 3, scale=w2.scale)))
    w3, (q3, k3, v3) = qkv("conc_f32", 1, 3, 200, 260, 48, "f32", True, 6002)
    calls.append(("fwd_chunked f32 d48 causal, 4 chunks",
                  lambda: A.fwd_chunked(q3, k3, v3, 4, causal=True, scale=w3.scale)))
    oa, la = A.fwd_ex(q, k, v, key_range=(0, 400), causal=True, causal_offset=200, out_dtype=torch.float32)
    ob, lb = A.fwd_ex(q, k, v, key_range=(400, 900), causal=True, causal_offset=-200, out_dtype=torch.float32)
    calls.append(("merge fp32 -> bf16", lambda: A.merge(oa, la, ob, lb, out_dtype=torch.bfloat16)))
    kp, vp = k.cpu().pin_memory(), v.cpu().pin_memory()
    calls.append(("fwd_streamed bf16 d128, 5 chunks",
                  lambda: A.fwd_streamed(q, kp, vp, 5, causal=True, scale=w.scale)))
    fw = W.FfnWorkload("conc_ffn", 300, 128, 512, 128, "gelu", seed=6003)
    x, w1, b1, w_2, b2 = (to_device(W.ffn_tensor(fw, t)) for t in (W.X_T, W.W1_T, W.B1_T, W.W2_T, W.B2_T))
    calls.append(("ffn_blockwise gelu", lambda: A.ffn_blockwise(x, w1, b1, w_2, b2, block=128)))
    torch.cuda.synchronize()
    return calls


def as_tuple(r):
    return r if isinstance(r, tuple) else (r,)


def test_threads_each_on_its_own_stream():
    calls = build_calls()
    alone = []
    for _, call in calls:
        alone.append(tuple(t.clone() for t in as_tuple(call())))
        torch.cuda.synchronize()

    reps = 3
    results: dict[tuple[int, int], tuple] = {}
    failures: list[str] = []
    start = threading.Barrier(len(calls), timeout=60)   # a thread that fails early breaks it for all

    def worker(i, call):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                start.wait()
                outs = [as_tuple(call()) for _ in range(reps)]
            s.synchronize()
            for r, out in enumerate(outs):
                results[(i, r)] = out
        except Exception as e:   # reported by the main thread
            failures.append(f"{calls[i][0]}: {e!r}")

    threads = [threading.Thread(target=worker, args=(i, c), daemon=True) for i, (_, c) in enumerate(calls)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not failures, failures
    for i, (name, _) in enumerate(calls):
        for r in range(reps):
            got = results[(i, r)]
            assert len(got) == len(alone[i])
            for a, b in zip(got, alone[i]):
                assert torch.equal(a, b), f"{name}, repetition {r}: differs from the call made alone"
    print(f"{len(calls)} threads x {reps} calls each, all bit-equal to the calls made alone", flush=True)
