"""The library's runtime switches on the GPU: launch timing (attn_timing_enable / attn_timing_read) counts
every launch and chunk copy of each kind and nothing while it is off; ATTN_DEBUG=1 (a synchronise and an
error check after every launch) gives results bit-equal to the asynchronous path.
"""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import workloads as W
from parity import to_device

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


def attn_inputs(seed=7000):
    w = W.Workload("rt_attn", 1, 2, 300, 600, 128, "bf16", False, 1, seed=seed)
    return w, [to_device(W.tensor_storage(w, t)) for t in (W.Q_T, W.K_T, W.V_T)]


def ffn_inputs(seed=7001):
    fw = W.FfnWorkload("rt_ffn", 300, 128, 256, 128, "gelu", seed=seed)
    return fw, [to_device(W.ffn_tensor(fw, t)) for t in (W.X_T, W.W1_T, W.B1_T, W.W2_T, W.B2_T)]


def test_launch_timing_counts_every_launch():
    w, (q, k, v) = attn_inputs()
    fw, (x, w1, b1, w2, b2) = ffn_inputs()
    oa, la = A.fwd_ex(q, k, v, key_range=(0, 250), out_dtype=torch.float32)
    ob, lb = A.fwd_ex(q, k, v, key_range=(250, 600), out_dtype=torch.float32)
    kp, vp = k.cpu().pin_memory(), v.cpu().pin_memory()
    torch.cuda.synchronize()
    A.timing_enable(True)
    try:
        A.timing_read()                                  # drop anything recorded before
        A.fwd_chunked(q, k, v, 3, scale=w.scale)         # 3 forward launches (every chunk is live)
        A.merge(oa, la, ob, lb)                          # 1 merge
        A.ffn_blockwise(x, w1, b1, w2, b2, block=128)    # 3 row blocks x 2 GEMMs
        A.fwd_streamed(q, kp, vp, 2, scale=w.scale)      # 2 chunk copies and 2 forward launches
        torch.cuda.synchronize()
        t = A.timing_read()
    finally:
        A.timing_enable(False)
    print(t, flush=True)
    assert {k_: c for k_, (c, _) in t.items()} == {"fwd": 5, "merge": 1, "copy": 2, "ffn": 6}
    assert all(ms > 0 for _, ms in t.values())
    A.fwd(q, k, v)                                       # timing off: nothing recorded
    torch.cuda.synchronize()
    assert all(c == 0 for c, _ in A.timing_read().values())


CHILD = r"""
import os, sys
sys.path.insert(0, os.environ["REPO"])
import numpy as np, torch
import test_gpu_runtime as T
import exact_blockwise_attention_fwd_amd as A
w, (q, k, v) = T.attn_inputs()
fw, (x, w1, b1, w2, b2) = T.ffn_inputs()
o, lse = A.fwd_chunked(q, k, v, 3, causal=True, scale=w.scale)
y = A.ffn_blockwise(x, w1, b1, w2, b2, block=128)
torch.cuda.synchronize()
out = os.environ["OUT"]
np.save(out + "/o.npy", o.view(torch.int16).cpu().numpy())
np.save(out + "/lse.npy", lse.cpu().numpy())
np.save(out + "/y.npy", y.view(torch.int16).cpu().numpy())
print("child done", flush=True)
"""


def test_debug_sync_gives_the_same_bits(tmp_path):
    """ATTN_DEBUG is read once per process, so the debug run is a child process on the same GPU."""
    w, (q, k, v) = attn_inputs()
    fw, (x, w1, b1, w2, b2) = ffn_inputs()
    o, lse = A.fwd_chunked(q, k, v, 3, causal=True, scale=w.scale)
    y = A.ffn_blockwise(x, w1, b1, w2, b2, block=128)
    torch.cuda.synchronize()
    env = dict(os.environ, ATTN_DEBUG="1", REPO=ROOT, OUT=str(tmp_path),
               PYTHONPATH=os.pathsep.join([os.path.join(ROOT, "tests"), ROOT, os.environ.get("PYTHONPATH", "")]))
    r = subprocess.run([sys.executable, "-c", CHILD], env=env, capture_output=True, text=True, timeout=150)
    print(r.stdout[-2000:], r.stderr[-2000:], flush=True)
    assert r.returncode == 0 and "child done" in r.stdout
    assert np.array_equal(np.load(tmp_path / "o.npy"), o.view(torch.int16).cpu().numpy())
    assert np.array_equal(np.load(tmp_path / "lse.npy"), lse.cpu().numpy())
    assert np.array_equal(np.load(tmp_path / "y.npy"), y.view(torch.int16).cpu().numpy())
