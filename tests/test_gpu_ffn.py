"""GPU parity of the blockwise feed-forward (attn_ffn_blockwise, through the C ABI) against the fp64 oracle.

Small shapes are compared in full: ragged row counts against the 256-row tiles and the block size, column
counts that end in a partial 256-column tile, reduction lengths of one or several 64-deep k-tiles, each
activation, with and without biases.  The measured shape (the ring-share model's feed-forward) is
compared on seeded rows that the oracle evaluates on their own.  Rows are independent, so the block size
must not change a single bit of the result.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import oracle.ffn64 as F
import workloads as W
from parity import assert_parity, errors, out_to_f64, storage_to_f64, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


def make(w: W.FfnWorkload):
    st = [W.ffn_tensor(w, t) for t in (W.X_T, W.W1_T, W.B1_T, W.W2_T, W.B2_T)]
    if not w.bias:
        st[2] = st[4] = None
    dev = [None if s is None else to_device(s) for s in st]
    return st, dev


def ffn_errors(y_dev, y_ref):
    """errors() with the output in place of O and no LSE."""
    y = out_to_f64(y_dev).reshape(y_ref.shape)
    return errors(y, np.zeros(y.shape[0]), y_ref, np.zeros(y.shape[0]))


SMALL = [
    # M, d_model, d_ff, block, act, bias
    (100, 64, 256, 64, "gelu", True),
    (300, 128, 512, 128, "relu", True),
    (1, 64, 64, 1, "gelu", True),
    (257, 192, 320, 100, "gelu", False),
    (513, 256, 1024, 512, "gelu", True),
    (700, 320, 448, 700, "none", True),
    (64, 512, 2048, 32, "relu", False),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "x".join(map(str, c[:4])) + f"-{c[4]}" + ("-b" if c[5] else ""))
def test_ffn_small_vs_oracle(case):
    M, d, d_ff, block, act, bias = case
    w = W.FfnWorkload("ffn_small", M, d, d_ff, block, act, seed=5000 + M + d_ff, bias=bias)
    st, (x, w1, b1, w2, b2) = make(w)
    y = A.ffn_blockwise(x, w1, b1, w2, b2, block=block, act=act)
    y_one = A.ffn_blockwise(x, w1, b1, w2, b2, block=M, act=act)
    torch.cuda.synchronize()
    ref = F.ffn_rows(storage_to_f64(st[0]), storage_to_f64(st[1]), st[2], storage_to_f64(st[3]), st[4], act)
    err = ffn_errors(y, ref)
    print(w, err, flush=True)
    assert_parity(err, "bf16", f"ffn {case}")
    assert torch.equal(y, y_one), "the block size changed the result"


def test_ffn_output_buffer_and_workspace_reuse():
    """A caller-supplied output and workspace, two calls of different sizes in a row, and NaN-poisoned output."""
    outs = []
    for M in (600, 250):
        w = W.FfnWorkload("ffn_reuse", M, 128, 512, 200, "gelu", seed=5100)
        st, (x, w1, b1, w2, b2) = make(w)
        ws = torch.empty(A.ffn_workspace_bytes(600, 512, 200), dtype=torch.uint8, device="cuda")
        y = torch.full((M, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        r = A.ffn_blockwise(x, w1, b1, w2, b2, block=200, out=y, workspace=ws)
        torch.cuda.synchronize()
        assert r.data_ptr() == y.data_ptr()
        ref = F.ffn_rows(storage_to_f64(st[0]), storage_to_f64(st[1]), st[2], storage_to_f64(st[3]), st[4], "gelu")
        err = ffn_errors(y, ref)
        assert not err["nan"]
        assert_parity(err, "bf16", f"ffn reuse M={M}")
        outs.append(y)


def test_ffn_ring_share_sampled():
    """The measured shape (16384 rows, d_model 4096, d_ff 16384, blocks of 4096, GELU) in the launch
    configuration the bench times: 64 seeded rows against the oracle."""
    w = W.FFN_WORKLOADS["ffn_ring_share"]
    st, (x, w1, b1, w2, b2) = make(w)
    y = A.ffn_blockwise(x, w1, b1, w2, b2, block=w.block, act=w.act)
    torch.cuda.synchronize()
    rows = W.ffn_sample_rows(w)
    ref = F.ffn_rows(storage_to_f64(st[0][rows]), storage_to_f64(st[1]), st[2], storage_to_f64(st[3]), st[4], w.act)
    err = ffn_errors(y.index_select(0, torch.from_numpy(rows).cuda()), ref)
    print(w, err, flush=True)
    assert_parity(err, "bf16", "ffn ring share sampled rows")


def test_ffn_graph_capture_and_replay():
    """attn_ffn_blockwise allocates nothing and never synchronises: captured into a HIP graph (three row
    blocks, six GEMM launches) it replays bit for bit equal to the eager call, with eager work between."""
    w = W.FfnWorkload("ffn_graph", 600, 128, 512, 256, "gelu", seed=5200)
    st, (x, w1, b1, w2, b2) = make(w)
    ws = torch.empty(A.ffn_workspace_bytes(w.M, w.d_ff, w.block), dtype=torch.uint8, device="cuda")
    y = torch.empty((w.M, w.d_model), dtype=torch.bfloat16, device="cuda")
    A.ffn_blockwise(x, w1, b1, w2, b2, block=w.block, out=y, workspace=ws)   # eager; sets the LDS attribute
    torch.cuda.synchronize()
    eager = y.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            A.ffn_blockwise(x, w1, b1, w2, b2, block=w.block, out=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        y.fill_(float("nan"))
        ws.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager), f"replay {rep} differs from the eager result"


def test_ffn_binding_checks():
    """The binding refuses tensors whose dtype, shape or device differ from what the call reads or writes."""
    w = W.FfnWorkload("ffn_bind", 64, 128, 256, 64, "gelu", seed=5300)
    _, (x, w1, b1, w2, b2) = make(w)
    bad = [
        lambda: A.ffn_blockwise(x.float(), w1, b1, w2, b2),
        lambda: A.ffn_blockwise(x, w1[:128].contiguous(), b1, w2, b2),
        lambda: A.ffn_blockwise(x, w1, b1[:100].contiguous(), w2, b2),
        lambda: A.ffn_blockwise(x, w1, b1.to(torch.bfloat16), w2, b2),
        lambda: A.ffn_blockwise(x, w1, b1, w2.t().contiguous(), b2),
        lambda: A.ffn_blockwise(x, w1, b1, w2, b2, act="swish"),
        lambda: A.ffn_blockwise(x, w1, b1, w2, b2, out=torch.empty((64, 128), device="cuda")),
        lambda: A.ffn_blockwise(x, w1, b1, w2, b2, workspace=torch.empty(1 << 20, dtype=torch.uint8)),
        lambda: A.ffn_blockwise(x, w1, b1, w2, b2, block=64, workspace=torch.empty(16, dtype=torch.uint8,
                                                                                  device="cuda")),
    ]
    for i, call in enumerate(bad):
        with pytest.raises((ValueError, TypeError, A.AttnError)):
            call()
            pytest.fail(f"case {i} accepted")


@pytest.mark.parametrize("act,bias", [("relu", False), ("none", True)])
def test_ffn_selection_weights_full_size_bit_exact(act, bias):
    """Every output of the measured shape (16384 x 4096, d_ff 16384, blocks of 4096) checked bit for bit.  With
    W1[n] the unit row e_sigma(n) and W2[j] the unit row e_tau(j) (sigma and tau seeded maps), each dot product
    has exactly one non-zero term, so the exact result is known elementwise:
        H[m][n] = act(X[m][sigma(n)] + b1[n])        rounded once to bf16 (the sum in fp32),
        Y[m][j] = H[m][tau(j)] + b2[j]               rounded once to bf16 (the sum in fp32).
    A misplaced tile, a skipped or repeated k-tile, a transposed operand or a wrong row block changes bits."""
    M, d, d_ff, block = 16384, 4096, 16384, 4096
    rng = np.random.default_rng(5400)
    sigma = rng.integers(0, d, size=d_ff)
    tau = rng.choice(d_ff, size=d, replace=False)
    w = W.FfnWorkload("ffn_select", M, d, d_ff, block, act, seed=5401, bias=bias)
    x_st = W.ffn_tensor(w, W.X_T)
    one = W.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    w1 = np.zeros((d_ff, d), np.uint16)
    w1[np.arange(d_ff), sigma] = one
    w2 = np.zeros((d, d_ff), np.uint16)
    w2[np.arange(d), tau] = one
    b1 = W.ffn_tensor(w, W.B1_T) if bias else None
    b2 = W.ffn_tensor(w, W.B2_T) if bias else None
    x32 = W.bf16_bits_to_f64(x_st).astype(np.float32)
    pre = x32[:, sigma[tau]] + (b1[tau] if bias else np.float32(0))      # fp32 sums, only the used columns
    h = W.bf16_bits_to_f64(W.f32_to_bf16_bits(np.maximum(pre, 0) if act == "relu" else pre)).astype(np.float32)
    want = W.f32_to_bf16_bits(h + (b2 if bias else np.float32(0)))
    dev = [to_device(a) if a is not None else None for a in (x_st, w1, b1, w2, b2)]
    y = A.ffn_blockwise(*dev, block=block, act=act)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    bad = int((got != want).sum())
    print(f"act {act}, bias {bias}: {bad} of {got.size} outputs differ", flush=True)
    assert bad == 0
