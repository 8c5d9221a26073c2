"""The seeded input module: bf16 rounding, regeneration per head, workload sizes and FLOP counts."""
import numpy as np
import pytest
import torch

import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 7,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.0078125, 1.01171875, 3.4e38, -1e-40],
                                 dtype=np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = W.bf16_bits_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy())


def test_heads_regenerate_independently():
    w = W.WORKLOADS["causal_prefill_4k"]
    small = W.Workload("t", 2, 3, 40, 56, 16, "bf16", True, 1, seed=9)
    full = W.tensor_storage(small, W.K_T)
    for b in range(2):
        for h in range(3):
            assert np.array_equal(full[b, h], W.head_storage(small, W.K_T, b, h))
    assert not np.array_equal(full[0, 0], full[0, 1])
    assert w.dtype == "bf16" and w.scale == pytest.approx(128 ** -0.5)


def test_peaky_q_has_std_four():
    w = W.WORKLOADS["peaky_16k"]
    q = W.head_f64(w, W.Q_T, 0, 0)
    k = W.head_f64(w, W.K_T, 0, 0)
    assert abs(q.std() - 4.0) < 0.02 and abs(k.std() - 1.0) < 0.01


def test_algorithmic_flops():
    # 4*d per visible pair; a square causal block counts N^2/2; the ring share's earlier chunks are full
    expect = {"tiny_fp32": 2.684e8, "causal_prefill_4k": 2.749e11, "peaky_16k": 1.0995e12,
              "ring_share_128k": 3.2985e13, "ulysses_share_256k": 1.4074e14}
    for name, f in expect.items():
        assert W.WORKLOADS[name].flops() == pytest.approx(f, rel=1e-3), name


def test_sample_rows_seeded_sorted_distinct():
    w = W.WORKLOADS["ulysses_share_256k"]
    r = W.sample_rows(w, 0, 3)
    assert len(r) == 64 and np.all(np.diff(r) > 0) and r[-1] < w.N_q
    assert np.array_equal(r, W.sample_rows(w, 0, 3))
    assert not np.array_equal(r, W.sample_rows(w, 0, 4))
