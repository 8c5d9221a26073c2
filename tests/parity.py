"""Shared helpers for the GPU parity tests: device upload of seeded inputs and the error metrics.

Tolerances (fixed for the path): fp32 inputs max-abs <= 1e-5; bf16 inputs with fp32 accumulation
max-abs <= 2e-2 and relative RMS <= 5e-3; lse <= 1e-4 absolute, and an lse of -inf must match exactly.
"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W

TOL = {"f32": {"max_abs": 1e-5}, "bf16": {"max_abs": 2e-2, "rel_rms": 5e-3}}
LSE_TOL = 1e-4


def to_device(storage: np.ndarray) -> torch.Tensor:
    """Storage array (float32, or uint16 bf16 patterns) -> device tensor of the same values."""
    if storage.dtype == np.uint16:
        return torch.from_numpy(storage.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(storage).cuda()


def storage_to_f64(storage: np.ndarray) -> np.ndarray:
    return W.bf16_bits_to_f64(storage) if storage.dtype == np.uint16 else storage.astype(np.float64)


def out_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def errors(o_gpu, lse_gpu, o_ref, lse_ref) -> dict:
    o_gpu, lse_gpu = np.asarray(o_gpu, np.float64), np.asarray(lse_gpu, np.float64)
    diff = o_gpu - o_ref
    ref_norm = np.linalg.norm(o_ref)
    inf_ref = np.isinf(lse_ref)
    lse_ok = np.array_equal(np.isinf(lse_gpu), inf_ref) and np.array_equal(lse_gpu[inf_ref], lse_ref[inf_ref])
    fin = ~inf_ref
    return {
        "max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
        "rel_rms": float(np.linalg.norm(diff) / ref_norm) if ref_norm > 0 else float(np.linalg.norm(diff)),
        "lse_abs": float(np.max(np.abs(lse_gpu[fin] - lse_ref[fin]))) if fin.any() else 0.0,
        "lse_inf_match": bool(lse_ok),
        "nan": bool(np.isnan(o_gpu).any() or np.isnan(lse_gpu).any()),
    }


def assert_parity(err: dict, dtype: str, what: str = ""):
    assert not err["nan"], f"{what}: NaN in output {err}"
    assert err["lse_inf_match"], f"{what}: -inf pattern of lse differs {err}"
    assert err["max_abs"] <= TOL[dtype]["max_abs"], f"{what}: max-abs {err}"
    if "rel_rms" in TOL[dtype]:
        assert err["rel_rms"] <= TOL[dtype]["rel_rms"], f"{what}: rel-RMS {err}"
    assert err["lse_abs"] <= LSE_TOL, f"{what}: lse {err}"
