"""Seeded synthetic inputs for exact attention, shared by the tests, the bench and the oracle checks.

This module only draws numbers and rounds them to the storage type the GPU reads; it holds none of the
attention arithmetic, so the GPU path and the CPU oracle can both consume it without sharing any of the
method's code.

Recipe (one recipe for every workload):
  * each (tensor, b, h) slice has its own stream: numpy ``Generator(PCG64(SeedSequence(seed,
    spawn_key=(tensor, b, h))))`` with tensor 0 = Q, 1 = K, 2 = V, so any single head can be regenerated
    on the host without drawing the others;
  * values are ``standard_normal(float32) * std`` (std 1, except Q of the peaky workload, std 4);
  * for bf16 workloads the fp32 draws are rounded to bf16 with round-to-nearest-even; the oracle reads
    back exactly those bf16 values widened to fp64.

The workloads are the five shapes the attention kernels are measured and checked on (the pages describe
long-context exact attention on language data; no dataset is needed because the method's result does not
depend on where Q, K and V come from, only on their values):

  tiny_fp32          B1 H4  N 512            d64  fp32 non-causal, plus a 4-chunk KV merge
  causal_prefill_4k  B4 H16 N 4096           d128 bf16 causal
  peaky_16k          B2 H8  N 16384          d64  bf16 non-causal, Q std 4 (large logits)
  ring_share_128k    B1 H32 N_q 16384, N_kv 131072 in 8 chunks, d128 bf16, bottom-right causal
                     (the last chunk is the diagonal one, the earlier ones are fully visible)
  ulysses_share_256k B1 H8  N 262144         d128 bf16 causal, oracle on 64 seeded rows per head

Blockwise feed-forward inputs (``FfnWorkload``) follow the same scheme with one stream per tensor
(SeedSequence(seed, spawn_key=(20 + tensor,)), tensor 0 = X, 1 = W1, 2 = b1, 3 = W2, 4 = b2): X ~ N(0, 1)
and the weights ~ N(0, 1/fan_in) rounded to bf16, the biases 0.1 * N(0, 1) kept fp32.  The measured
shape is the feed-forward of the ring-share model: the 16384 local rows of d_model = 32 heads x 128 = 4096,
d_ff = 4 x d_model, GELU, in blocks of 4096 rows.
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

Q_T, K_T, V_T = 0, 1, 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N_q: int
    N_kv: int
    d: int
    dtype: str          # "f32" or "bf16": the storage type of Q, K, V and O
    causal: bool
    chunks: int         # P: number of KV chunks folded through the merge (1 = single pass)
    seed: int
    q_std: float = 1.0
    sample_rows: int = 0  # >0: the oracle is checked on this many seeded query rows per head
    row_seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def offset(self) -> int:
        # bottom-right causal alignment: key j is visible to query i when j <= i + (N_kv - N_q)
        return self.N_kv - self.N_q

    def visible_pairs(self) -> float:
        """Number of visible (query, key) pairs per (b, h), with a square causal block counted as N^2/2."""
        if not self.causal:
            return float(self.N_q) * self.N_kv
        full = self.N_q * max(self.N_kv - self.N_q, 0)
        return float(full) + 0.5 * float(min(self.N_q, self.N_kv)) ** 2

    def flops(self) -> float:
        """Algorithmic FLOPs: 4*d per visible pair (2d for Q.K, 2d for P.V)."""
        return 4.0 * self.d * self.B * self.H * self.visible_pairs()


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", 1, 4, 512, 512, 64, "f32", False, 4, seed=1),
        Workload("causal_prefill_4k", 4, 16, 4096, 4096, 128, "bf16", True, 1, seed=2),
        Workload("peaky_16k", 2, 8, 16384, 16384, 64, "bf16", False, 1, seed=3, q_std=4.0),
        Workload("ring_share_128k", 1, 32, 16384, 131072, 128, "bf16", True, 8, seed=4),
        Workload("ulysses_share_256k", 1, 8, 262144, 262144, 128, "bf16", True, 1, seed=5,
                 sample_rows=64, row_seed=105),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) and return the 16-bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float64 exactly."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def _stream(seed: int, tensor: int, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor, b, h))))


def head_f32(seed: int, tensor: int, b: int, h: int, n: int, d: int, std: float = 1.0) -> np.ndarray:
    """The fp32 draws of one (tensor, b, h) slice, shape [n, d]."""
    x = _stream(seed, tensor, b, h).standard_normal((n, d), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def head_storage(w: Workload, tensor: int, b: int, h: int) -> np.ndarray:
    """One (tensor, b, h) slice in the GPU's storage type: float32, or uint16 bf16 bit patterns."""
    n = w.N_q if tensor == Q_T else w.N_kv
    std = w.q_std if tensor == Q_T else 1.0
    x = head_f32(w.seed, tensor, b, h, n, w.d, std)
    return x if w.dtype == "f32" else f32_to_bf16_bits(x)


def head_f64(w: Workload, tensor: int, b: int, h: int) -> np.ndarray:
    """One (tensor, b, h) slice as the exact fp64 values the GPU reads."""
    s = head_storage(w, tensor, b, h)
    return s.astype(np.float64) if w.dtype == "f32" else bf16_bits_to_f64(s)


def tensor_storage(w: Workload, tensor: int, threads: int | None = None) -> np.ndarray:
    """A whole [B, H, N, d] tensor in storage type, drawn head by head (threads release the GIL)."""
    n = w.N_q if tensor == Q_T else w.N_kv
    out = np.empty((w.B, w.H, n, w.d), dtype=np.float32 if w.dtype == "f32" else np.uint16)
    jobs = [(b, h) for b in range(w.B) for h in range(w.H)]

    def fill(bh):
        b, h = bh
        out[b, h] = head_storage(w, tensor, b, h)

    threads = threads or min(16, len(os.sched_getaffinity(0)))
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(fill, jobs))
    return out


def sample_rows(w: Workload, b: int, h: int) -> np.ndarray:
    """Seeded query-row subset for one head: distinct rows drawn uniformly from [0, N_q), sorted."""
    n = w.sample_rows if w.sample_rows else w.N_q
    if n >= w.N_q:
        return np.arange(w.N_q)
    g = _stream(w.row_seed, 3, b, h)
    return np.sort(g.choice(w.N_q, size=n, replace=False))


# ------------------------------------------------------------------------------ blockwise feed-forward
X_T, W1_T, B1_T, W2_T, B2_T = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class FfnWorkload:
    name: str
    M: int              # rows of the sequence
    d_model: int
    d_ff: int
    block: int          # rows per block
    act: str            # "gelu", "relu" or "none"
    seed: int
    bias: bool = True
    sample_rows: int = 0  # >0: the oracle is checked on this many seeded rows

    def flops(self) -> float:
        """Algorithmic FLOPs: two products of 2 * M * d_model * d_ff each."""
        return 4.0 * self.M * self.d_model * self.d_ff


FFN_WORKLOADS = {
    w.name: w
    for w in [
        FfnWorkload("ffn_ring_share", 16384, 4096, 16384, 4096, "gelu", seed=6, sample_rows=64),
    ]
}


def ffn_tensor(w: FfnWorkload, tensor: int) -> np.ndarray:
    """One tensor of a feed-forward workload: X, W1, W2 as uint16 bf16 patterns, b1, b2 as float32."""
    shape = {X_T: (w.M, w.d_model), W1_T: (w.d_ff, w.d_model), B1_T: (w.d_ff,), W2_T: (w.d_model, w.d_ff),
             B2_T: (w.d_model,)}[tensor]
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(20 + tensor,))))
    x = g.standard_normal(shape, dtype=np.float32)
    if tensor in (B1_T, B2_T):
        return x * np.float32(0.1)
    if tensor == W1_T:
        x *= np.float32(1.0 / math.sqrt(w.d_model))
    elif tensor == W2_T:
        x *= np.float32(1.0 / math.sqrt(w.d_ff))
    return f32_to_bf16_bits(x)


def ffn_sample_rows(w: FfnWorkload) -> np.ndarray:
    """Seeded row subset: distinct rows drawn uniformly from [0, M), sorted (all rows if not sampled)."""
    if not w.sample_rows or w.sample_rows >= w.M:
        return np.arange(w.M)
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(w.seed, spawn_key=(30,))))
    return np.sort(g.choice(w.M, size=w.sample_rows, replace=False))
