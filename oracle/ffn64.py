"""fp64 CPU oracle for the blockwise feed-forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this module; only the
tests, the smoke check and the bench's CPU-baseline leg do.  It shares no code with the HIP library.

Source: "Ring Attention with Blockwise Parallel Transformers" explainer, section 3 (blockwise computation):
the long sequence is cut into small contiguous blocks, and self-attention and the feedforward are applied
block by block.  The pages name the feedforward of a standard Transformer without defining it; the
readings taken here (each listed with its reason in the design notes):
  * the feedforward is the position-wise two-layer network  FFN(x) = act(x W1^T + b1) W2^T + b2  applied
    to every row x of the sequence, with W1 [d_ff, d] and W2 [d, d_ff] in the [out, in] layout;
  * act is GELU in its exact form x * Phi(x) (Phi the standard normal CDF), or ReLU, or none (the two
    linear layers alone, which the library also offers);
  * the blockwise form applies it to contiguous row blocks of `block` rows, the last one ragged; rows are
    independent, so every block size gives the same result.

All arithmetic is float64.  Inputs are the exact values the GPU reads (bf16 widened losslessly, fp32
biases).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def gelu(x) -> np.ndarray:
    """x * Phi(x) with Phi(x) = (1 + erf(x / sqrt(2))) / 2."""
    x = _as64(x)
    return x * 0.5 * (1.0 + erf(x / np.sqrt(2.0)))


def relu(x) -> np.ndarray:
    return np.maximum(_as64(x), 0.0)


def identity(x) -> np.ndarray:
    return _as64(x)


ACTS = {"gelu": gelu, "relu": relu, "none": identity}


def ffn_rows(x, w1, b1, w2, b2, act: str = "gelu") -> np.ndarray:
    """FFN of every row of x [n, d]: act(x W1^T + b1) W2^T + b2 -> [n, d].  b1 / b2 may be None (zero)."""
    x, w1, w2 = _as64(x), _as64(w1), _as64(w2)
    pre = x @ w1.T
    if b1 is not None:
        pre = pre + _as64(b1)[None, :]
    h = ACTS[act](pre)
    y = h @ w2.T
    if b2 is not None:
        y = y + _as64(b2)[None, :]
    return y


def block_bounds(n: int, block: int) -> list[int]:
    """Row-block starts 0, block, 2*block, ... and the end n: the last block holds the remainder."""
    return list(range(0, n, block)) + [n]


def ffn_blockwise(x, w1, b1, w2, b2, act: str = "gelu", block: int = 1) -> np.ndarray:
    """The blockwise form: the rows of x in contiguous blocks of `block`, each through ffn_rows."""
    x = _as64(x)
    bb = block_bounds(x.shape[0], block)
    out = np.empty((x.shape[0], np.shape(w2)[0]))
    for i in range(len(bb) - 1):
        out[bb[i]:bb[i + 1]] = ffn_rows(x[bb[i]:bb[i + 1]], w1, b1, w2, b2, act)
    return out
