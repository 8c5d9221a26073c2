"""fp64 CPU oracle for exact attention, the (O, lse) merge and the chunked fold.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or execute this module; only the
tests, the smoke check and the bench's CPU-baseline leg do.  It shares no code with the HIP library.

Sources (the pages this follows):
  [FA]    "FlashAttention by hand" (IT-news explainer): the three standard steps (similarity logits, a row
          softmax whose rows sum to one, product with V); the online-softmax paragraph (running max and
          running denominator while streaming key blocks, fused with the product by V); the per-tile flow
          paragraph (tile-local statistics folded into global ones); the rescaling paragraph (a new larger
          max rescales the running output and denominator); the loop paragraph (one division by the
          final denominator after the last tile); the scope paragraph (deferred normalisation equals the
          paper's progressive normalisation).
  [A2D]   "ATTENTION2D" explainer, sections 2 and 3: per-fragment statistics combined through their
          commutativity and associativity give the exact result without approximation.
  [Ring]  "Ring Attention with Blockwise Parallel Transformers" explainer, section 3: the sequence is cut
          into contiguous blocks and key/value blocks are visited one after another.
  [SWIFT] "HOF SWIFT Attention", section 3, Transform stage: causal masking.

Readings where the pages are silent (each is listed with its reason in the design notes):
  * logits are scale * q.k with the scale supplied by the caller;
  * lse is the natural-log log-sum-exp of the scaled logits over the visible keys;
  * causal masking is bottom-right aligned: key j is visible to query i iff j <= i + offset, with the
    default offset N_kv - N_q;
  * a query with no visible key has O = 0 and lse = -inf, which is the identity of the merge;
  * chunk p of P covers keys [floor(p*N_kv/P), floor((p+1)*N_kv/P)) and is seen with offset - c_p;
  * chunks are folded left to right.

All arithmetic is float64.  Inputs are the exact values the GPU reads (fp32 or bf16 widened losslessly).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible(rows: np.ndarray, start: int, stop: int, causal: bool, offset: int) -> np.ndarray:
    """Boolean [len(rows), stop - start]: is key j in [start, stop) visible to the query at position i?

    Causal masking ([SWIFT] section 3) keeps j <= i + offset; without it every key is visible."""
    j = np.arange(start, stop)
    if not causal:
        return np.ones((len(rows), stop - start), dtype=bool)
    return j[None, :] <= (np.asarray(rows)[:, None] + offset)


def _rows_offset(n: int, n_kv: int, rows, offset):
    if rows is None:
        rows = np.arange(n)
    elif offset is None:
        raise ValueError("an explicit causal offset is needed when query positions are given")
    return np.asarray(rows), (n_kv - n if offset is None else offset)


def naive_head(q, k, v, scale: float, causal: bool = False, offset: int | None = None, rows=None):
    """The plain definition for one (b, h): full logit matrix, row softmax, product with V ([FA] steps).

    q: [n, d] queries, which sit at sequence positions ``rows`` (default 0..n-1); k, v: [n_kv, d].
    Returns (O [n, d], lse [n]).
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    n, n_kv = q.shape[0], k.shape[0]
    rows, offset = _rows_offset(n, n_kv, rows, offset)
    vis = visible(rows, 0, n_kv, causal, offset)
    s = scale * (q @ k.T)                       # logits
    s = np.where(vis, s, NEG_INF)
    o = np.zeros((n, v.shape[1]))
    lse = np.full(n, NEG_INF)
    has = vis.any(axis=1)
    if has.any():
        sh = s[has]
        m = sh.max(axis=1)
        lse[has] = m + np.log(np.exp(sh - m[:, None]).sum(axis=1))
        p = np.exp(sh - lse[has][:, None])      # softmax: each row sums to one
        o[has] = p @ v
    return o, lse


def blockwise_head(q, k, v, scale: float, causal: bool = False, offset: int | None = None, rows=None,
                   block: int = 64):
    """Online softmax over key blocks of ``block`` keys, ascending ([FA] online-softmax, per-tile flow,
    rescaling and loop paragraphs): running max m, running denominator l and unnormalised output a;
    one final division."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    n, n_kv = q.shape[0], k.shape[0]
    rows, offset = _rows_offset(n, n_kv, rows, offset)
    m = np.full(n, NEG_INF)
    l = np.zeros(n)
    a = np.zeros((n, v.shape[1]))
    for start in range(0, n_kv, block):
        stop = min(start + block, n_kv)
        vis = visible(rows, start, stop, causal, offset)
        s = np.where(vis, scale * (q @ k[start:stop].T), NEG_INF)   # tile logits
        m_tile = s.max(axis=1)                                      # tile-local max
        m_new = np.maximum(m, m_tile)
        live = m_new > NEG_INF                                      # rows that have seen a visible key
        m_ref = np.where(live, m_new, 0.0)          # the exponent reference (any finite value if not live)
        # rescale factor for what was accumulated under the old max (0 when nothing was accumulated)
        had = m > NEG_INF
        alpha = np.where(had, np.exp(np.where(had, m, m_ref) - m_ref), 0.0)
        p = np.where(vis & live[:, None], np.exp(s - m_ref[:, None]), 0.0)
        l = alpha * l + p.sum(axis=1)
        a = alpha[:, None] * a + p @ v[start:stop]
        m = m_new
    o = np.zeros_like(a)
    lse = np.full(n, NEG_INF)
    ok = l > 0
    o[ok] = a[ok] / l[ok][:, None]              # the single final division
    lse[ok] = m[ok] + np.log(l[ok])
    return o, lse


def merge(o_a, lse_a, o_b, lse_b):
    """Combine two partial results over disjoint key sets ([A2D] sections 2-3; rescale rule of [FA]).

    Each partial is (O_x, L_x) with O_x the softmax-weighted output over its keys and L_x their
    log-sum-exp.  With M = max(L_a, L_b): w_x = exp(L_x - M); O = (w_a O_a + w_b O_b) / (w_a + w_b);
    L = M + ln(w_a + w_b).  Rows with M = -inf stay (0, -inf).
    """
    o_a, o_b = _as64(o_a), _as64(o_b)
    lse_a, lse_b = _as64(lse_a), _as64(lse_b)
    big = np.maximum(lse_a, lse_b)
    live = big > NEG_INF
    safe = np.where(live, big, 0.0)
    w_a = np.where(live, np.exp(lse_a - safe), 0.0)
    w_b = np.where(live, np.exp(lse_b - safe), 0.0)
    tot = w_a + w_b
    den = np.where(live, tot, 1.0)
    o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / den[..., None]
    lse = np.where(live, safe + np.log(np.where(live, tot, 1.0)), NEG_INF)
    return o, lse


def chunk_bounds(n_kv: int, chunks: int) -> list[int]:
    """c_p = floor(p * N_kv / P), p = 0..P: contiguous chunks whose sizes differ by at most one."""
    return [(p * n_kv) // chunks for p in range(chunks + 1)]


def chunked_head(q, k, v, scale: float, causal: bool = False, offset: int | None = None, rows=None,
                 chunks: int = 1, form: str = "naive", block: int = 64):
    """Split the keys into P contiguous chunks ([Ring] section 3), attend to each on its own with the
    causal offset shifted by the chunk start, and fold the partials left to right with ``merge``."""
    q = _as64(q)
    n, n_kv = q.shape[0], np.shape(k)[0]
    rows, offset = _rows_offset(n, n_kv, rows, offset)
    cb = chunk_bounds(n_kv, chunks)
    o = np.zeros((n, np.shape(v)[1]))
    lse = np.full(n, NEG_INF)
    for p in range(chunks):
        lo, hi = cb[p], cb[p + 1]
        if hi == lo:
            continue                         # an empty chunk is the merge identity
        if form == "naive":
            o_p, lse_p = naive_head(q, k[lo:hi], v[lo:hi], scale, causal, offset - lo, rows)
        else:
            o_p, lse_p = blockwise_head(q, k[lo:hi], v[lo:hi], scale, causal, offset - lo, rows, block)
        if p == 0:
            o, lse = o_p, lse_p
        else:
            o, lse = merge(o, lse, o_p, lse_p)
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False, offset: int | None = None, form: str = "naive",
              block: int = 64, chunks: int = 1):
    """Batched front end: q [..., N_q, d], k and v [..., N_kv, d] -> (O [..., N_q, d], lse [..., N_q])."""
    q, k, v = _as64(q), _as64(k), _as64(v)
    lead = q.shape[:-2]
    n, d = q.shape[-2], v.shape[-1]
    qf = q.reshape(-1, n, q.shape[-1])
    kf = k.reshape(-1, k.shape[-2], k.shape[-1])
    vf = v.reshape(-1, v.shape[-2], d)
    o = np.empty((qf.shape[0], n, d))
    lse = np.empty((qf.shape[0], n))
    for i in range(qf.shape[0]):
        if chunks > 1:
            o[i], lse[i] = chunked_head(qf[i], kf[i], vf[i], scale, causal, offset, None, chunks, form, block)
        elif form == "naive":
            o[i], lse[i] = naive_head(qf[i], kf[i], vf[i], scale, causal, offset)
        else:
            o[i], lse[i] = blockwise_head(qf[i], kf[i], vf[i], scale, causal, offset, None, block)
    return o.reshape(*lead, n, d), lse.reshape(*lead, n)
