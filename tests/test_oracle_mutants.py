"""Planted mistakes in a copy of the oracle must each fail at least one pin.

Each mutant edits the oracle's source text (on the CPU, in memory) in one plausible way: a dropped term,
a wrong sign or index, a transposed operand, an off-by-one mask, a missing rescale.  If a mutant passed
every check in ``oracle_pins``, that mistake could hide in the oracle undetected.
"""
import types

import numpy as np
import pytest

import oracle.fp64 as base
import oracle_pins

with open(base.__file__) as _f:
    SOURCE = _f.read()

MUTANTS = {
    "scale_dropped": ("s = scale * (q @ k.T)", "s = (q @ k.T)"),
    "logits_transposed": ("s = scale * (q @ k.T)", "s = scale * (k @ q.T).T[:, ::-1]"),
    "causal_off_by_one": ("j[None, :] <= (np.asarray(rows)[:, None] + offset)",
                          "j[None, :] < (np.asarray(rows)[:, None] + offset)"),
    "causal_top_left": ("(n_kv - n if offset is None else offset)", "(0 if offset is None else offset)"),
    "lse_base2": ("lse[has] = m + np.log(np.exp(sh - m[:, None]).sum(axis=1))",
                  "lse[has] = m + np.log2(np.exp(sh - m[:, None]).sum(axis=1))"),
    "softmax_sign": ("p = np.exp(sh - lse[has][:, None])", "p = np.exp(lse[has][:, None] - sh)"),
    "v_rows_reversed": ("o[has] = p @ v", "o[has] = p @ v[::-1]"),
    "blockwise_no_rescale_acc": ("a = alpha[:, None] * a + p @ v[start:stop]", "a = a + p @ v[start:stop]"),
    "blockwise_no_rescale_den": ("l = alpha * l + p.sum(axis=1)", "l = l + p.sum(axis=1)"),
    "blockwise_max_not_running": ("m_new = np.maximum(m, m_tile)", "m_new = np.where(m_tile > NEG_INF, m_tile, m)"),
    "blockwise_lse_drops_max": ("lse[ok] = m[ok] + np.log(l[ok])", "lse[ok] = np.log(l[ok])"),
    "merge_weights_swapped": ("o = (w_a[..., None] * o_a + w_b[..., None] * o_b)",
                              "o = (w_b[..., None] * o_a + w_a[..., None] * o_b)"),
    "merge_lse_drops_max": ("lse = np.where(live, safe + np.log(", "lse = np.where(live, np.log("),
    "merge_no_normalise": ("/ den[..., None]", "/ 1.0"),
    "chunk_offset_not_shifted": ("scale, causal, offset - lo, rows)", "scale, causal, offset, rows)"),
    "chunk_overlap": ("lo, hi = cb[p], cb[p + 1]", "lo, hi = cb[p], min(cb[p + 1] + 1, n_kv)"),
    "batched_heads_reversed": ("kf = k.reshape(-1, k.shape[-2], k.shape[-1])",
                               "kf = k.reshape(-1, k.shape[-2], k.shape[-1])[::-1]"),
    "batched_chunked_offset_dropped": ("chunked_head(qf[i], kf[i], vf[i], scale, causal, offset, None",
                                       "chunked_head(qf[i], kf[i], vf[i], scale, causal, None, None"),
    "batched_values_of_head_zero": ("vf = v.reshape(-1, v.shape[-2], d)",
                                   "vf = np.repeat(v.reshape(-1, v.shape[-2], d)[:1], qf.shape[0], axis=0)"),
    "chunk_bounds_drop_last_key": ("return [(p * n_kv) // chunks for p in range(chunks + 1)]",
                                   "return [(p * (n_kv - 1)) // chunks for p in range(chunks + 1)]"),
}


def _build(name):
    old, new = MUTANTS[name]
    assert old in SOURCE, f"mutant {name}: snippet not found in the oracle source"
    mod = types.ModuleType(f"oracle_mutant_{name}")
    exec(compile(SOURCE.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _build(name)
    failures = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):   # a broken oracle may overflow; that is the mistake being caught
                check(mod)
        except Exception as e:  # noqa: BLE001 - any failure (assertion or crash) counts as caught
            failures.append(f"{check.__name__}: {type(e).__name__}")
    assert failures, f"planted mistake {name!r} passed every pin"
