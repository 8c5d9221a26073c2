"""GPU parity of the partial-result entry points on seeded random cases: attn_fwd_ex over a random key range of a
longer K/V (strided heads) with a random causal offset and output dtype, attn_fwd_acc folding a second random
range into the first range's fp32 partial (in place or not, ranges in either order), and attn_merge of random
partials.  Each result is compared in full against the fp64 oracle: the range's own attention ("FlashAttention by
hand", online softmax with one final division; causal visibility j <= i + offset as in the SWIFT paper,
section 3) and the oracle's two-term merge ("ATTENTION2D" explainer, section 2).

Offsets are drawn across and beyond the range's key count, so a case can hold rows that see every key, rows that
see part of the range, and rows that see none (O = 0, LSE = -inf), the cases a ring or 2-D scheme hands to one
device.  For bf16 the workgroup size alternates between four and eight waves (ATTN_BF16_D{d}_WAVES).
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import exact_blockwise_attention_fwd_amd as A
import oracle
import workloads as W
from parity import TOL, LSE_TOL, assert_parity, errors, out_to_f64, storage_to_f64, to_device

pytestmark = pytest.mark.gpu


def _offset(rng, n_q: int, n_kv: int) -> int:
    """A causal offset: the bottom-right default, one that hides the whole range, one that shows it all,
    or any value in between."""
    kind = int(rng.integers(0, 4))
    if kind == 0:
        return n_kv - n_q
    if kind == 1:
        return int(rng.integers(-n_q - 40, 0))         # the first rows (or all rows) see nothing
    if kind == 2:
        return int(rng.integers(n_kv, n_kv + 50))      # every row sees the whole range
    return int(rng.integers(-n_q, n_kv + 1))


def _cases(n: int = 60):
    rng = np.random.default_rng(20261204)
    out = []
    for i in range(n):
        dt = "bf16" if i % 3 != 2 else "f32"
        d = int(rng.choice([128, 64])) if dt == "bf16" else int(rng.choice([64, 37, 128, 8]))
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 5))
        N_q = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 600))]))
        n_total = int(rng.integers(2, 1600))
        lo1 = int(rng.integers(0, n_total - 1))
        hi1 = int(rng.integers(lo1 + 1, n_total + 1))
        causal = bool(rng.integers(0, 4) != 0)
        off1 = _offset(rng, N_q, hi1 - lo1)
        mode = "ex" if i % 2 == 0 else "acc"
        # the folded range: disjoint from the first, before or after it, of any length; its offset keeps both
        # ranges on one query-key timeline (key j of the whole K/V is visible when j <= i + offset_global)
        rest = [(0, lo1), (hi1, n_total)]
        rest = [(a, b) for a, b in rest if b > a]
        if mode == "acc" and rest:
            a, b = rest[int(rng.integers(0, len(rest)))]
            lo2 = int(rng.integers(a, b))
            hi2 = int(rng.integers(lo2 + 1, b + 1))
        else:
            mode, lo2, hi2 = "ex", 0, 0
        out_f32 = bool(rng.integers(0, 2)) if dt == "bf16" else True
        in_place = mode == "acc" and bool(rng.integers(0, 2))
        waves = ("4" if i % 2 else "8") if dt == "bf16" else None
        out.append(dict(i=i, dt=dt, d=d, B=B, H=H, N_q=N_q, n_total=n_total, r1=(lo1, hi1), r2=(lo2, hi2),
                        causal=causal, off1=off1, mode=mode, out_f32=out_f32, in_place=in_place, waves=waves))
    return out


CASES = _cases()


def _id(c):
    r1 = f"{c['r1'][0]}-{c['r1'][1]}"
    r2 = f"+{c['r2'][0]}-{c['r2'][1]}" if c["mode"] == "acc" else ""
    return (f"{c['mode']}{'_ip' if c['in_place'] else ''}-{c['B']}x{c['H']}x{c['N_q']}of{c['n_total']}k{r1}{r2}"
            f"d{c['d']}{c['dt']}{'c' if c['causal'] else 'n'}o{c['off1']}{'f' if c['out_f32'] else ''}"
            + (f"w{c['waves']}" if c["waves"] else ""))


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    A.lib()


def _inputs(c):
    w = W.Workload("partials", c["B"], c["H"], c["N_q"], c["n_total"], c["d"], c["dt"], c["causal"], 1,
                   seed=9000 + c["i"])
    st = [W.tensor_storage(w, t) for t in (W.Q_T, W.K_T, W.V_T)]
    return w.scale, st


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_random_partial(case, monkeypatch):
    c = case
    if c["waves"]:
        monkeypatch.setenv(f"ATTN_BF16_D{c['d']}_WAVES", c["waves"])
    scale, st = _inputs(c)
    q, k, v = (to_device(s) for s in st)
    qq, kk, vv = (storage_to_f64(s) for s in st)
    causal, (lo1, hi1), off1 = c["causal"], c["r1"], c["off1"]
    ref1 = oracle.attention(qq, kk[:, :, lo1:hi1], vv[:, :, lo1:hi1], scale, causal, off1)
    odt = torch.float32 if c["out_f32"] else q.dtype
    o1, l1 = A.fwd_ex(q, k, v, causal, scale, causal_offset=off1, key_range=(lo1, hi1), out_dtype=odt)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o1), out_to_f64(l1), *ref1)
    print(_id(c), "range", err, flush=True)
    assert_parity(err, c["dt"], _id(c) + " range")
    if c["mode"] != "acc":
        return
    lo2, hi2 = c["r2"]
    off2 = off1 + lo1 - lo2                          # the same global offset, seen from the second range
    ref2 = oracle.attention(qq, kk[:, :, lo2:hi2], vv[:, :, lo2:hi2], scale, causal, off2)
    ref = oracle.merge(*ref1, *ref2)
    if not c["out_f32"]:                             # fwd_acc folds into an fp32 partial
        o1, l1 = A.fwd_ex(q, k, v, causal, scale, causal_offset=off1, key_range=(lo1, hi1),
                          out_dtype=torch.float32)
    if c["in_place"]:
        o, lse = A.fwd_acc(q, k, v, o1, l1, causal, scale, causal_offset=off2, key_range=(lo2, hi2),
                           out_dtype=torch.float32, out=o1, lse=l1)
        assert o.data_ptr() == o1.data_ptr() and lse.data_ptr() == l1.data_ptr()
    else:
        o, lse = A.fwd_acc(q, k, v, o1, l1, causal, scale, causal_offset=off2, key_range=(lo2, hi2),
                           out_dtype=torch.float32 if c["i"] % 4 == 1 else q.dtype)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), *ref)
    print(_id(c), "fold", err, flush=True)
    assert_parity(err, c["dt"], _id(c) + " fold")


# --------------------------------------------------------------------------------------------- merge
def _merge_cases(n: int = 24):
    rng = np.random.default_rng(20261205)
    out = []
    for i in range(n):
        din = "bf16" if i % 3 == 0 else "f32"
        dout = "bf16" if i % 4 == 1 else "f32"
        d = int(rng.choice([1, 3, 4, 8, 16, 37, 64, 100, 128, 192, 256, 257, 300]))
        lead = (int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.integers(1, 900)))
        spread = float(rng.choice([0.5, 5.0, 60.0]))   # LSE differences from near-ties to one side vanishing
        out.append((i, din, dout, d, lead, spread))
    return out


MERGE = _merge_cases()


@pytest.mark.parametrize("case", MERGE, ids=lambda c: f"{c[1]}to{c[2]}d{c[3]}r{'x'.join(map(str, c[4]))}s{c[5]:g}")
def test_random_merge(case):
    """Partials with LSE offsets up to the fp32 exponent's reach, exact ties, and -inf rows on either side
    or both; shapes [B, H, N] with any d from 1 up, so both merge kernels and ragged row groups are met."""
    i, din, dout, d, lead, spread = case
    rng = np.random.default_rng((20261206, i))
    oa = rng.standard_normal(lead + (d,)).astype(np.float32)
    ob = rng.standard_normal(lead + (d,)).astype(np.float32)
    la = (rng.standard_normal(lead) * spread).astype(np.float32)
    lb = (rng.standard_normal(lead) * spread).astype(np.float32)
    tie = rng.random(lead) < 0.1
    lb[tie] = la[tie]
    for o_, l_, p in ((oa, la, 0.08), (ob, lb, 0.08)):
        empty = rng.random(lead) < p
        l_[empty] = -np.inf
        o_[empty] = 0.0
    if din == "bf16":
        oa, ob = W.f32_to_bf16_bits(oa), W.f32_to_bf16_bits(ob)
    ref_o, ref_l = oracle.merge(storage_to_f64(oa), la.astype(np.float64), storage_to_f64(ob),
                                lb.astype(np.float64))
    tdt = torch.bfloat16 if dout == "bf16" else torch.float32
    o, lse = A.merge(to_device(oa), to_device(la), to_device(ob), to_device(lb), out_dtype=tdt)
    torch.cuda.synchronize()
    err = errors(out_to_f64(o), out_to_f64(lse), ref_o, ref_l)
    print(case, err, flush=True)
    assert not err["nan"] and err["lse_inf_match"], err
    assert err["max_abs"] <= TOL[dout]["max_abs"], err
    if dout == "bf16":
        assert err["rel_rms"] <= TOL["bf16"]["rel_rms"], err
    # the LSE of a merge is fp32 arithmetic on fp32 inputs: a few ulps of its magnitude
    assert err["lse_abs"] <= max(LSE_TOL * 0.1, 4 * np.finfo(np.float32).eps * float(np.max(np.abs(
        np.where(np.isfinite(ref_l), ref_l, 0.0)), initial=1.0))), err
    assert math.isfinite(err["max_abs"])
