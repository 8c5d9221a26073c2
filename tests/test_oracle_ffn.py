"""The blockwise feed-forward oracle against its pins, and planted mistakes in copies of it, each of which
must fail at least one pin."""
import types

import pytest

import oracle.ffn64 as base
import oracle_ffn_pins

with open(base.__file__) as _f:
    SOURCE = _f.read()

MUTANTS = {
    "gelu_tanh_form": ("return x * 0.5 * (1.0 + erf(x / np.sqrt(2.0)))",
                       "return x * 0.5 * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.044715 * x ** 3)))"),
    "gelu_sign": ("erf(x / np.sqrt(2.0))", "erf(-x / np.sqrt(2.0))"),
    "gelu_scale": ("erf(x / np.sqrt(2.0))", "erf(x / 2.0)"),
    "b1_dropped": ("pre = pre + _as64(b1)[None, :]", "pre = pre"),
    "b2_dropped": ("y = y + _as64(b2)[None, :]", "y = y"),
    "w1_untransposed": ("pre = x @ w1.T", "pre = (w1 @ x.T).T[:, ::-1]"),
    "act_after_w2": ("h = ACTS[act](pre)\n    y = h @ w2.T", "h = pre\n    y = ACTS[act](h @ w2.T)"),
    "blocks_drop_last_row": ("return list(range(0, n, block)) + [n]", "return list(range(0, n, block)) + [n - 1]"),
    "blocks_overlap": ("out[bb[i]:bb[i + 1]] = ffn_rows(x[bb[i]:bb[i + 1]]",
                       "out[bb[i]:bb[i + 1]] = ffn_rows(x[max(bb[i] - 1, 0):bb[i + 1] - (bb[i] > 0)]"),
}


def _build(name):
    old, new = MUTANTS[name]
    assert old in SOURCE, f"mutant {name}: snippet not found in the oracle source"
    mod = types.ModuleType(f"ffn_mutant_{name}")
    exec(compile(SOURCE.replace(old, new), f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("check", oracle_ffn_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_ffn_oracle_pin(check):
    check(base)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_ffn_mutant_is_caught(name):
    mod = _build(name)
    failures = []
    for check in oracle_ffn_pins.ALL_CHECKS:
        try:
            check(mod)
        except Exception as e:  # noqa: BLE001 - any failure (assertion or crash) counts as caught
            failures.append(f"{check.__name__}: {type(e).__name__}")
    assert failures, f"planted mistake {name!r} passed every pin"
