"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (never in the
oracle itself: the copy is compiled into a module of its own, on the CPU),
points the pins of test_oracle_pins at that copy and requires the named pin
to fail.  The unmodified oracle passes the same pins (test_oracle_pins), so a
failure here can only come from the planted mistake."""
import inspect
import types

import pytest

import test_oracle_pins as pins
from oracle import attention as orc

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

_SRC = inspect.getsource(orc)

# (label, text in the oracle, its mistaken replacement, pin, pin arguments)
MUTANTS = [
    ("group_index", "g = h // G", "g = h % Hkv",
     pins.test_against_torch_sdpa, dict(causal=True, window=0, sink=False, hq=4, hkv=2)),
    ("window_off_by_one", "m &= kpos > qpos - window", "m &= kpos >= qpos - window",
     pins.test_window_counts, {}),
    ("causal_off_by_one", "m &= kpos <= qpos", "m &= kpos < qpos",
     pins.test_length_one_sequences_closed_form, {}),
    ("dS_without_scale", "dS = P * (dP - delta[h, rows][:, None]) * scale",
     "dS = P * (dP - delta[h, rows][:, None])",
     pins.test_finite_differences, dict(causal=True, window=0, sink=False)),
    ("dsink_sign", "dsink = -(np.exp(sink[:, None] - lse) * delta).sum(axis=1)",
     "dsink = (np.exp(sink[:, None] - lse) * delta).sum(axis=1)",
     pins.test_finite_differences, dict(causal=False, window=0, sink=True)),
    ("delta_from_wrong_operand", 'delta = np.einsum("thd,thd->ht", do, o)',
     'delta = np.einsum("thd,thd->ht", do, q)',
     pins.test_invariants, dict(causal=True, window=0, sink=False)),
    ("dK_from_dO", "dk[keys, g] += dS.T @ Qr", "dk[keys, g] += dS.T @ dOr",
     pins.test_finite_differences, dict(causal=False, window=0, sink=False)),
    ("dQ_from_V", "dq[rows, h] = dS @ Kc", "dq[rows, h] = dS @ Vc",
     pins.test_zero_queries_closed_form, dict(causal=True, window=3)),
    ("dV_perturbed", "dv[keys, g] += P.T @ dOr", "dv[keys, g] += 1.001 * (P.T @ dOr)",
     pins.test_invariants, dict(causal=False, window=0, sink=False)),
    ("sink_left_out", "tot = tot + np.exp(sink_h - mz)", "tot = tot + 0.0",
     pins.test_against_torch_sdpa, dict(causal=True, window=3, sink=True, hq=4, hkv=4)),
    ("lse_base_2", "lse = np.where(ok, mz + np.log(tot), -np.inf)",
     "lse = np.where(ok, mz + np.log2(tot), -np.inf)",
     pins.test_against_torch_sdpa, dict(causal=False, window=0, sink=False, hq=4, hkv=4)),
    ("key_range_drops_last_key", "    k1 = r1 if causal else L", "    k1 = r1 - 1 if causal else L",
     pins.test_row_chunking_does_not_change_results, {}),
]


def _mutant(old: str, new: str) -> types.ModuleType:
    assert _SRC.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(_SRC.replace(old, new), "<oracle mutant>", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("label,old,new,pin,kw", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pin_catches_mutant(label, old, new, pin, kw, monkeypatch):
    monkeypatch.setattr(pins, "orc", _mutant(old, new))
    with pytest.raises(AssertionError):
        pin(**kw)


def test_unmutated_copy_passes_the_same_pins(monkeypatch):
    # the compile-a-copy route itself changes nothing
    monkeypatch.setattr(pins, "orc", _mutant("g = h // G", "g = h // G"))
    for _, _, _, pin, kw in MUTANTS:
        pin(**kw)
