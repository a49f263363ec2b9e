"""Plant plausible mistakes in the oracle (on the CPU) and require that the
pins catch every one of them: a pin set that a dropped term, a wrong sign or
index, or a swapped operand slips through would not be worth trusting."""
import math

import numpy as np
import pytest

import oracle
import oracle.attention as oa
from pin_checks import ALL_DIRECT_CHECKS


def _run_all(direct):
    caught = []
    for chk in ALL_DIRECT_CHECKS:
        if chk(direct):
            caught.append(chk.__name__)
    return caught


def _dropped_scale(q, k, v, scale=None, causal=False, **kw):
    return oracle.direct_attention(q, k, v, scale=1.0, causal=causal, **kw)


def _swapped_kv(q, k, v, scale=None, causal=False, **kw):
    if np.shape(k) != np.shape(v):
        return oracle.direct_attention(q, k, v, scale=scale, causal=causal, **kw)
    return oracle.direct_attention(q, v, k, scale=scale, causal=causal, **kw)


def _no_max_shift(q, k, v, scale=None, causal=False, **kw):
    kw.pop("subtract_max", None)
    return oracle.direct_attention(q, k, v, scale=scale, causal=causal, subtract_max=False, **kw)


def _lse_log2(q, k, v, scale=None, causal=False, **kw):
    o, lse = oracle.direct_attention(q, k, v, scale=scale, causal=causal, **kw)
    return o, lse / math.log(2.0)


def _lse_without_max(q, k, v, scale=None, causal=False, **kw):
    o, lse = oracle.direct_attention(q, k, v, scale=scale, causal=causal, **kw)
    # a planted mistake: log of the shifted sum only (the max term dropped)
    q_, k_ = np.asarray(q, float), np.asarray(k, float)
    sc = scale if scale is not None else 1.0 / math.sqrt(q_.shape[-1])
    if k_.shape[-2] == 0:
        return o, lse
    m = (q_ @ np.swapaxes(k_, -1, -2) * sc).max(axis=-1)
    return o, np.where(np.isfinite(lse), lse - m, lse)


def _reversed_values(q, k, v, scale=None, causal=False, **kw):
    return oracle.direct_attention(q, k, np.asarray(v)[..., ::-1, :], scale=scale,
                                   causal=causal, **kw)


MUTANTS = {
    "dropped_scale": _dropped_scale,
    "swapped_k_v": _swapped_kv,
    "no_max_shift": _no_max_shift,
    "lse_in_log2": _lse_log2,
    "lse_without_max": _lse_without_max,
    "reversed_value_rows": _reversed_values,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    assert _run_all(MUTANTS[name]), f"no pin caught the planted mistake {name}"


def _causal_off_by_one(i, Sq, Skv, causal):
    if not causal:
        return Skv
    return max(0, min(Skv, i + (Skv - Sq)))          # j < i instead of j <= i


def _causal_top_left(i, Sq, Skv, causal):
    if not causal:
        return Skv
    return max(0, min(Skv, i + 1))                    # ignores the Skv - Sq offset


def _causal_ignored(i, Sq, Skv, causal):
    return Skv


@pytest.mark.parametrize("bad", [_causal_off_by_one, _causal_top_left, _causal_ignored],
                         ids=lambda f: f.__name__)
def test_planted_mask_mistake_is_caught(monkeypatch, bad):
    monkeypatch.setattr(oa, "last_visible_key", bad)
    assert _run_all(oracle.direct_attention), f"no pin caught {bad.__name__}"


def test_real_oracle_passes_everything():
    assert _run_all(oracle.direct_attention) == []
