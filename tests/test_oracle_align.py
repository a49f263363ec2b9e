"""Pins of the oracle's start-aligned causal option (the pages' ``j <= i``
rule of "Verify tiled attention", section "Compare the attention outputs",
read literally for Sq != Skv), each against something other than the
function itself: the end-aligned path where the two readings coincide,
non-causal attention over a key prefix, and plain Python loops."""
import math

import numpy as np
import pytest

import oracle


def _qkv(Sq, Skv, d, seed):
    rng = np.random.default_rng(seed)
    return rng.normal(size=(Sq, d)), rng.normal(size=(Skv, d)), rng.normal(size=(Skv, d))


def test_start_equals_end_when_square():
    q, k, v = _qkv(37, 37, 8, 1)
    oe, le = oracle.direct_attention(q, k, v, causal=True, align="end")
    os_, ls = oracle.direct_attention(q, k, v, causal=True, align="start")
    assert np.array_equal(oe, os_) and np.array_equal(le, ls)


@pytest.mark.parametrize("Sq,Skv", [(5, 9), (12, 7), (1, 6), (6, 1)])
def test_start_aligned_row_is_prefix_attention(Sq, Skv):
    # row i sees keys 0..i: the non-causal attention of that row over the
    # first min(i + 1, Skv) keys
    q, k, v = _qkv(Sq, Skv, 4, Sq * 10 + Skv)
    o, lse = oracle.direct_attention(q, k, v, causal=True, align="start")
    for i in range(Sq):
        n = min(i + 1, Skv)
        oi, li = oracle.direct_attention(q[i:i + 1], k[:n], v[:n], causal=False)
        assert np.max(np.abs(o[i] - oi[0])) < 1e-14 and abs(lse[i] - li[0]) < 1e-12


def test_start_aligned_brute_force():
    q, k, v = _qkv(3, 4, 2, 7)
    scale = 0.7
    o, lse = oracle.direct_attention(q, k, v, scale=scale, causal=True, align="start")
    for i in range(3):
        w = [math.exp(scale * sum(q[i][c] * k[j][c] for c in range(2))) for j in range(i + 1)]
        tot = sum(w)
        for c in range(2):
            ref = sum(w[j] * v[j][c] for j in range(i + 1)) / tot
            assert abs(o[i][c] - ref) < 1e-14
        assert abs(lse[i] - math.log(tot)) < 1e-13


def test_alignments_differ_when_not_square():
    # the pins above would catch an offset mix-up: the readings disagree here
    q, k, v = _qkv(5, 9, 4, 3)
    oe, _ = oracle.direct_attention(q, k, v, causal=True, align="end")
    os_, _ = oracle.direct_attention(q, k, v, causal=True, align="start")
    assert np.max(np.abs(oe - os_)) > 0.1


def test_unknown_alignment_rejected():
    with pytest.raises(ValueError):
        oracle.last_visible_key(0, 4, 4, True, align="middle")
