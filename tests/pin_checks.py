"""Checks that pin the fp64 oracle to facts fixed by the pages and by
mathematics, not by the oracle itself.

Each ``check_*`` takes the direct-attention callable under test (same
signature as ``oracle.direct_attention``) and returns a list of failure
messages; an empty list means the pin holds.  ``test_oracle_pins.py`` runs
them on the oracle; ``test_oracle_mutants.py`` runs them on oracles with a
planted mistake and requires that every mistake is caught by some pin.
"""
from __future__ import annotations

import json
import math
import os
from decimal import Decimal, getcontext
from typing import Callable, List

import numpy as np
import torch

from seeded_inputs import p1_make_qkv

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _catch(fn) -> List[str]:
    try:
        return fn()
    except Exception as e:  # a crash of the implementation under test is a failed pin
        return [f"raised {type(e).__name__}: {e}"]


# ---------------------------------------------------------------- worked example
def worked_example_closed_form():
    """Scores 0, 10, 20 over values 1, 3, 5 ("A failing baseline" on "Tiled
    attention: preserving results without a full score matrix"), evaluated
    exactly in 50-digit decimal arithmetic: softmax weights e^s / sum e^s."""
    getcontext().prec = 50
    s = [Decimal(0), Decimal(10), Decimal(20)]
    vals = [Decimal(1), Decimal(3), Decimal(5)]
    e = [x.exp() for x in s]
    full = sum(w * x for w, x in zip(e, vals)) / sum(e)
    lse = sum(e).ln()
    first = (e[0] * vals[0] + e[1] * vals[1]) / (e[0] + e[1])
    block_avg = (first + vals[2]) / 2
    return float(full), float(lse), float(block_avg)


def check_worked_example(direct: Callable) -> List[str]:
    def run():
        fails = []
        full, lse_ref, _ = worked_example_closed_form()
        q = np.array([[1.0]])
        k = np.array([[0.0], [10.0], [20.0]])
        v = np.array([[1.0], [3.0], [5.0]])
        o, lse = direct(q, k, v, scale=1.0, causal=False)
        if abs(o[0, 0] - full) > 1e-13:
            fails.append(f"worked example O {o[0,0]!r} != {full!r}")
        if abs(lse[0] - lse_ref) > 1e-13:
            fails.append(f"worked example LSE {lse[0]!r} != {lse_ref!r}")
        return fails
    return _catch(run)


# ---------------------------------------------------------------- printed lab values
def check_p1_printed(direct: Callable) -> List[str]:
    def run():
        g = golden("p1_lab_results.json")
        st, pr = g["setup"], g["printed"]
        q, k, v = p1_make_qkv(st["seq_len"], st["head_dim"], st["seed"])
        o, _ = direct(q, k, v, scale=1.0 / math.sqrt(st["head_dim"]), causal=True)
        fails = []
        for got, want, name in ((o[0, :4], pr["sample_row0_first4"], "row0"),
                                (o[-1, :4], pr["sample_last_row_first4"], "last row")):
            # the page rounds to 6 decimals: the exact value lies within 5e-7
            if np.max(np.abs(np.asarray(got) - np.asarray(want))) > 5.0000001e-7:
                fails.append(f"{name} {got} does not round to printed {want}")
        return fails
    return _catch(run)


# ---------------------------------------------------------------- library routine
def _mask(Sq: int, Skv: int, causal: bool) -> torch.Tensor:
    i = torch.arange(Sq)[:, None]
    j = torch.arange(Skv)[None, :]
    return (j <= i + (Skv - Sq)) if causal else torch.ones(Sq, Skv, dtype=torch.bool)


def check_library_sdpa(direct: Callable) -> List[str]:
    """torch's own CPU scaled-dot-product attention in float64 (an independent
    implementation) with an explicit boolean mask, and torch.logsumexp of the
    masked scaled scores for the LSE."""
    def run():
        fails = []
        g = torch.Generator().manual_seed(1234)
        cases = [(2, 3, 17, 17, 8, False, None), (1, 2, 33, 33, 16, True, None),
                 (2, 1, 5, 40, 32, True, 0.3), (1, 1, 24, 9, 4, False, 1.7),
                 (1, 2, 12, 31, 8, True, None)]
        for B, H, Sq, Skv, d, causal, scale in cases:
            q = torch.randn(B, H, Sq, d, generator=g, dtype=torch.float64)
            k = torch.randn(B, H, Skv, d, generator=g, dtype=torch.float64)
            v = torch.randn(B, H, Skv, d, generator=g, dtype=torch.float64)
            sc = scale if scale is not None else 1.0 / math.sqrt(d)
            m = _mask(Sq, Skv, causal)
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, attn_mask=m, scale=sc)
            s = torch.matmul(q, k.transpose(-1, -2).contiguous()) * sc
            s = s.masked_fill(~m, -math.inf)
            lse_ref = torch.logsumexp(s, dim=-1)
            o, lse = direct(q.numpy(), k.numpy(), v.numpy(), scale=sc, causal=causal)
            err = float(np.max(np.abs(o - ref.numpy())))
            lerr = float(np.max(np.abs(lse - lse_ref.numpy())))
            if not err < 1e-12:
                fails.append(f"O vs torch SDPA {err:.3e} at {(B,H,Sq,Skv,d,causal)}")
            if not lerr < 1e-12:
                fails.append(f"LSE vs torch logsumexp {lerr:.3e} at {(B,H,Sq,Skv,d,causal)}")
        return fails
    return _catch(run)


# ---------------------------------------------------------------- closed forms
def check_zero_queries(direct: Callable) -> List[str]:
    """Q = 0 makes every visible score 0, so softmax is uniform: O_i is the
    mean of the visible V rows and LSE_i = ln |Vis_i|."""
    def run():
        fails = []
        rng = np.random.default_rng(5)
        for Sq, Skv, causal in ((16, 16, True), (6, 20, True), (20, 7, True), (9, 13, False)):
            d = 4
            q = np.zeros((Sq, d))
            k = rng.standard_normal((Skv, d))
            v = rng.standard_normal((Skv, d))
            o, lse = direct(q, k, v, causal=causal)
            for i in range(Sq):
                n = Skv if not causal else max(0, min(Skv, i + Skv - Sq + 1))
                want_o = v[:n].mean(axis=0) if n else np.zeros(d)
                want_l = math.log(n) if n else -math.inf
                if np.max(np.abs(o[i] - want_o)) > 1e-13:
                    fails.append(f"Q=0 row {i} O mismatch ({Sq},{Skv},{causal})")
                if not (lse[i] == want_l or abs(lse[i] - want_l) < 1e-13):
                    fails.append(f"Q=0 row {i} LSE {lse[i]} != {want_l} ({Sq},{Skv},{causal})")
        return fails
    return _catch(run)


def check_single_visible_key(direct: Callable) -> List[str]:
    """A causal first row (Sq == Skv) sees only key 0: weight exp(0)/1 = 1, so
    O_0 is V_0 exactly and LSE_0 is the scaled score itself."""
    def run():
        rng = np.random.default_rng(6)
        q, k, v = (rng.standard_normal((10, 8)) for _ in range(3))
        o, lse = direct(q, k, v, causal=True)
        fails = []
        if not np.array_equal(o[0], v[0]):
            fails.append("row 0 is not V_0 bit for bit")
        if abs(lse[0] - float(q[0] @ k[0]) / math.sqrt(8)) > 1e-14:
            fails.append("row 0 LSE is not its own scaled score")
        return fails
    return _catch(run)


def check_two_keys(direct: Callable) -> List[str]:
    """Two keys: the weights are the logistic function of the score gap,
    sigma(x) = 1 / (1 + e^-x)."""
    def run():
        q = np.array([[0.7, -1.1, 0.25]])
        k = np.array([[1.0, 0.5, -2.0], [-0.3, 0.8, 1.5]])
        v = np.array([[2.0, -1.0, 0.0], [0.5, 4.0, -3.0]])
        sc = 0.9
        s1, s2 = sc * float(q[0] @ k[0]), sc * float(q[0] @ k[1])
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        want = w1 * v[0] + (1.0 - w1) * v[1]
        want_lse = max(s1, s2) + math.log1p(math.exp(-abs(s1 - s2)))
        o, lse = direct(q, k, v, scale=sc, causal=False)
        fails = []
        if np.max(np.abs(o[0] - want)) > 1e-14:
            fails.append(f"two-key O {o[0]} != {want}")
        if abs(lse[0] - want_lse) > 1e-14:
            fails.append(f"two-key LSE {lse[0]} != {want_lse}")
        return fails
    return _catch(run)


def check_overflow_case(direct: Callable) -> List[str]:
    """The overflow check of "Read the executable checks" on "Verify tiled
    attention": with the max shift the result stays finite.  Closed form:
    scores 500*2/sqrt(2) and 500*4/sqrt(2); weights are logistic in the gap."""
    def run():
        c = golden("p1_unit_checks.json")["overflow"]
        q, k, v = (np.array(c[x]) for x in ("q", "k", "v"))
        o, lse = direct(q, k, v, causal=False)
        s1, s2 = 1000.0 / math.sqrt(2.0), 2000.0 / math.sqrt(2.0)
        w1 = 1.0 / (1.0 + math.exp(s2 - s1))
        fails = []
        for i in range(2):
            if abs(o[i, 0] - w1) > 1e-300 or abs(o[i, 1] - (1.0 - w1)) > 1e-15:
                fails.append(f"overflow row {i} O {o[i]}")
            if abs(lse[i] - s2) > 1e-12:
                fails.append(f"overflow row {i} LSE {lse[i]} != {s2}")
        return fails
    return _catch(run)


# ---------------------------------------------------------------- invariants
def check_invariants(direct: Callable) -> List[str]:
    def run():
        fails = []
        rng = np.random.default_rng(7)
        Sq, Skv, d = 11, 19, 6
        q = rng.standard_normal((Sq, d)) * 3
        k = rng.standard_normal((Skv, d)) * 3
        v = rng.standard_normal((Skv, d))
        o, lse = direct(q, k, v, causal=False)
        # convex hull: every output is a convex combination of V rows
        lo, hi = v.min(axis=0), v.max(axis=0)
        if np.any(o < lo - 1e-12) or np.any(o > hi + 1e-12):
            fails.append("output outside the convex hull of V rows")
        # joint permutation of key/value rows leaves non-causal attention unchanged
        perm = rng.permutation(Skv)
        o2, lse2 = direct(q, k[perm], v[perm], causal=False)
        if np.max(np.abs(o - o2)) > 1e-13 or np.max(np.abs(lse - lse2)) > 1e-12:
            fails.append("joint K/V permutation changed the result")
        # adding u to every key shifts each score of row i by scale*q_i.u
        u = rng.standard_normal(d)
        o3, lse3 = direct(q, k + u, v, causal=False)
        if np.max(np.abs(o - o3)) > 1e-12:
            fails.append("key shift changed O")
        if np.max(np.abs(lse3 - (lse + (q @ u) / math.sqrt(d)))) > 1e-11:
            fails.append("key shift did not shift LSE by scale*q.u")
        # O is linear in V
        w = rng.standard_normal((Skv, d))
        o4, _ = direct(q, k, 2.0 * v - 0.5 * w, causal=False)
        o5, _ = direct(q, k, w, causal=False)
        if np.max(np.abs(o4 - (2.0 * o - 0.5 * o5))) > 1e-12:
            fails.append("O is not linear in V")
        # causal row i equals non-causal attention over the visible prefix
        oc, lc = direct(q, k, v, causal=True)
        for i in range(Sq):
            n = max(0, min(Skv, i + Skv - Sq + 1))
            op, lp = direct(q[i:i + 1], k[:n], v[:n], causal=False)
            if np.max(np.abs(oc[i] - op[0])) > 1e-13 or abs(lc[i] - lp[0]) > 1e-12:
                fails.append(f"causal row {i} differs from prefix attention")
        return fails
    return _catch(run)


def check_empty_rows(direct: Callable) -> List[str]:
    """Rows with no visible key: O = 0 and LSE = -inf, no NaN."""
    def run():
        fails = []
        rng = np.random.default_rng(8)
        q = rng.standard_normal((8, 4))
        k = rng.standard_normal((5, 4))
        v = rng.standard_normal((5, 4))
        o, lse = direct(q, k, v, causal=True)      # rows 0..2 see nothing
        if np.any(np.isnan(o)) or np.any(np.isnan(lse)):
            fails.append("NaN in a causal Sq > Skv result")
        if not (np.all(o[:3] == 0.0) and np.all(lse[:3] == -math.inf)):
            fails.append("masked rows are not O = 0, LSE = -inf")
        if not np.all(np.isfinite(lse[3:])):
            fails.append("visible rows lost their LSE")
        o0, l0 = direct(q, k[:0], v[:0], causal=False)
        if o0.shape != (8, 4) or np.any(o0 != 0.0) or np.any(l0 != -math.inf):
            fails.append("Skv = 0 is not O = 0, LSE = -inf")
        return fails
    return _catch(run)


ALL_DIRECT_CHECKS = [check_worked_example, check_p1_printed, check_library_sdpa,
                     check_zero_queries, check_single_visible_key, check_two_keys,
                     check_overflow_case, check_invariants, check_empty_rows]
