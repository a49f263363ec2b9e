"""Plain fp64 CPU attention oracle -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it and it
never calls the HIP library; the two share no code.

Pages cited (by title and section):

* "Verify tiled attention" -- sections "Keep the softmax state between
  tiles", "Compare the attention outputs" (the direct and tiled lab
  functions and their printed results), "Separate storage savings from
  runtime" and "Read the executable checks" (the unit tests).
* "FlashAttention implemented, verified and measured" -- sections "The
  reference implementation, in full" and "Correctness first".
* "Tiled attention: preserving results without a full score matrix" --
  sections "A failing baseline", "Online normalization" and "Recorded
  results".

Everything is computed in float64.  Inputs may be fp32 or bf16 values; both
widen to float64 exactly.

Readings taken where the pages are silent (each is also listed in the design
notes):

* Causal visibility for Sq != Skv is bottom-right aligned by default: query
  row ``i`` sees key ``j`` iff ``j <= i + (Skv - Sq)``.  The pages only use
  Sq == Skv, where this is their ``j <= i`` rule.  ``align="start"`` takes the
  rule literally instead (``j <= i``, top-left aligned) for the other reading.
* A row that sees no key gets O = 0 and LSE = -inf (the online-normalization
  section says such rows need separate handling; it does not say how).
* LSE is the natural log of the sum of exponentials of the *scaled* scores.
* ``scale`` is the caller's; it defaults to 1/sqrt(d) as on every page.

Parity status: every function here is pinned by a ``-m "not gpu"`` test
(worked example, printed lab values, closed forms, library routines,
invariants); none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    return a.astype(np.float64, copy=False)


def last_visible_key(i: int, Sq: int, Skv: int, causal: bool, align: str = "end") -> int:
    """Index one past the last key row ``i`` may attend to.

    Non-causal rows see every key.  Causal rows see keys ``j <= i + Skv - Sq``
    (the ``j <= i`` rule of the direct lab function on "Verify tiled
    attention", section "Compare the attention outputs", aligned to the end of
    the key sequence when Sq != Skv), or ``j <= i`` with ``align="start"``.
    The result is clamped to [0, Skv]."""
    if not causal:
        return Skv
    if align not in ("end", "start"):
        raise ValueError("align is 'end' or 'start'")
    offset = Skv - Sq if align == "end" else 0
    return max(0, min(Skv, i + offset + 1))


def _rows_direct(q_rows: np.ndarray, row_ids: Sequence[int], k: np.ndarray, v: np.ndarray,
                 Sq: int, scale: float, causal: bool, subtract_max: bool, align: str = "end"
                 ) -> Tuple[np.ndarray, np.ndarray, int]:
    """Direct attention for a set of query rows of one head, materialising
    each row's full score vector and probability vector (the three steps of
    the direct lab function on "Verify tiled attention": scores, row softmax,
    probabilities times V)."""
    Skv, d = k.shape
    n_rows = len(row_ids)
    out = np.zeros((n_rows, v.shape[1]), dtype=np.float64)
    lse = np.full((n_rows,), NEG_INF, dtype=np.float64)
    materialised = 0
    if n_rows == 0 or Skv == 0:
        return out, lse, materialised
    # 1. scores s_ij = scale * q_i . k_j for every key (library matmul as one step)
    scores = (q_rows @ k.T) * scale
    for r, i in enumerate(row_ids):
        n = last_visible_key(int(i), Sq, Skv, causal, align)
        if n == 0:
            continue                      # no visible key: O = 0, LSE = -inf
        s = scores[r, :n]
        # 2. row softmax, shifted by the row maximum unless asked not to
        m = s.max() if subtract_max else 0.0
        with np.errstate(over="ignore"):
            e = np.exp(s - m)
        if not np.all(np.isfinite(e)):
            raise OverflowError("exp of an unshifted score overflowed")
        l = e.sum()
        p = e / l
        materialised += 2 * n             # one score vector and one probability vector
        # 3. output row O_i = sum_j p_ij v_j
        out[r] = p @ v[:n]
        lse[r] = m + math.log(l)
    return out, lse, materialised


def direct_attention(q, k, v, scale: float | None = None, causal: bool = False,
                     subtract_max: bool = True, row_chunk: int = 256,
                     return_meta: bool = False, align: str = "end"):
    """Exact scaled-dot-product attention forward, the definition that the
    tiled method reaches up to rounding ("Keep the softmax state between
    tiles" on "Verify tiled attention"; "Correctness first" on
    "FlashAttention implemented, verified and measured").

    ``q`` is ``[..., Sq, d]``, ``k`` and ``v`` are ``[..., Skv, d]`` with the
    same leading dimensions.  For each leading index and row ``i``:
    ``s_ij = scale * q_i . k_j`` over the visible keys, ``m_i = max_j s_ij``,
    ``p_ij = exp(s_ij - m_i)``, ``l_i = sum_j p_ij``, ``O_i = sum_j p_ij v_j / l_i``
    and ``LSE_i = m_i + ln l_i``.  Rows without a visible key give O = 0 and
    LSE = -inf.  ``subtract_max=False`` is the unshifted softmax of the
    overflow check in "Read the executable checks"; it raises
    ``OverflowError`` when an exponential overflows.  ``align`` chooses the
    causal alignment (see ``last_visible_key``).

    Rows are processed in chunks of ``row_chunk`` (full rows each, no running
    state carried between chunks).  Returns ``(O, LSE)`` as float64, plus a
    dict with the number of materialised score and probability elements when
    ``return_meta``."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if q.ndim < 2 or k.ndim != q.ndim or v.shape[:-1] != k.shape[:-1]:
        raise ValueError("expected q [..., Sq, d] and k, v [..., Skv, d]")
    Sq, d = q.shape[-2], q.shape[-1]
    Skv = k.shape[-2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lead = q.shape[:-2]
    n_lead = int(np.prod(lead, dtype=np.int64))
    qf = q.reshape(n_lead, Sq, d)
    kf = k.reshape(n_lead, Skv, d)
    vf = v.reshape(n_lead, Skv, v.shape[-1])
    out = np.zeros(qf.shape[:2] + (v.shape[-1],), dtype=np.float64)
    lse = np.full(qf.shape[:2], NEG_INF, dtype=np.float64)
    materialised = 0
    for h in range(qf.shape[0]):
        for r0 in range(0, Sq, row_chunk):
            rows = list(range(r0, min(Sq, r0 + row_chunk)))
            o_c, l_c, n_c = _rows_direct(qf[h, rows], rows, kf[h], vf[h], Sq, scale,
                                         causal, subtract_max, align)
            out[h, r0:r0 + len(rows)] = o_c
            lse[h, r0:r0 + len(rows)] = l_c
            materialised += n_c
    out = out.reshape(lead + (Sq, v.shape[-1]))
    lse = lse.reshape(lead + (Sq,))
    if return_meta:
        return out, lse, {"materialized_nxn_elements": materialised}
    return out, lse


def direct_attention_rows(q_head, row_ids: Sequence[int], k_head, v_head, Sq: int,
                          scale: float, causal: bool, align: str = "end"
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """Direct attention for selected query rows ``row_ids`` of one head.
    ``q_head`` holds exactly those rows (``[len(row_ids), d]``); ``k_head`` and
    ``v_head`` are the head's full ``[Skv, d]`` keys and values, and ``Sq`` is
    the head's full query length (needed for the causal offset).  Used to check
    sampled outputs at sizes where the whole output would take too long."""
    o, l, _ = _rows_direct(_as_f64(q_head), list(row_ids), _as_f64(k_head), _as_f64(v_head),
                           Sq, scale, causal, True, align)
    return o, l


def online_tiled_attention(q, k, v, block_q: int, block_kv: int, scale: float | None = None,
                           causal: bool = False, rescale_accumulator: bool = True
                           ) -> Tuple[np.ndarray, np.ndarray, Dict[str, int]]:
    """The tiled online-softmax method on one head, in float64 -- used only to
    check the oracle against the pages' own tiled results, never as the
    reference for the GPU.

    The recurrence of "Online normalization" on "Tiled attention: preserving
    results without a full score matrix" (also "Keep the softmax state
    between tiles" on "Verify tiled attention"), written per query tile with
    whole-tile array operations.  Every row of a query tile of ``block_q``
    rows carries a running maximum ``mx`` (initially -inf), a normaliser
    ``den`` and an unnormalised output ``num`` (initially 0).  The key tiles
    of ``block_kv`` rows are taken in order -- for causal attention up to the
    last one any row of the query tile can see -- and each one updates the
    state of every row through its visibility mask:

        tile_max = max over the row's visible keys of the tile's scores
        new_max  = max(mx, tile_max)
        shrink   = exp(mx - new_max)              (0 while mx is -inf)
        w        = exp(scores - new_max) on visible keys, 0 elsewhere
        num      = shrink * num + w @ v_tile
        den      = shrink * den + sum(w)
        mx       = new_max

    Rows with no visible key in a tile keep their state.  At the end
    ``O = num / den`` and ``LSE = mx + ln den``; rows that never saw a key
    give O = 0 and LSE = -inf.  ``rescale_accumulator=False`` is the mistake
    the pages warn about: ``den`` shrinks with the maximum but ``num`` does
    not.

    ``q`` is ``[Sq, d]``, ``k`` and ``v`` ``[Skv, d]``; the causal mask is
    aligned to the end of the keys.  Returns ``(O, LSE, counters)`` with
    ``counters["tiles_visited"]`` the number of (query tile, key tile) pairs
    visited and ``counters["max_score_tile_elements"] = block_q * block_kv``."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Sq, d = q.shape
    Skv = k.shape[0]
    dv = v.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if block_q <= 0 or block_kv <= 0:
        raise ValueError("tile sizes must be positive")
    # one past the last visible key of every query row
    seen = np.array([last_visible_key(i, Sq, Skv, causal) for i in range(Sq)], dtype=np.int64)
    out = np.zeros((Sq, dv), dtype=np.float64)
    lse = np.full((Sq,), NEG_INF, dtype=np.float64)
    pairs = 0
    for lo in range(0, Sq, block_q):
        hi = min(lo + block_q, Sq)
        rows = slice(lo, hi)
        mx = np.full(hi - lo, NEG_INF)
        den = np.zeros(hi - lo)
        num = np.zeros((hi - lo, dv))
        key_end = int(seen[rows].max()) if causal else Skv
        for kl in range(0, key_end, block_kv):
            kh = min(kl + block_kv, Skv)
            pairs += 1
            visible = np.arange(kl, kh)[None, :] < seen[rows, None]          # [rows, keys]
            scores = (q[rows] @ k[kl:kh].T) * scale
            live = visible.any(axis=1)                                       # rows that see a key here
            tile_max = np.where(visible, scores, NEG_INF).max(axis=1)
            new_max = np.where(live, np.maximum(mx, tile_max), mx)
            with np.errstate(invalid="ignore"):
                shrink = np.where(mx > NEG_INF, np.exp(mx - new_max), 0.0)
            shrink = np.where(live, shrink, 1.0)
            w = np.where(visible, np.exp(scores - np.where(live, new_max, 0.0)[:, None]), 0.0)
            num = (shrink[:, None] if rescale_accumulator else 1.0) * num + w @ v[kl:kh]
            den = shrink * den + w.sum(axis=1)
            mx = new_max
        has = den > 0.0
        out[lo:hi][has] = num[has] / den[has, None]
        lse[lo:hi][has] = mx[has] + np.log(den[has])
    return out, lse, {"tiles_visited": pairs,
                      "max_score_tile_elements": block_q * block_kv,
                      "materialized_nxn_elements": 0}


def block_average_attention(q, k, v, block: int, scale: float | None = None) -> np.ndarray:
    """The intentionally wrong baseline of "Tiled attention: preserving
    results without a full score matrix" (section "A failing baseline"): each
    key block is softmax-normalised on its own, the per-block outputs are
    computed, and the block outputs are averaged with equal weight, which
    discards the probability mass each block holds.  Non-causal; ``q`` is
    ``[Sq, d]``, ``k`` and ``v`` ``[Skv, d]``.  Kept so the tests can show the
    oracle tells it apart from attention."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Sq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for k0 in range(0, k.shape[0], block):
        S = (q @ k[k0:k0 + block].T) * scale
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        outs.append(P @ v[k0:k0 + block])
    return np.mean(outs, axis=0)


def max_abs_diff(a, b) -> float:
    """Largest absolute element difference (the comparison used by all three
    pages)."""
    a, b = _as_f64(a), _as_f64(b)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))
