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
                           causal: bool = False, rescale_previous_acc: bool = True
                           ) -> Tuple[np.ndarray, np.ndarray, Dict[str, int]]:
    """The tiled online-softmax method on one head, in float64 -- used only to
    check the oracle against the pages' own tiled results, never as the
    reference for the GPU.

    Follows "Online normalization" on "Tiled attention: preserving results
    without a full score matrix" and the tiled lab function of "Verify tiled
    attention" ("Keep the softmax state between tiles"): queries are split
    into tiles of ``block_q`` rows; each row keeps a running maximum ``m``
    (initially -inf), a denominator ``l`` and an unnormalised accumulator
    ``a`` (initially 0).  Key/value tiles of ``block_kv`` rows are visited in
    order; for causal attention the visit stops at the first key tile that no
    row of the query tile can see.  For each visited tile and each row with at
    least one visible key in it:

        m_new   = max(m, max_j S_j)
        rescale = exp(m - m_new)            (0 while m is still -inf)
        P_j     = exp(S_j - m_new)
        a       = a * rescale + sum_j P_j v_j
        l       = l * rescale + sum_j P_j
        m       = m_new

    and finally ``O = a / l``.  ``rescale_previous_acc=False`` reproduces the
    mistake the pages warn about: ``l`` is rescaled but ``a`` is not.

    ``q`` is ``[Sq, d]``, ``k`` and ``v`` ``[Skv, d]``.  Returns ``(O, LSE,
    meta)`` with ``meta["tiles_visited"]`` the number of (query tile, key
    tile) pairs visited and ``meta["max_score_tile_elements"] = block_q *
    block_kv``."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    Sq, d = q.shape
    Skv = k.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if block_q <= 0 or block_kv <= 0:
        raise ValueError("tile sizes must be positive")
    out = np.zeros((Sq, v.shape[1]), dtype=np.float64)
    lse = np.full((Sq,), NEG_INF, dtype=np.float64)
    tiles_visited = 0
    offset = Skv - Sq
    for q0 in range(0, Sq, block_q):
        q1 = min(q0 + block_q, Sq)
        m = [NEG_INF] * (q1 - q0)
        l = [0.0] * (q1 - q0)
        a = np.zeros((q1 - q0, v.shape[1]), dtype=np.float64)
        for k0 in range(0, Skv, block_kv):
            # causal: the tile's last row sees keys up to (q1 - 1) + offset
            if causal and k0 > (q1 - 1) + offset:
                break
            k1 = min(k0 + block_kv, Skv)
            tiles_visited += 1
            for r in range(q1 - q0):
                i = q0 + r
                n = last_visible_key(i, Sq, Skv, causal)
                cols = range(k0, min(k1, n))
                if len(cols) == 0:
                    continue
                S = (k[k0:k0 + len(cols)] @ q[i]) * scale
                m_new = max(m[r], float(S.max()))
                rescale = math.exp(m[r] - m_new) if m[r] > NEG_INF else 0.0
                P = np.exp(S - m_new)
                acc_scale = rescale if rescale_previous_acc else 1.0
                a[r] = a[r] * acc_scale + P @ v[k0:k0 + len(cols)]
                l[r] = l[r] * rescale + float(P.sum())
                m[r] = m_new
        for r in range(q1 - q0):
            if l[r] > 0.0:
                out[q0 + r] = a[r] / l[r]
                lse[q0 + r] = m[r] + math.log(l[r])
    return out, lse, {"tiles_visited": tiles_visited,
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
