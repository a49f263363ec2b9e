"""Work and byte accounting for the attention forward (host-side arithmetic
used by the bench and the tile selector tests; no attention values here).

* FLOPs: ``4 * B * H * Sq * Skv * d`` (one multiply-add per (query, key,
  channel) for QK^T and one for PV), halved for causal attention.
* Compulsory bytes: Q, K, V read once and O, LSE written once.
* The logical-access model of "Verify tiled attention" (section "Compare the
  attention outputs", the access calculator of the lab): with the query-tile
  loop outermost and causal tile skipping, every query tile re-reads the key
  and value rows up to its own end, and no cache reuse is assumed.  The page
  stresses that this counts logical accesses, not measured HBM traffic.
"""
from __future__ import annotations

import math
from typing import Dict


def attention_flops(B: int, H: int, Sq: int, Skv: int, d: int, causal: bool) -> float:
    f = 4.0 * B * H * Sq * Skv * d
    return f / 2.0 if causal else f


def compulsory_bytes(B: int, H: int, Sq: int, Skv: int, d: int, in_bytes: int,
                     out_bytes: int, with_lse: bool = True) -> int:
    """Bytes every implementation must move at least once: Q, K, V read, O
    written, and the fp32 LSE written when requested."""
    per_head = Sq * d * in_bytes + 2 * Skv * d * in_bytes + Sq * d * out_bytes
    if with_lse:
        per_head += 4 * Sq
    return B * H * per_head


def visible_pairs(Sq: int, Skv: int, causal: bool) -> int:
    """Number of (query, key) pairs that enter the softmax for one head, under
    the end-aligned causal rule (row i sees keys j <= i + Skv - Sq)."""
    if not causal:
        return Sq * Skv
    total = 0
    off = Skv - Sq
    # rows with i + off + 1 in [1, Skv] see i + off + 1 keys, rows beyond see all
    for i in range(Sq):
        total += max(0, min(Skv, i + off + 1))
    return total


def tiles_visited(Sq: int, Skv: int, block_q: int, block_kv: int, causal: bool) -> int:
    """(query tile, key tile) pairs an outer-query-tile loop visits when it
    stops at the first key tile no row of the query tile can see."""
    n = 0
    off = Skv - Sq
    for q0 in range(0, Sq, block_q):
        q1 = min(Sq, q0 + block_q)
        last = Skv if not causal else max(0, min(Skv, q1 - 1 + off + 1))
        n += -(-last // block_kv) if last > 0 else 0
    return n


def logical_access_model(seq_len: int, num_heads: int = 32, head_dim: int = 128,
                         bytes_per_elem: int = 2, block_q: int = 128) -> Dict[str, float]:
    """The lab's access calculator on "Verify tiled attention" restated:
    standard attention moves Q, K, V, O once plus writes and reads the N x N
    score matrix and the N x N probability matrix; causal outer-Q tiling reads
    Q and writes O once, and reads every K and V row up to the end of each
    query tile again for that tile.  Values in bytes."""
    S, H, d, b = seq_len, num_heads, head_dim, bytes_per_elem
    qkvo = 4 * H * S * d * b
    nxn = 4 * H * S * S * b
    kv_rows = sum(min(S, start + block_q) for start in range(0, S, block_q))
    tiled = (2 * H * S * d + 2 * H * kv_rows * d) * b
    return {
        "qkvo_bytes": float(qkvo),
        "nxn_matrix_bytes": float(nxn),
        "standard_total_bytes": float(qkvo + nxn),
        "tiled_logical_bytes": float(tiled),
        "num_q_blocks": math.ceil(S / block_q),
    }
