"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module only draws random numbers and arranges them into Q, K, V
tensors of the attention workloads.  It holds none of the attention
arithmetic, imports nothing from ``oracle`` or from the HIP package, and
both sides receive exactly the same host tensors from it.

Workloads (shapes are ``[B, H, S, d]`` row-major, ``d`` fastest, the layout
used by "FlashAttention implemented, verified and measured", section "The
reference implementation, in full"):

* ``single_head_s64_d32`` -- one head, Sq = Skv = 64, d = 32, fp32,
  Q, K, V i.i.d. uniform(-0.8, 0.8) (the distribution of the lab on
  "Verify tiled attention", section "Compare the attention outputs"),
  scale 1/sqrt(d), causal and non-causal, 16 x 16 tiles.
* ``b2h4_s512_d64`` -- B = 2, H = 4, S = 512, d = 64, fp32, standard
  normal, non-causal (the shape of the correctness check of "FlashAttention
  implemented, verified and measured", section "Correctness first"; d = 64
  is our choice where that page is silent), 64-key tiles: the block size of
  that page's tiled function ("The reference implementation, in full") is a
  block of K/V rows taken against every query row, so the queries go in
  16-row blocks, the GPU's own split.
* ``prefill_h32_s4096_d128`` -- B = 1, H = 32, S = 4096, d = 128, causal,
  uniform(-0.8, 0.8) rounded to bf16 (the S = 4096, H = 32, d = 128 row of
  the logical-access sweep on "Verify tiled attention").
* ``longctx_h64_s32768_d128`` -- B = 1, H = 64, S = 32768, d = 128, causal,
  standard normal rounded to bf16.
* ``prefill_h32_s4096_d128_f16``, ``prefill_h32_s4096_d64``,
  ``prefill_h32_s4096_d32`` -- the S = 4096 prefill in fp16, and in bf16 at
  the other 16-bit head dims.
* ``stress_b3h2_d32_skv{64,257,1000,1024}`` and ``stress_b3h2_d32_sq1000`` --
  B = 3, H = 2, d = 32, fp32; Q and K uniform(-0.8, 0.8) times 20 (scores
  of magnitude ~100 and above, the "increase score magnitudes" exercise of
  "Tiled attention: preserving results without a full score matrix"),
  V uniform(-1, 1); Sq = 8 against Skv in {64, 257, 1000, 1024}, plus the
  causal Sq = Skv = 1000 case.

Rounding to bf16 (or fp16, for the fp16 path) is torch's round-to-nearest-even
``.to(torch.bfloat16)`` (``.to(torch.float16)``).
"""
from __future__ import annotations

import dataclasses
import random
from typing import Dict, List, Tuple

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Sq: int
    Skv: int
    d: int
    dtype: str          # storage type of Q, K, V: "f32", "bf16" or "f16"
    dist: str           # "uniform0.8", "normal", "stress"
    seed: int
    causal_modes: Tuple[bool, ...]
    tiles: Tuple[int, int] | None = None   # forced (block_m, block_n), None = selector

    @property
    def elems_q(self) -> int:
        return self.B * self.H * self.Sq * self.d

    @property
    def elems_kv(self) -> int:
        return self.B * self.H * self.Skv * self.d


def _stress(name: str, sq: int, skv: int, seed: int, modes: Tuple[bool, ...]) -> Workload:
    return Workload(name, 3, 2, sq, skv, 32, "f32", "stress", seed, modes)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("single_head_s64_d32", 1, 1, 64, 64, 32, "f32", "uniform0.8", 101,
                 (False, True), (16, 16)),
        Workload("b2h4_s512_d64", 2, 4, 512, 512, 64, "f32", "normal", 202,
                 (False,), (16, 64)),
        Workload("prefill_h32_s4096_d128", 1, 32, 4096, 4096, 128, "bf16", "uniform0.8",
                 303, (True,)),
        Workload("longctx_h64_s32768_d128", 1, 64, 32768, 32768, 128, "bf16", "normal",
                 404, (True,)),
        # the S = 4096, H = 32, d = 128 prefill with fp16 storage (the other
        # 2-byte element the byte model of "Verify tiled attention" assumes)
        Workload("prefill_h32_s4096_d128_f16", 1, 32, 4096, 4096, 128, "f16", "uniform0.8",
                 306, (True,)),
        # the same prefill at the other 16-bit head dims (same FLOP formula,
        # 4 B H Sq Skv d / 2), for their rates
        Workload("prefill_h32_s4096_d64", 1, 32, 4096, 4096, 64, "bf16", "uniform0.8",
                 307, (True,)),
        Workload("prefill_h32_s4096_d32", 1, 32, 4096, 4096, 32, "bf16", "uniform0.8",
                 308, (True,)),
        _stress("stress_b3h2_d32_skv64", 8, 64, 501, (False, True)),
        _stress("stress_b3h2_d32_skv257", 8, 257, 502, (False, True)),
        _stress("stress_b3h2_d32_skv1000", 8, 1000, 503, (False, True)),
        _stress("stress_b3h2_d32_skv1024", 8, 1024, 504, (False, True)),
        _stress("stress_b3h2_d32_sq1000", 1000, 1000, 505, (True,)),
    ]
}


def _uniform(g: torch.Generator, shape, lo: float, hi: float) -> torch.Tensor:
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def make_tensors(w: Workload, seed: int | None = None
                 ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Host (CPU) Q, K, V for workload ``w``: Q is ``[B,H,Sq,d]``, K and V
    ``[B,H,Skv,d]``, contiguous, in the workload's storage dtype.  Draw order
    is Q, then K, then V, from one ``torch.Generator`` seeded with ``seed``
    (default: the workload's own seed)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed if seed is None else seed)
    qs = (w.B, w.H, w.Sq, w.d)
    ks = (w.B, w.H, w.Skv, w.d)
    if w.dist == "uniform0.8":
        q, k, v = _uniform(g, qs, -0.8, 0.8), _uniform(g, ks, -0.8, 0.8), _uniform(g, ks, -0.8, 0.8)
    elif w.dist == "normal":
        q = torch.randn(qs, generator=g, dtype=torch.float32)
        k = torch.randn(ks, generator=g, dtype=torch.float32)
        v = torch.randn(ks, generator=g, dtype=torch.float32)
    elif w.dist == "stress":
        q = _uniform(g, qs, -0.8, 0.8) * 20.0
        k = _uniform(g, ks, -0.8, 0.8) * 20.0
        v = _uniform(g, ks, -1.0, 1.0)
    else:
        raise ValueError(f"unknown distribution {w.dist!r}")
    if w.dtype in ("bf16", "f16"):
        t = torch.bfloat16 if w.dtype == "bf16" else torch.float16
        q, k, v = q.to(t), k.to(t), v.to(t)
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return q.contiguous(), k.contiguous(), v.contiguous()


def random_tensors(B: int, H: int, Sq: int, Skv: int, d: int, dtype: str, dist: str,
                   seed: int) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Ad-hoc shapes (edge cases, sweeps) with the same recipes as ``WORKLOADS``."""
    w = Workload("adhoc", B, H, Sq, Skv, d, dtype, dist, seed, (False, True))
    return make_tensors(w)


def p1_make_qkv(seq_len: int, head_dim: int, seed: int = 42
                ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """The lab generator of "Verify tiled attention" (section "Compare the
    attention outputs"): Python's ``random.Random(seed)``, each element
    uniform(-0.8, 0.8), drawn for all of Q row by row, then K, then V.
    Returned as ``[seq_len, head_dim]`` float64 arrays (the values are the
    Python floats themselves)."""
    rng = random.Random(seed)

    def block() -> List[List[float]]:
        return [[rng.uniform(-0.8, 0.8) for _ in range(head_dim)] for _ in range(seq_len)]

    q = block()
    k = block()
    v = block()
    return (np.array(q, dtype=np.float64), np.array(k, dtype=np.float64),
            np.array(v, dtype=np.float64))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of an fp32 / bf16 / fp16 host tensor to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()
