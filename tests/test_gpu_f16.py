"""GPU parity of the fp16 path (fp16 inputs on the fp16 MFMA, fp32
accumulation, P rounded to fp16) against the fp64 oracle on the same
fp16-rounded inputs, through the C ABI.  The oracle is the direct attention
of "Verify tiled attention" (section "Compare the attention outputs").
Tolerance: O max-abs 2e-3 (derived in ``parity.py``)."""
import math

import numpy as np
import pytest
import torch

from parity import (LSE_TOL, O_TOL, check_full, check_sampled, gpu_run, log, oracle_full,
                    compare, sample_rows)
from seeded_inputs import WORKLOADS, make_tensors, random_tensors

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", [(128, 32), (64, 64), (128, 128), None],
                         ids=["128x32", "64x64", "128x128", "selector"])
def test_f16_ragged_tiles(d, causal, tiles):
    if d == 32 and tiles == (128, 32):
        pytest.skip("d = 32 takes 64- or 128-key tiles only")
    if d != 32 and tiles == (128, 128):
        pytest.skip("128-key tiles are built for d = 32 only")
    q, k, v = random_tensors(1, 3, 300, 333, d, "f16", "uniform0.8", seed=31 + d)
    check_full(q, k, v, causal, tiles=tiles, what=f"f16 300x333 d={d}")
    check_full(q, k, v, causal, tiles=tiles, out_dtype=torch.float32,
               what=f"f16->f32 300x333 d={d}")


def test_f16_every_tile_count():
    # 1 .. 10 key tiles: every trip count and remainder of the tile loop
    for n in range(1, 11):
        for skv in sorted({(n - 1) * 32 + 1, n * 32}):
            q, k, v = random_tensors(1, 2, 70, skv, 128, "f16", "normal", seed=2000 + skv)
            for causal in (False, True):
                check_full(q, k, v, causal, out_dtype=torch.float32, tiles=(128, 32),
                           what=f"f16->f32 70x{skv}")


def test_f16_prefill_h32_s4096_d128_sampled():
    w = WORKLOADS["prefill_h32_s4096_d128_f16"]
    q, k, v = make_tensors(w)
    log("prefill_h32_s4096_d128_f16 causal, selector tiles")
    o, lse = gpu_run(q, k, v, True)
    assert o.dtype == torch.float16
    check_sampled(q, k, v, o, lse, True, [(0, 0), (0, 17), (0, 31)], sample_rows(w.Sq, 16, 8),
                  1.0 / math.sqrt(w.d), O_TOL["f16"], LSE_TOL["f16"], "prefill f16",
                  bf16_out=False)


def test_f16_split_and_edges():
    q, k, v = random_tensors(1, 8, 16, 3000, 128, "f16", "uniform0.8", seed=44)
    for causal in (False, True):
        check_full(q, k, v, causal, splits=0, what=f"f16 split 16x3000 causal={causal}")
    # one visible key: the V row exactly
    q, k, v = random_tensors(1, 2, 40, 40, 64, "f16", "normal", seed=45)
    o, _ = gpu_run(q, k, v, True)
    assert torch.equal(o.cpu()[:, :, 0], v[:, :, 0])
    # no keys
    q, k, v = random_tensors(2, 2, 10, 0, 64, "f16", "normal", seed=46)
    o, lse = gpu_run(q, k, v, False)
    assert torch.all(o == 0) and torch.all(lse == -math.inf)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_batched_heads_16bit(dt):
    # B > 1: heads of different batch entries must not mix
    q, k, v = random_tensors(3, 5, 130, 150, 128, dt, "uniform0.8", seed=81)
    for causal in (False, True):
        check_full(q, k, v, causal, what=f"{dt} B=3 H=5 130x150 causal={causal}")
