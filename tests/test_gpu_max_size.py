"""Parity at the longest key range the ABI accepts: one head's K and V each
just under 2 GiB in fp32 (Skv * d * 4 < 2^31 at d = 128), where the kernels'
32-bit byte offsets are at their limit.  Few query rows (a decode after a
maximal key cache), every row checked against the fp64 oracle, unsplit and
split."""
import math

import pytest
import torch

import oracle
from parity import LSE_TOL, O_TOL, compare, gpu_run, log
from seeded_inputs import random_tensors, to_f64

pytestmark = pytest.mark.gpu

SKV_MAX = (2 ** 31 - 1) // (128 * 4)       # 4194303 keys at d = 128


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_longest_key_range(dt):
    Sq, d = 8, 128
    q, k, v = random_tensors(1, 1, Sq, SKV_MAX, d, dt, "uniform0.8", seed=77)
    log(f"max key range {dt}: Skv={SKV_MAX}, K {k.numel() * k.element_size() / 2**30:.3f} GiB")
    rows = list(range(Sq))
    q64, k64, v64 = to_f64(q[0, 0]), to_f64(k[0, 0]), to_f64(v[0, 0])
    for causal in (False, True):
        o_ref, lse_ref = oracle.direct_attention_rows(q64, rows, k64, v64, Sq,
                                                      1.0 / math.sqrt(d), causal)
        for splits in (None, 0):
            o, lse = gpu_run(q, k, v, causal, splits=splits,
                             out_dtype=torch.float32 if dt == "bf16" else None)
            compare(to_f64(o[0, 0]), to_f64(lse[0, 0]), o_ref, lse_ref, O_TOL[dt], LSE_TOL[dt],
                    f"{dt} Skv={SKV_MAX} causal={causal} splits={splits}")
            del o, lse
    del q, k, v, q64, k64, v64
    torch.cuda.empty_cache()
