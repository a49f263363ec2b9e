"""GPU parity of the 16-bit kernel's running maximum, against the fp64
oracle through the C ABI.

The online normalisation ("Tiled attention: preserving results without a
full score matrix", section "Online normalization") keeps a running maximum
m per query row and rescales l and the accumulator by exp(m_old - m_new)
whenever a key tile raises it.  The 16-bit kernel takes every key tile's row
maxima and moves m lazily: only when a tile's maximum exceeds m by more
than 8 in base-2 units, so that every probability stays at or below 2^8.
The inputs below make the scores of later keys rise or fall by a chosen
amount:

* q and k entries in [0.5, 1) (every score positive), keys from ``jump_at``
  on multiplied by ``factor``;
* with d = 128 and scale 1/sqrt(d), ``factor`` 2 raises those scores by
  about 9 in base 2 (past the slack of 8: m moves once, with a rescale),
  ``factor`` 6 by about 46 (a rescale by 2^-46);
* ``test_rise_at_fp16_limit``: a single later score exactly 15.5, 15.9998
  or 16.5 base-2 units above the first tile's maximum while the other keys
  of its tile sit 16 units below it.  Against the first tile's maximum that
  key's probability would be 2^15.9998 = 65527, which rounds to +inf in
  fp16 (largest finite value 65504): the running maximum must move first.

Tolerances are those of ``parity.py`` (O max-abs 1e-2 bf16, 2e-3 fp16)."""
import math

import pytest
import torch

from parity import check_full, log
from tiled_online_softmax_05_amd import binding

pytestmark = pytest.mark.gpu

TILES = [(128, 32), (64, 64), (256, 32), (128, 64), (64, 32)]
TILE_IDS = ["128x32", "64x64", "256x32", "128x64", "64x32"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def rising(B, H, Sq, Skv, d, factor, jump_at, seed, dtype=torch.bfloat16, rows=None):
    """Seeded inputs whose scores rise at key ``jump_at`` (rows: the query
    rows that get positive entries; the others get entries in [-0.05, 0.05),
    so their scores stay near 0)."""
    g = torch.Generator().manual_seed(seed)
    q = 0.5 + 0.5 * torch.rand(B, H, Sq, d, generator=g)
    if rows is not None:
        small = 0.1 * torch.rand(B, H, Sq, d, generator=g) - 0.05
        keep = torch.zeros(Sq, dtype=torch.bool)
        keep[rows] = True
        q = torch.where(keep[None, None, :, None], q, small)
    k = 0.5 + 0.5 * torch.rand(B, H, Skv, d, generator=g)
    k[:, :, jump_at:] *= factor
    v = 2.0 * torch.rand(B, H, Skv, d, generator=g) - 1.0
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("tiles", TILES, ids=TILE_IDS)
@pytest.mark.parametrize("factor", [2.0, 6.0], ids=["rise9", "rise46"])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores(tiles, factor, causal):
    q, k, v = rising(1, 2, 300, 333, 128, factor, 100, seed=71)
    log(f"rising scores x{factor} causal={causal} tiles={tiles}")
    check_full(q, k, v, causal, tiles=tiles, what=f"rise x{factor} {tiles}")
    check_full(q, k, v, causal, tiles=tiles, out_dtype=torch.float32,
               what=f"rise x{factor} {tiles} ->f32")


@pytest.mark.parametrize("factor", [2.0, 6.0], ids=["rise9", "rise46"])
def test_rising_scores_fp16_d64(factor):
    # d = 64: at the same factor the scores rise less (x2 by about 7 in base
    # 2, x6 by about 32, still far past 2^16)
    q, k, v = rising(2, 2, 200, 260, 64, factor, 70, seed=72, dtype=torch.float16)
    for causal in (False, True):
        log(f"fp16 d=64 rising x{factor} causal={causal}")
        check_full(q, k, v, causal, what=f"fp16 rise x{factor}")


def test_one_wave_rises():
    # only query rows 40..50 (part of one wave of the first query tile) see
    # the rise; every row, risen or not, must match
    q, k, v = rising(1, 1, 256, 256, 128, 6.0, 64, seed=73, rows=list(range(40, 51)))
    for tiles in [(128, 32), (256, 32), (64, 64)]:
        log(f"one wave rises tiles={tiles}")
        check_full(q, k, v, False, tiles=tiles, what=f"one wave {tiles}")


def test_paired_causal_tiles_one_rises():
    # causal, 4 query tiles of 128 rows paired (3, 0) and (2, 1): keys from
    # 300 on rise, so the heavy tiles 2 and 3 move their maximum and the
    # light tiles 0 and 1 of the same workgroups do not
    q, k, v = rising(1, 2, 512, 512, 128, 6.0, 300, seed=74)
    check_full(q, k, v, True, tiles=(128, 32), what="paired causal, heavy tiles rise")


def test_falling_scores():
    # the first key tile holds the largest scores; the maximum never moves
    # after it and later probabilities are tiny
    q, k, v = rising(1, 2, 300, 333, 128, 1.0 / 6.0, 32, seed=75)
    for causal in (False, True):
        check_full(q, k, v, causal, what=f"falling causal={causal}")


@pytest.mark.parametrize("splits", [2, 5])
def test_rising_scores_split(splits):
    # each key chunk runs its own maximum from its own first tile; the
    # chunks past the rise start high, the first one starts low and rises
    q, k, v = rising(1, 2, 40, 1000, 128, 6.0, 150, seed=76)
    for causal in (False, True):
        check_full(q, k, v, causal, splits=splits, what=f"split {splits} rise causal={causal}")


def one_rise(d, delta, jump, dtype, Sq=96, Skv=300, H=2, seed=77):
    """q = e_0 for every row; k[j, 0] = 0 for the keys of the first tiles,
    -64 from key 64 on, and +64 at key ``jump``; the other channels of k
    are random (they meet q's zeros).  With scale = delta / (64 log2 e) the
    key ``jump`` scores exactly ``delta`` base-2 units above the first
    tile's maximum (0), and its tile's other keys ``delta`` units below."""
    g = torch.Generator().manual_seed(seed)
    q = torch.zeros(1, H, Sq, d)
    q[..., 0] = 1.0
    k = 2.0 * torch.rand(1, H, Skv, d, generator=g) - 1.0
    k[..., 0] = 0.0
    k[:, :, 64:, 0] = -64.0
    k[:, :, jump, 0] = 64.0
    v = 2.0 * torch.rand(1, H, Skv, d, generator=g) - 1.0
    scale = delta / (64.0 * math.log2(math.e))
    return q.to(dtype), k.to(dtype), v.to(dtype), scale


@pytest.mark.parametrize("delta", [15.5, 15.9998, 16.5])
@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16], ids=["f16", "bf16"])
@pytest.mark.parametrize("tiles", [None, (64, 64), (64, 32)], ids=["selector", "64x64", "64x32"])
def test_rise_at_fp16_limit(delta, dtype, tiles):
    for d in (32, 64, 128):
        if d == 32 and tiles == (64, 32):
            continue   # d = 32 takes 64- or 128-key tiles only
        q, k, v, scale = one_rise(d, delta, jump=150, dtype=dtype)
        for causal in (False, True):
            log(f"one rise of {delta} (base 2) d={d} {dtype} causal={causal} tiles={tiles}")
            o, lse, o_ref, lse_ref = check_full(q, k, v, causal, scale=scale, tiles=tiles,
                                                what=f"rise {delta} d={d}")
            assert torch.isfinite(o).all() and not torch.isnan(lse).any()
            check_full(q, k, v, causal, scale=scale, tiles=tiles, out_dtype=torch.float32,
                       what=f"rise {delta} d={d} ->f32")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16], ids=["bf16", "f16"])
@pytest.mark.parametrize("scale", [1e-3, 0.02, 1.0, 4.0])
def test_threshold_across_scales(dtype, scale):
    # the running-maximum test compares raw scores with (m + 8) / (scale
    # log2 e): tiny scales make that threshold huge, large ones put many
    # rises in every row; rising scores (x6 from key 150) at d = 64 and 128
    for d in (64, 128):
        q, k, v = rising(1, 2, 96, 300, d, 6.0, 150, seed=81, dtype=dtype)
        for causal in (False, True):
            log(f"threshold scale={scale} d={d} {dtype} causal={causal}")
            o, lse, o_ref, lse_ref = check_full(q, k, v, causal, scale=scale,
                                                out_dtype=torch.float32,
                                                what=f"scale {scale} d={d}")
            assert torch.isfinite(o).all() and torch.isfinite(lse).all()
