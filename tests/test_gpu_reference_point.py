"""GPU parity of the 16-bit kernel's choice of reference point, against the
fp64 oracle through the C ABI.

The online normalisation ("Tiled attention: preserving results without a
full score matrix", section "Online normalization") gives the same O and LSE
for any reference point that keeps the exponentials in range.  The 16-bit
kernel takes the reference from a query tile's first key tile and keeps it
for the later tiles; a query tile whose later scores rise so far above it
that a lane's per-tile sum of probabilities passes 2^16 is computed again
with every row's maximum taken first.  The inputs below make the scores of
later keys rise by a chosen amount:

* q and k entries in [0.5, 1) (every score positive), keys from ``jump_at``
  on multiplied by ``factor``;
* with d = 128 and scale 1/sqrt(d), ``factor`` 2 raises those scores by
  about 9 in base 2 (probabilities up to ~2^9 against the first tile's
  reference, accepted), ``factor`` 6 by about 46 (far past 2^16: the query
  tile runs again with its maxima preset).

Tolerances are those of ``parity.py`` (O max-abs 1e-2 bf16, 2e-3 fp16)."""
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
    # only query rows 40..50 (one wave of the first 128-row tile) see the
    # rise; the workgroup computes the whole tile again, and every row, risen
    # or not, must match
    q, k, v = rising(1, 1, 256, 256, 128, 6.0, 64, seed=73, rows=list(range(40, 51)))
    for tiles in [(128, 32), (256, 32), (64, 64)]:
        log(f"one wave rises tiles={tiles}")
        check_full(q, k, v, False, tiles=tiles, what=f"one wave {tiles}")


def test_paired_causal_tiles_one_rises():
    # causal, 4 query tiles of 128 rows paired (3, 0) and (2, 1): keys from
    # 300 on rise, so query tiles 2 and 3 run again and tiles 0 and 1 do
    # not, within the same workgroups
    q, k, v = rising(1, 2, 512, 512, 128, 6.0, 300, seed=74)
    check_full(q, k, v, True, tiles=(128, 32), what="paired causal, heavy tiles rise")


def test_falling_scores():
    # the first key tile holds the largest scores; later probabilities are
    # tiny against its reference
    q, k, v = rising(1, 2, 300, 333, 128, 1.0 / 6.0, 32, seed=75)
    for causal in (False, True):
        check_full(q, k, v, causal, what=f"falling causal={causal}")


@pytest.mark.parametrize("splits", [2, 5])
def test_rising_scores_split(splits):
    # each key chunk picks its own reference from its own first tile; the
    # chunks past the rise start high, the first one starts low and rises
    q, k, v = rising(1, 2, 40, 1000, 128, 6.0, 150, seed=76)
    for causal in (False, True):
        check_full(q, k, v, causal, splits=splits, what=f"split {splits} rise causal={causal}")
