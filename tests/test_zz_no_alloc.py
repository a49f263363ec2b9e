"""attn_fwd_split_noalloc (the split path on the library's static scratch)
against attn_fwd_split (the split path on a workspace the caller allocates):
same chunk plan and kernels, so O and LSE must agree bit for bit.  Each case
makes two calls in a row on the shared scratch, the second with a smaller
problem, so a second call that read the first call's partial states would
show.  One case fills the scratch to its last bytes."""
import pytest
import torch

from parity import check_full, log
from seeded_inputs import random_tensors
from tiled_online_softmax_05_amd import binding

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def _pair(q, k, v, causal, splits, out_dtype=None):
    """(O, LSE) of attn_fwd_split_noalloc and of attn_fwd_split, both on
    output buffers allocated here beforehand."""
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    res = []
    for noalloc in (True, False):
        odt = out_dtype or q.dtype
        out = torch.full(q.shape, float("nan"), dtype=odt, device=DEV)
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
        binding.fwd(q, k, v, causal=causal, out_dtype=out_dtype, out=out, lse=lse,
                    splits=splits, noalloc=noalloc)
        torch.cuda.synchronize()
        res.append((out, lse))
    return res


def _same(a, b, what):
    (o1, l1), (o2, l2) = a, b
    assert torch.isfinite(o1).all(), what
    assert torch.equal(o1, o2), f"{what}: O differs (max {(o1.float() - o2.float()).abs().max()})"
    assert torch.equal(l1, l2), f"{what}: LSE differs"


@pytest.mark.parametrize("dt,d", [("bf16", 128), ("f16", 64), ("f32", 32)])
@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_split_twice(dt, d, causal):
    # first call: 8 heads x 100 queries against 3000 keys in 8 chunks
    big = random_tensors(1, 8, 100, 3000, d, dt, "uniform0.8", seed=500 + d)
    # second call, smaller: 2 heads x 16 queries, 777 keys, 3 chunks
    small = random_tensors(1, 2, 16, 777, d, dt, "normal", seed=600 + d)
    for (q, k, v), n, what in ((big, 8, "first, 8x100x3000"), (small, 3, "second, 2x16x777")):
        log(f"noalloc {dt} d={d} causal={causal} {what} splits={n}")
        a, b = _pair(q, k, v, causal, n)
        _same(a, b, f"{dt} d={d} causal={causal} {what}")
    # the second, smaller call also against the oracle
    check_full(*small, causal, splits=3, what=f"split reference {dt} d={d}")


def test_noalloc_automatic_chunks_and_fp32_output():
    q, k, v = random_tensors(1, 4, 1, 4000, 128, "bf16", "normal", seed=71)
    log("noalloc decode 4 heads x 1 query x 4000 keys, automatic chunks")
    for out_dtype in (None, torch.float32):
        a, b = _pair(q, k, v, True, 0, out_dtype=out_dtype)
        _same(a, b, f"automatic chunks out={out_dtype}")


def test_noalloc_fills_the_scratch_then_a_smaller_call():
    # 16 heads x 125 queries (2000 rows) x 64 chunks of 64 keys at d = 128:
    # 64 * 2000 * (512 + 8) bytes, within 1 % of the static scratch
    need = binding.split_workspace_bytes(1, 16, 125, 128, 64)
    assert 0.99 * binding.NOALLOC_SCRATCH_BYTES < need <= binding.NOALLOC_SCRATCH_BYTES
    q, k, v = random_tensors(1, 16, 125, 4096, 128, "bf16", "uniform0.8", seed=72)
    log(f"noalloc near-full scratch: {need} bytes")
    a, b = _pair(q, k, v, False, 64)
    _same(a, b, "near-full scratch")
    q, k, v = random_tensors(1, 1, 40, 500, 128, "bf16", "uniform0.8", seed=73)
    log("noalloc after the near-full call: 1x40x500, 4 chunks")
    a, b = _pair(q, k, v, False, 4)
    _same(a, b, "smaller call after the near-full one")


def test_noalloc_refuses_beyond_the_scratch_and_enqueues_nothing():
    q, k, v = random_tensors(1, 64, 256, 4096, 128, "bf16", "uniform0.8", seed=74)
    q, k, v = q.to(DEV), k.to(DEV), v.to(DEV)
    out = torch.zeros(q.shape, dtype=q.dtype, device=DEV)
    with pytest.raises(binding.AttnError, match="scratch"):
        binding.fwd(q, k, v, causal=False, out=out, splits=16, noalloc=True)
    torch.cuda.synchronize()
    assert not out.any()
