"""GPU parity of the start-aligned causal mask (causal = 2: key j visible to
query i iff j <= i, the "j <= i" rule of "Verify tiled attention", section
"Compare the attention outputs", taken literally when Sq != Skv) against the
oracle's start-aligned reading, for every dtype, some tile shapes and the
split path.  With Sq == Skv it must equal the end-aligned result."""
import pytest
import torch

from parity import check_full, gpu_run
from seeded_inputs import random_tensors
from tiled_online_softmax_05_amd import binding

pytestmark = pytest.mark.gpu
START = binding.CAUSAL_START


@pytest.mark.parametrize("Sq,Skv", [(77, 133), (133, 77), (8, 1000), (1, 300)])
def test_start_aligned_f32(Sq, Skv):
    q, k, v = random_tensors(2, 2, Sq, Skv, 32, "f32", "normal", seed=Sq * 7 + Skv)
    check_full(q, k, v, START, what=f"f32 start {Sq}x{Skv}")
    check_full(q, k, v, START, tiles=(16, 16), what=f"f32 start {Sq}x{Skv} (16,16)")
    check_full(q, k, v, START, splits=0, what=f"f32 start {Sq}x{Skv} split")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("Sq,Skv", [(300, 333), (333, 300), (16, 3000)])
def test_start_aligned_16bit(dt, Sq, Skv):
    q, k, v = random_tensors(1, 4, Sq, Skv, 128, dt, "uniform0.8", seed=Sq + Skv)
    check_full(q, k, v, START, what=f"{dt} start {Sq}x{Skv}")
    check_full(q, k, v, START, tiles=(64, 64), what=f"{dt} start {Sq}x{Skv} (64,64)")
    check_full(q, k, v, START, splits=3, what=f"{dt} start {Sq}x{Skv} split")


def test_start_equals_end_when_square():
    q, k, v = random_tensors(1, 4, 257, 257, 128, "bf16", "normal", seed=3)
    o1, l1 = gpu_run(q, k, v, True)
    o2, l2 = gpu_run(q, k, v, START)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
