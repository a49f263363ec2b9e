"""The entry points under HIP graph capture: attn_fwd and
attn_fwd_split_noalloc (the allocation-free split path, made for callers that
capture) recorded into one graph through torch's capture stream, replayed
several times with eager work and synchronisations between the replays, and
every replay compared bit for bit with the eager result of the same call."""
import pytest
import torch

from parity import log
from seeded_inputs import random_tensors
from tiled_online_softmax_05_amd import binding

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


def test_capture_and_replay_fwd_and_noalloc_split():
    # a prefill-like call and a decode-like split call (4 heads x 1 query
    # against 4000 keys, automatic chunk count)
    qa, ka, va = (t.to(DEV) for t in random_tensors(1, 4, 300, 333, 128, "bf16", "uniform0.8",
                                                    seed=91))
    qb, kb, vb = (t.to(DEV) for t in random_tensors(1, 4, 1, 4000, 128, "bf16", "normal",
                                                    seed=92))
    oa = torch.empty_like(qa)
    la = torch.empty(qa.shape[:3], dtype=torch.float32, device=DEV)
    ob = torch.empty(qb.shape, dtype=torch.float32, device=DEV)
    lb = torch.empty(qb.shape[:3], dtype=torch.float32, device=DEV)

    def calls():
        binding.fwd(qa, ka, va, causal=True, out=oa, lse=la)
        binding.fwd(qb, kb, vb, causal=True, out_dtype=torch.float32, out=ob, lse=lb,
                    splits=0, noalloc=True)

    # eager reference (also finds the static scratch's address on this
    # device before capture)
    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (oa, la, ob, lb)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    torch.cuda.synchronize()

    for rep in range(4):
        for t in (oa, la, ob, lb):
            t.fill_(float("nan"))
        # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        for name, got, want in zip(("O", "LSE", "O split", "LSE split"), (oa, la, ob, lb), ref):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
