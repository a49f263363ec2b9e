"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
the same seeded host inputs.  Tolerances: O max-abs 1e-5 (fp32 inputs) and
1e-2 (bf16 inputs); LSE as documented in ``parity.py``."""
import math

import numpy as np
import pytest
import torch

import oracle
from parity import (LSE_TOL, O_TOL, bf16_half_ulp, check_full, check_sampled, compare, gpu_run,
                    log, oracle_full, sample_rows)
from seeded_inputs import WORKLOADS, make_tensors, random_tensors, to_f64
from tiled_online_softmax_05_amd import binding

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    binding.load()


# ------------------------------------------------------------------ configs 1, 2, 5 (fp32)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", [(16, 16), None], ids=["tiles16x16", "selector"])
def test_single_head_s64_d32(causal, tiles):
    w = WORKLOADS["single_head_s64_d32"]
    q, k, v = make_tensors(w)
    log(f"single_head_s64_d32 causal={causal} tiles={tiles}")
    check_full(q, k, v, causal, tiles=tiles, what="single_head_s64_d32")


@pytest.mark.parametrize("tiles", [(16, 64), (64, 64), None],
                         ids=["tiles16x64", "tiles64x64", "selector"])
def test_b2h4_s512_d64(tiles):
    w = WORKLOADS["b2h4_s512_d64"]
    q, k, v = make_tensors(w)
    log(f"b2h4_s512_d64 non-causal tiles={tiles}")
    check_full(q, k, v, False, tiles=tiles, what="b2h4_s512_d64")


STRESS = [n for n in WORKLOADS if n.startswith("stress_")]


@pytest.mark.parametrize("name", STRESS)
@pytest.mark.parametrize("causal", [False, True])
def test_stress_fp32(name, causal):
    w = WORKLOADS[name]
    if causal not in w.causal_modes:
        pytest.skip("mode not part of this workload")
    q, k, v = make_tensors(w)
    log(f"{name} causal={causal}")
    check_full(q, k, v, causal, what=name)
    # the same inputs through every fp32 tile shape with a 64-key tile
    for bm in (16, 32, 64):
        check_full(q, k, v, causal, tiles=(bm, 64), what=f"{name} tiles ({bm},64)")


# ------------------------------------------------------------------ config 3 (bf16, full size)
@pytest.fixture(scope="module")
def prefill():
    w = WORKLOADS["prefill_h32_s4096_d128"]
    q, k, v = make_tensors(w)
    return w, q, k, v


def test_prefill_h32_s4096_d128_full(prefill):
    """The benchmarked launch (selector tiles, bf16 output) against the fp64
    oracle on every element of O and LSE: all 32 heads x 4096 rows."""
    w, q, k, v = prefill
    log("prefill_h32_s4096_d128 causal, selector tiles (the benchmarked launch), whole output")
    o, lse = gpu_run(q, k, v, True)
    o_ref, lse_ref = oracle_full(q, k, v, True)
    compare(o, lse, o_ref, lse_ref, O_TOL["bf16"], LSE_TOL["bf16"], "prefill_h32_s4096_d128")


@pytest.mark.parametrize("name", ["prefill_h32_s4096_d64", "prefill_h32_s4096_d32"])
def test_prefill_other_head_dims_full(name):
    """The S = 4096 causal prefill at d = 64 and 32 (selector tiles, bf16
    output), every element against the fp64 oracle."""
    w = WORKLOADS[name]
    q, k, v = make_tensors(w)
    log(f"{name} causal, selector tiles, whole output")
    o, lse = gpu_run(q, k, v, True)
    o_ref, lse_ref = oracle_full(q, k, v, True)
    compare(o, lse, o_ref, lse_ref, O_TOL["bf16"], LSE_TOL["bf16"], name)


def test_prefill_determinism(prefill):
    w, q, k, v = prefill
    o1, l1 = gpu_run(q, k, v, True)
    o2, l2 = gpu_run(q, k, v, True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prefill_zero_queries_closed_form():
    """Q = 0 makes every visible weight equal: causal row i is the mean of
    V rows 0..i and LSE_i = ln(i + 1), at the full S = 4096, H = 32 shape
    (exercises every mask and tile boundary)."""
    w = WORKLOADS["prefill_h32_s4096_d128"]
    _, k, v = make_tensors(w)
    q = torch.zeros_like(k)
    o, lse = gpu_run(q, k, v, True)
    vf = to_f64(v)[0]                                    # [H, S, d]
    ref = np.cumsum(vf, axis=1) / np.arange(1, w.Skv + 1)[None, :, None]
    err = float(np.abs(to_f64(o)[0] - ref).max())
    log(f"  zero-Q prefix means: max|dO| = {err:.3e}")
    assert err < O_TOL["bf16"]
    lerr = float(np.abs(to_f64(lse)[0] - np.log(np.arange(1, w.Skv + 1))[None, :]).max())
    assert lerr < 1e-4 * math.log(w.Skv)


# ------------------------------------------------------------------ config 4 (bf16, full size)
@pytest.fixture(scope="module")
def longctx():
    w = WORKLOADS["longctx_h64_s32768_d128"]
    q, k, v = make_tensors(w)
    return w, q, k, v


def test_longctx_h64_s32768_d128(longctx):
    """Both output dtypes against the fp64 oracle: every element of 8 whole
    heads, one on each XCD under the XCD-major workgroup order (heads 0, 8,
    ..., 56), and sampled rows of the other 56 heads.  Gated at 1e-2 with an
    fp32 output; with a bf16 output the stored O carries bf16's own rounding
    (half an ulp, up to 1.6e-2 where |O| >= 4), which is allowed on top of
    the 1e-2."""
    w, q, k, v = longctx
    scale = 1.0 / math.sqrt(w.d)
    outs = {}
    for out_dtype in (torch.float32, torch.bfloat16):
        log(f"longctx_h64_s32768_d128 causal out={out_dtype}")
        o, lse = gpu_run(q, k, v, True, out_dtype=out_dtype)
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()
        outs[out_dtype] = (o.cpu(), lse.cpu())
        del o, lse
        torch.cuda.empty_cache()
    for h in range(0, w.H, 8):
        log(f"  whole head {h}")
        o_ref, lse_ref = oracle.direct_attention(to_f64(q[0, h]), to_f64(k[0, h]), to_f64(v[0, h]),
                                                 scale=scale, causal=True)
        for out_dtype, (o, lse) in outs.items():
            bf16_out = out_dtype == torch.bfloat16
            compare(to_f64(o[0, h]), to_f64(lse[0, h]), o_ref, lse_ref, O_TOL["bf16"],
                    LSE_TOL["bf16"], f"longctx head {h} out={out_dtype}",
                    bf16_half_ulp(o_ref) if bf16_out else None)
    rows = sample_rows(w.Sq, 16, seed=4)
    others = [(0, h) for h in range(w.H) if h % 8]
    for out_dtype, (o, lse) in outs.items():
        check_sampled(q, k, v, o, lse, True, others, rows, scale, O_TOL["bf16"],
                      LSE_TOL["bf16"], f"longctx sampled out={out_dtype}",
                      bf16_out=(out_dtype == torch.bfloat16))


# ------------------------------------------------------------------ other full-size 16-bit shapes
@pytest.mark.parametrize("B_,H,Sq,Skv,d,causal,dist", [
    (1, 32, 4096, 4096, 64, True, "normal"),          # d = 64 at the headline size
    (1, 16, 4096, 4096, 128, False, "uniform0.8"),    # non-causal, every key tile of every row
    (2, 8, 1024, 8192, 128, True, "normal"),          # prefill after a key cache (end-aligned)
], ids=["d64_causal_s4096", "d128_noncausal_s4096", "sq1024_skv8192_causal"])
def test_bf16_full_size_sampled(B_, H, Sq, Skv, d, causal, dist):
    q, k, v = random_tensors(B_, H, Sq, Skv, d, "bf16", dist, seed=Sq + Skv + d)
    log(f"bf16 full size B={B_} H={H} Sq={Sq} Skv={Skv} d={d} causal={causal} {dist}")
    o, lse = gpu_run(q, k, v, causal, out_dtype=torch.float32)
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    heads = [(0, 0), (B_ - 1, H // 2), (B_ - 1, H - 1)]
    rows = sample_rows(Sq, 12, seed=d + H)
    check_sampled(q, k, v, o, lse, causal, heads, rows, 1.0 / math.sqrt(d), O_TOL["bf16"],
                  LSE_TOL["bf16"], f"bf16 {B_}x{H}x{Sq}x{Skv} d={d}", bf16_out=False)


# ------------------------------------------------------------------ smaller bf16 shapes, whole output
@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("tiles", [(256, 32), (128, 128), (128, 64), (128, 32), (64, 64), (64, 32),
                                   None],
                         ids=["256x32", "128x128", "128x64", "128x32", "64x64", "64x32", "selector"])
def test_bf16_ragged_tiles(d, causal, tiles):
    if tiles == (256, 32) and d != 128:
        pytest.skip("256-row tiles are built for d = 128 only")
    if tiles == (128, 128) and d != 32:
        pytest.skip("128-key tiles are built for d = 32 only")
    if d == 32 and tiles is not None and tiles[1] == 32:
        pytest.skip("d = 32 takes 64- or 128-key tiles only")
    q, k, v = random_tensors(1, 3, 300, 333, d, "bf16", "uniform0.8", seed=17 + d)
    log(f"bf16 ragged d={d} causal={causal} tiles={tiles}")
    check_full(q, k, v, causal, tiles=tiles, what=f"bf16 300x333 d={d}")
    check_full(q, k, v, causal, tiles=tiles, out_dtype=torch.float32,
               what=f"bf16->f32 300x333 d={d}")


@pytest.mark.parametrize("d,tiles", [(128, (128, 32)), (128, (64, 64)), (128, (256, 32)),
                                     (64, (128, 64)), (32, (128, 128)), (32, (128, 64)),
                                     (32, (64, 64))],
                         ids=["d128-128x32", "d128-64x64", "d128-256x32", "d64-128x64",
                              "d32-128x128", "d32-128x64", "d32-64x64"])
def test_bf16_every_tile_count(d, tiles):
    # key lengths giving 1 .. 10 key tiles, full and ragged, so that every
    # entry and exit of the pipelined tile loop runs: no next tile, the
    # four-step unrolled loop run zero, one or two times, and every remainder
    # of zero to three steps after it
    bn = tiles[1]
    for n in range(1, 11):
        for skv in sorted({(n - 1) * bn + 1, n * bn}):
            q, k, v = random_tensors(1, 2, 70, skv, d, "bf16", "normal", seed=1000 + skv)
            log(f"bf16 tile count {n} Skv={skv} tiles={tiles}")
            for causal in (False, True):
                check_full(q, k, v, causal, tiles=tiles, what=f"bf16 70x{skv} {tiles}")


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_ragged_all_tiles(d, causal):
    q, k, v = random_tensors(2, 2, 77, 133, d, "f32", "normal", seed=23 + d)
    log(f"fp32 ragged d={d} causal={causal}")
    for bm in (16, 32, 64):
        for bn in (16, 32, 64):
            check_full(q, k, v, causal, tiles=(bm, bn), what=f"fp32 77x133 d={d} ({bm},{bn})")
    # 128-key tiles (16-row query blocks only): eight key waves, four at d = 128
    check_full(q, k, v, causal, tiles=(16, 128), what=f"fp32 77x133 d={d} (16,128)")


@pytest.mark.parametrize("heads,kw", [(32, 2), (64, 1)], ids=["2 key waves", "1 key wave"])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_key_waves_follow_the_grid(heads, kw, causal):
    # forced 16 x 64 tiles on 17 query tiles per head: 544 query tiles give
    # two waves per query block (each taking half of every key tile), 1088
    # give one; small grids (above) give four
    q, k, v = random_tensors(1, heads, 17 * 16 - 5, 200, 32, "f32", "normal", seed=31 + heads)
    log(f"fp32 {heads} heads, {kw} key waves, causal={causal}")
    check_full(q, k, v, causal, tiles=(16, 64), what=f"fp32 {heads} heads 16x64 kw={kw}")


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_empty_keys(dt):
    d = 64
    q, k, v = random_tensors(2, 2, 10, 0, d, dt, "normal", seed=1)
    o, lse = gpu_run(q, k, v, False)
    assert torch.all(o == 0) and torch.all(lse == -math.inf)
    o, lse = gpu_run(q, k, v, True)
    assert torch.all(o == 0) and torch.all(lse == -math.inf)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_empty_queries_is_a_no_op(dt):
    q, k, v = random_tensors(1, 2, 0, 16, 64, dt, "normal", seed=2)
    o, lse = gpu_run(q, k, v, True)
    assert o.shape == (1, 2, 0, 64) and lse.shape == (1, 2, 0)


@pytest.mark.parametrize("dt,d", [("f32", 32), ("bf16", 128)])
def test_causal_more_queries_than_keys(dt, d):
    """Causal Sq > Skv: the first Sq - Skv rows see no key (O = 0, LSE = -inf)."""
    q, k, v = random_tensors(2, 3, 150, 40, d, dt, "normal", seed=5)
    o, lse, o_ref, lse_ref = check_full(q, k, v, True, what=f"{dt} Sq=150 Skv=40 causal")
    assert torch.all(o[:, :, :110] == 0) and torch.all(lse[:, :, :110] == -math.inf)


@pytest.mark.parametrize("dt,d", [("f32", 32), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_single_visible_key_is_exact(dt, d):
    """Causal row 0 (Sq == Skv) sees one key: its weight is exactly 1, so
    O_0 equals V_0 bit for bit."""
    q, k, v = random_tensors(1, 4, 130, 130, d, dt, "normal", seed=6)
    o, lse = gpu_run(q, k, v, True)
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_single_query_row():
    for dt, d in (("f32", 64), ("bf16", 128)):
        q, k, v = random_tensors(2, 2, 1, 500, d, dt, "normal", seed=7)
        check_full(q, k, v, False, what=f"{dt} Sq=1")
        check_full(q, k, v, True, what=f"{dt} Sq=1 causal")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_worked_example_on_gpu(dt):
    """Scores 0, 10, 20 over values 1, 3, 5 ("A failing baseline" on "Tiled
    attention: preserving results without a full score matrix"), embedded at
    d = 32 (f32) / 64 (bf16) with zero padding, scale 1."""
    d = 32 if dt == "f32" else 64
    q = torch.zeros(1, 1, 1, d)
    k = torch.zeros(1, 1, 3, d)
    v = torch.zeros(1, 1, 3, d)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor([0.0, 10.0, 20.0])
    v[0, 0, :, 0] = torch.tensor([1.0, 3.0, 5.0])
    if dt == "bf16":
        q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    o, lse = gpu_run(q, k, v, False, scale=1.0, out_dtype=torch.float32)
    full = (1.0 + 3.0 * math.exp(10) + 5.0 * math.exp(20)) / (1.0 + math.exp(10) + math.exp(20))
    assert abs(float(o[0, 0, 0, 0]) - full) < O_TOL[dt]
    assert abs(float(lse[0, 0, 0]) - math.log(1 + math.exp(10) + math.exp(20))) < 1e-5 * 20
    assert torch.all(o[0, 0, 0, 1:] == 0)


def test_scale_is_honoured():
    q, k, v = random_tensors(1, 2, 64, 96, 64, "f32", "normal", seed=9)
    check_full(q, k, v, False, scale=0.37, what="fp32 scale 0.37")
    q, k, v = random_tensors(1, 2, 64, 96, 64, "bf16", "normal", seed=9)
    check_full(q, k, v, True, scale=0.05, what="bf16 scale 0.05")


def test_runs_on_the_callers_stream():
    q, k, v = random_tensors(1, 4, 256, 256, 128, "bf16", "uniform0.8", seed=10)
    dev = torch.device("cuda", 0)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        o, lse = binding.fwd(qd, kd, vd, causal=True)
    s.synchronize()
    o_ref, lse_ref = oracle_full(q, k, v, True)
    compare(o, lse, o_ref, lse_ref, O_TOL["bf16"], LSE_TOL["bf16"], "side stream")


def test_no_lse_pointer():
    q, k, v = random_tensors(1, 2, 100, 100, 128, "bf16", "normal", seed=11)
    dev = torch.device("cuda", 0)
    o, lse = binding.fwd(q.to(dev), k.to(dev), v.to(dev), causal=True, with_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    o_ref, _ = oracle_full(q, k, v, True)
    compare(o, None, o_ref, None, O_TOL["bf16"], 0, "no LSE")


# ------------------------------------------------------------------ the pages' pinned example on the GPU
def test_p1_pinned_example_d16_on_gpu():
    # "Verify tiled attention" (section "Compare the attention outputs"): the
    # lab's seed-42 example, S = 64, d = 16, causal, scale 1/4, 16 x 16 tiles,
    # with the printed sample rows (6 decimals) -- here on the GPU in fp32
    from pin_checks import golden
    from seeded_inputs import p1_make_qkv
    g = golden("p1_lab_results.json")
    st = g["setup"]
    qn, kn, vn = p1_make_qkv(st["seq_len"], st["head_dim"], st["seed"])
    q, k, v = [torch.from_numpy(x).to(torch.float32).reshape(1, 1, 64, 16) for x in (qn, kn, vn)]
    scale = 1.0 / math.sqrt(st["head_dim"])
    for tiles in ((st["block_q"], st["block_kv"]), None):
        o, lse = gpu_run(q, k, v, True, scale=scale, tiles=tiles)
        o_ref, lse_ref = oracle.direct_attention(to_f64(q), to_f64(k), to_f64(v), scale=scale,
                                                 causal=True)
        compare(o, lse, o_ref, lse_ref, O_TOL["f32"], LSE_TOL["f32"], f"P1 seed 42 d=16 {tiles}")
        oc = o.cpu().double().numpy()[0, 0]
        # row 0 sees one key: exactly V[0]
        assert np.array_equal(o.cpu()[0, 0, 0], v[0, 0, 0])
        # printed rows, rounded to 6 decimals, from fp64 inputs (fp32 here: ~1e-7 more)
        pr = g["printed"]
        assert np.max(np.abs(oc[0, :4] - pr["sample_row0_first4"])) <= 5e-7 + 1e-6
        assert np.max(np.abs(oc[63, :4] - pr["sample_last_row_first4"])) <= 5e-7 + 1e-6


@pytest.mark.parametrize("Sq,Skv", [(1000, 1000), (1008, 700), (700, 1300)])
@pytest.mark.parametrize("causal", [True, 2], ids=["end", "start"])
def test_fp32_paired_causal_tiles(Sq, Skv, causal):
    # causal fp32 grids with more query tiles than compute units run two
    # query tiles per workgroup (heavy, then light); odd and even tile
    # counts, both mask alignments, the split path on top
    q, k, v = random_tensors(2, 3, Sq, Skv, 64, "f32", "normal", seed=Sq + Skv)
    log(f"fp32 paired causal={causal} {Sq}x{Skv}")
    check_full(q, k, v, causal, what=f"fp32 paired {Sq}x{Skv} causal={causal}")
    check_full(q, k, v, causal, splits=3, what=f"fp32 paired split {Sq}x{Skv} causal={causal}")
