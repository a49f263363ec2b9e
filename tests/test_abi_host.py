"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, the selector is a pure host function, and every invalid
argument is rejected on the host before any HIP call."""
import ctypes
import os
import re

import pytest

from tiled_online_softmax_05_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:long\s+long|\w+)\**\s+\**(attn_\w+)\s*\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        pytest.fail("libattn.so is not built; run python -m tiled_online_softmax_05_amd.build")
    return B.load()


def test_header_declares_the_binding_surface():
    assert _declared_functions() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version(lib):
    assert lib.attn_version() == 102


@pytest.mark.parametrize("args,want", [
    # (d, Sq, Skv, BH, dtype, causal) -> (block_m, block_n, waves)
    # fp32: 16-row query tiles (chosen only while 32-row ones would leave CUs
    # idle, so fewer than 512 of them) with four waves splitting each 64-key
    # tile, or eight splitting each 128-key tile over more than 128 keys at
    # d <= 64; 16-key tiles cannot split
    ((32, 64, 64, 1, B.F32, 1), (16, 64, 4)),
    ((64, 512, 512, 8, B.F32, 0), (16, 128, 8)),
    ((32, 8, 1000, 6, B.F32, 1), (16, 128, 8)),
    ((32, 8, 129, 6, B.F32, 1), (16, 128, 8)),
    ((32, 8, 128, 6, B.F32, 1), (16, 64, 4)),
    ((128, 8, 1000, 6, B.F32, 0), (16, 64, 4)),        # d = 128 keeps 64-key tiles
    ((32, 8, 16, 6, B.F32, 0), (16, 16, 1)),
    ((64, 2048, 2048, 8, B.F32, 0), (64, 64, 4)),       # four query waves, no key split
    ((128, 4096, 4096, 32, B.BF16, 1), (128, 32, 4)),
    ((128, 32768, 32768, 64, B.BF16, 1), (128, 32, 4)),
    ((128, 256, 256, 2, B.BF16, 1), (64, 32, 2)),
    ((64, 4096, 4096, 32, B.BF16_OUT_F32, 0), (128, 64, 4)),   # d = 64: 64-key tiles
    ((64, 1024, 1024, 8, B.BF16, 1), (64, 32, 2)),              # ... but 32-key at 64 rows
    ((128, 4096, 4096, 16, B.BF16, 1), (128, 32, 4)),
    ((128, 1024, 1024, 2, B.BF16, 1), (64, 32, 2)),
    ((32, 4096, 4096, 32, B.BF16, 1), (128, 128, 4)),   # d = 32: 128-key tiles
    ((32, 1024, 1024, 8, B.BF16, 1), (64, 64, 2)),      # ... 64-key at 64 rows
    ((32, 512, 512, 2, B.F16, 0), (64, 64, 2)),
    ((128, 4096, 4096, 32, B.F16, 1), (128, 32, 4)),
    ((64, 4096, 4096, 32, B.F16_OUT_F32, 0), (128, 64, 4)),
])
def test_selector(lib, args, want):
    bm, bn, waves, lds = B.select_tiles(*args)
    assert (bm, bn, waves) == want
    assert 0 < lds <= 160 * 1024


def test_selector_rejects(lib):
    with pytest.raises(B.AttnError) as e:
        B.select_tiles(48, 64, 64, 1, B.F32, 0)
    assert e.value.status == B.ERR_UNSUPPORTED
    with pytest.raises(B.AttnError) as e:
        B.select_tiles(128, 64, 64, 1, 7, 0)
    assert e.value.status == B.ERR_INVALID_ARG


# Fake device addresses: every call below fails validation, so nothing is
# ever dereferenced and no HIP call is made.
A0, A1, A2, A3, A4 = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000


def _call(lib, q=A0, k=A1, v=A2, o=A3, lse=A4, Bn=1, H=2, Sq=64, Skv=64, d=64, scale=0.125,
          causal=0, dtype=B.F32, tiles=None):
    args = (q, k, v, o, lse, Bn, H, Sq, Skv, d, scale, causal, dtype, None)
    if tiles is None:
        return lib.attn_fwd(*args)
    return lib.attn_fwd_tiles(*args, *tiles)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), B.ERR_INVALID_ARG),
    (dict(o=None), B.ERR_INVALID_ARG),
    (dict(k=None), B.ERR_INVALID_ARG),
    (dict(v=None), B.ERR_INVALID_ARG),
    (dict(Bn=-1), B.ERR_INVALID_ARG),
    (dict(Sq=-3), B.ERR_INVALID_ARG),
    (dict(Skv=-1), B.ERR_INVALID_ARG),
    (dict(d=0), B.ERR_INVALID_ARG),
    (dict(d=48), B.ERR_UNSUPPORTED),
    (dict(d=16, dtype=B.BF16), B.ERR_UNSUPPORTED),
    (dict(dtype=5), B.ERR_INVALID_ARG),
    (dict(d=16, dtype=B.F16), B.ERR_UNSUPPORTED),
    (dict(d=32, dtype=B.BF16, tiles=(128, 32)), B.ERR_UNSUPPORTED),   # d = 32 takes 64- or 128-key tiles
    (dict(scale=float("nan")), B.ERR_INVALID_ARG),
    (dict(scale=float("inf")), B.ERR_INVALID_ARG),
    (dict(scale=0.0), B.ERR_INVALID_ARG),
    (dict(scale=-0.5), B.ERR_INVALID_ARG),
    (dict(causal=3), B.ERR_INVALID_ARG),
    (dict(causal=-1), B.ERR_INVALID_ARG),
    (dict(q=A0 + 4), B.ERR_MISALIGNED),
    (dict(o=A3 + 8), B.ERR_MISALIGNED),
    (dict(lse=A4 + 2), B.ERR_MISALIGNED),
    (dict(o=A0), B.ERR_INVALID_ARG),                     # o aliases q
    (dict(o=A2 + 64), B.ERR_INVALID_ARG),                # o overlaps v
    (dict(Bn=65536, H=65536), B.ERR_INVALID_ARG),        # B*H overflows
    (dict(tiles=(48, 16)), B.ERR_UNSUPPORTED),
    (dict(tiles=(16, 0)), B.ERR_INVALID_ARG),
    (dict(tiles=(-16, 16)), B.ERR_INVALID_ARG),
    (dict(dtype=B.BF16, tiles=(32, 64)), B.ERR_UNSUPPORTED),
])
def test_invalid_arguments_rejected_on_host(lib, kw, status):
    assert _call(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_empty_problems_are_no_ops(lib):
    # nothing to compute: OK without touching the (null) pointers or the GPU
    assert _call(lib, q=None, k=None, v=None, o=None, lse=None, Sq=0) == B.OK
    assert _call(lib, q=None, k=None, v=None, o=None, lse=None, Bn=0) == B.OK
    assert lib.attn_last_error().decode() == ""


def test_binding_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        B.fwd(q, q, q)


# ------------------------------------------------------------------ attn_fwd_split (host side)
def test_split_workspace_bytes(lib):
    # partial O (fp32) rounded up to 256 bytes, then partial LSE (fp64)
    rows = 3 * 2 * 8
    for n in (1, 2, 7):
        want = (n * rows * 32 * 4 + 255) // 256 * 256 + n * rows * 8
        assert B.split_workspace_bytes(3, 2, 8, 32, n) == want
    for bad in ((3, 2, 8, 32, 0), (3, 2, 8, 0, 2), (-1, 2, 8, 32, 2), (3, 2, 8, 32, 5000)):
        with pytest.raises(B.AttnError):
            B.split_workspace_bytes(*bad)


@pytest.mark.parametrize("args,split", [
    # (d, Sq, Skv, BH, dtype, causal): the stress workloads fill the GPU only when split
    ((32, 8, 1000, 6, B.F32, 0), True),
    ((32, 8, 257, 6, B.F32, 1), False),           # three key tiles: the merge costs more
    ((32, 8, 513, 6, B.F32, 1), True),
    ((32, 8, 64, 6, B.F32, 1), False),            # one key tile: nothing to split
    ((128, 1, 4000, 8, B.BF16, 0), True),
    ((128, 4096, 4096, 32, B.BF16, 1), False),     # enough query tiles already
    ((64, 100, 0, 8, B.BF16, 0), False),           # no keys
])
def test_select_splits(lib, args, split):
    n, chunk = B.select_splits(*args)
    d, Sq, Skv, BH, dtype, causal = args
    _, bn, _, _ = B.select_tiles(*args)
    assert (n > 1) == split
    assert 1 <= n <= 64
    if Skv:
        assert chunk % bn == 0 and (n - 1) * chunk < Skv <= n * chunk


@pytest.mark.parametrize("args,want", [
    # fp32: four waves per CU (1024 in all; a wave owns 16 query rows)
    ((64, 512, 512, 8, B.F32, 0), (1, 512)),       # 256 query tiles of eight key waves
    ((32, 1000, 1000, 6, B.F32, 1), (1, 1024)),    # 378 query tiles of eight key waves
    ((32, 8, 1000, 6, B.F32, 0), (8, 128)),        # 48 waves; capped by the 8 key tiles
    ((32, 16, 4096, 16, B.F32, 0), (8, 512)),      # 16 query tiles x 8 waves -> 8 chunks
    ((64, 2048, 2048, 8, B.F32, 0), (1, 2048)),    # 256 four-wave query tiles already
    # 16-bit: one workgroup per CU (256)
    ((128, 1, 4000, 8, B.BF16, 0), (32, 128)),     # 8 tiles x 32 chunks of 4 key tiles
    ((64, 512, 4096, 16, B.BF16, 0), (2, 2048)),   # 128 query tiles of 64 rows
])
def test_select_splits_counts(lib, args, want):
    assert B.select_splits(*args) == want


def _split(lib, n_splits=2, ws=0x600000, ws_bytes=1 << 20, **kw):
    # 1000 keys in 64-key tiles: two requested chunks do run, so each case
    # below fails validation before any HIP call
    base = dict(q=A0, k=A1, v=A2, o=A3, lse=A4, Bn=1, H=2, Sq=8, Skv=1000, d=32, scale=0.125,
                causal=0, dtype=B.F32)
    base.update(kw)
    return lib.attn_fwd_split(base["q"], base["k"], base["v"], base["o"], base["lse"], base["Bn"],
                              base["H"], base["Sq"], base["Skv"], base["d"], base["scale"],
                              base["causal"], base["dtype"], None, n_splits, ws, ws_bytes)


@pytest.mark.parametrize("kw,status", [
    (dict(n_splits=-1), B.ERR_INVALID_ARG),
    (dict(n_splits=5000), B.ERR_INVALID_ARG),
    (dict(ws=None), B.ERR_INVALID_ARG),                       # chunks need a workspace
    (dict(ws_bytes=64), B.ERR_INVALID_ARG),                   # too small
    (dict(ws=0x600000 + 16), B.ERR_MISALIGNED),
    (dict(ws=A3), B.ERR_INVALID_ARG),                         # overlaps o
    (dict(ws=A0), B.ERR_INVALID_ARG),                         # overlaps q
    (dict(causal=3), B.ERR_INVALID_ARG),
    (dict(causal=-1), B.ERR_INVALID_ARG),
    (dict(d=48), B.ERR_UNSUPPORTED),
    (dict(n_splits=0, ws=None), B.ERR_INVALID_ARG),           # auto split, no workspace
    (dict(ws_bytes=1 << 10, n_splits=16), B.ERR_INVALID_ARG), # too small for the chunks that run
])
def test_split_invalid_arguments_rejected_on_host(lib, kw, status):
    assert _split(lib, **kw) == status
    assert lib.attn_last_error().decode() != ""


def test_sequence_length_limit_per_head(lib):
    # one head's Q, K or V is addressed with 32-bit byte offsets: S * d * 4 must
    # stay below 2^31 (4-byte elements assumed for every dtype)
    smax = (2 ** 31 - 1) // (128 * 4)                  # 4194303 rows at d = 128
    for dtype in (B.F32, B.BF16):
        assert _call(lib, Skv=smax + 1, d=128, dtype=dtype) == B.ERR_INVALID_ARG
        assert "too long" in lib.attn_last_error().decode()
        assert _call(lib, Sq=smax + 1, d=128, dtype=dtype) == B.ERR_INVALID_ARG


def _noalloc(lib, n_splits, Sq, H=64, Skv=4096, d=128, dtype=B.BF16, causal=0):
    # addresses 4 GiB apart: never dereferenced, and far enough apart that
    # no overlap check fires first
    g = 1 << 32
    return lib.attn_fwd_split_noalloc(g, 2 * g, 3 * g, 4 * g, 5 * g, 1, H, Sq, Skv, d, 0.125,
                                      causal, dtype, None, n_splits)


def test_noalloc_rejects_more_than_its_scratch(lib):
    # 64 heads x 256 query rows x 16 chunks of 256 keys at d = 128 need
    # 16 * 16384 * (512 + 8) bytes, beyond the static scratch: refused on the
    # host, with the sizes in the message, before any HIP call
    need = B.split_workspace_bytes(1, 64, 256, 128, 16)
    assert need > B.NOALLOC_SCRATCH_BYTES
    assert _noalloc(lib, 16, 256) == B.ERR_INVALID_ARG
    msg = lib.attn_last_error().decode()
    assert "scratch" in msg and str(need) in msg and str(B.NOALLOC_SCRATCH_BYTES) in msg


@pytest.mark.parametrize("kw,status", [
    (dict(n_splits=-1), B.ERR_INVALID_ARG),
    (dict(n_splits=5000), B.ERR_INVALID_ARG),
    (dict(causal=3), B.ERR_INVALID_ARG),
    (dict(d=48), B.ERR_UNSUPPORTED),
    (dict(dtype=9), B.ERR_INVALID_ARG),
])
def test_noalloc_invalid_arguments_rejected_on_host(lib, kw, status):
    args = dict(n_splits=2, Sq=8)
    args.update(kw)
    assert _noalloc(lib, **args) == status
    assert lib.attn_last_error().decode() != ""


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define ATTN_NOALLOC_SCRATCH_BYTES \((\d+)ll << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.NOALLOC_SCRATCH_BYTES


PROBE_HEADER = os.path.join(ROOT, "include", "attn_probe.h")


def test_probe_library_exports_its_header_and_rejects_bad_kinds():
    # the matrix-core rate probe (measurement only): every function the probe
    # header declares is exported, an invalid kind is refused before any HIP
    # call, and the FLOP count is 16 MFMAs of 32x32x16 per iteration per wave
    path = os.path.join(os.path.dirname(B.lib_path()), "libattn_probe.so")
    assert os.path.exists(path), "libattn_probe.so is not built"
    probe = ctypes.CDLL(path)
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    names = re.findall(r"^\s*(?:int|double)\s+(attn_probe_\w+)\s*\(", text, flags=re.M)
    assert sorted(names) == ["attn_probe_mfma", "attn_probe_mfma_flops"]
    for n in names:
        getattr(probe, n)
    probe.attn_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p]
    probe.attn_probe_mfma_flops.argtypes = [ctypes.c_int] * 3
    probe.attn_probe_mfma_flops.restype = ctypes.c_double
    assert probe.attn_probe_mfma(-1, 10, 4, 0x1000, None) == 1
    assert probe.attn_probe_mfma(4, 10, 4, 0x1000, None) == 1
    assert probe.attn_probe_mfma(0, 0, 4, 0x1000, None) == 1
    assert probe.attn_probe_mfma(0, 10, 4, None, None) == 1
    assert probe.attn_probe_mfma_flops(1, 10, 4) == 16 * 2 * 32 * 32 * 16 * 10 * 4 * 4


def test_last_error_is_per_thread(lib):
    # a failing call on one thread keeps its message while another thread's
    # calls succeed (and clear only their own message)
    import threading
    barrier = threading.Barrier(2)
    seen = {}

    def failing():
        st = lib.attn_select_tiles(48, 64, 64, 1, B.F32, 0, None, None, None, None)
        barrier.wait()          # the other thread succeeds in between
        barrier.wait()
        seen["fail"] = (st, lib.attn_last_error().decode())

    def succeeding():
        barrier.wait()
        st = lib.attn_select_tiles(64, 64, 64, 1, B.F32, 0, None, None, None, None)
        seen["ok"] = (st, lib.attn_last_error().decode())
        barrier.wait()

    threads = [threading.Thread(target=failing), threading.Thread(target=succeeding)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=30)
    assert seen["fail"][0] == B.ERR_UNSUPPORTED and "48" in seen["fail"][1]
    assert seen["ok"] == (B.OK, "")
