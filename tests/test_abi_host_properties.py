"""Property test of the C ABI's host-side validation (no GPU): any non-empty
problem carrying one or more invalid arguments is rejected before any HIP
call, with an argument status (never OK, never a HIP status) and a message.
The faults are the ones include/attn.h documents; each single fault's exact
status is pinned in test_abi_host.py."""
import os

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tiled_online_softmax_05_amd import binding as B

# distinct, 16-byte aligned fake device addresses far apart (never dereferenced:
# every call below fails validation on the host)
BASE = {"q": 1 << 40, "k": 2 << 40, "v": 3 << 40, "o": 4 << 40, "lse": 5 << 40}
DIMS = {B.F32: [16, 32, 64, 128], B.BF16: [32, 64, 128], B.BF16_OUT_F32: [32, 64, 128],
        B.F16: [32, 64, 128], B.F16_OUT_F32: [32, 64, 128]}
FAULTS = ["q_null", "o_null", "k_null", "v_null", "negative_size", "d_nonpositive",
          "d_unsupported", "dtype_unknown", "scale_bad", "causal_bad", "ptr_misaligned",
          "lse_misaligned", "o_overlaps", "tiles_bad"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.lib_path()):
        pytest.fail("libattn.so is not built; run python -m tiled_online_softmax_05_amd.build")
    return B.load()


@st.composite
def faulty_call(draw):
    dtype = draw(st.sampled_from(sorted(DIMS)))
    a = dict(ptr=dict(BASE), Bn=draw(st.integers(1, 4)), H=draw(st.integers(1, 8)),
             Sq=draw(st.integers(1, 300)), Skv=draw(st.integers(1, 300)),
             d=draw(st.sampled_from(DIMS[dtype])), scale=draw(st.floats(1e-3, 4.0)),
             causal=draw(st.integers(0, 2)), dtype=dtype, tiles=None)
    faults = draw(st.lists(st.sampled_from(FAULTS), min_size=1, max_size=4, unique=True))
    for f in faults:
        if f.endswith("_null"):
            a["ptr"][f[:-5]] = None
        elif f == "negative_size":
            a[draw(st.sampled_from(["Bn", "H", "Sq", "Skv"]))] = -draw(st.integers(1, 5))
        elif f == "d_nonpositive":
            a["d"] = -draw(st.integers(0, 64))
        elif f == "d_unsupported":
            a["d"] = draw(st.sampled_from([8, 24, 48, 96, 256] +
                                          ([16] if a["dtype"] != B.F32 else [])))
        elif f == "dtype_unknown":
            a["dtype"] = draw(st.sampled_from([-1, 5, 6, 100]))
        elif f == "scale_bad":
            a["scale"] = draw(st.sampled_from([0.0, -0.5, float("nan"), float("inf"),
                                               -float("inf")]))
        elif f == "causal_bad":
            a["causal"] = draw(st.sampled_from([-1, 3, 7]))
        elif f == "ptr_misaligned":
            name = draw(st.sampled_from(["q", "k", "v", "o"]))
            if a["ptr"][name] is not None:
                a["ptr"][name] += draw(st.integers(1, 15))
        elif f == "lse_misaligned":
            a["ptr"]["lse"] += draw(st.integers(1, 3))
        elif f == "o_overlaps":
            if a["ptr"]["o"] is not None:
                a["ptr"]["o"] = BASE[draw(st.sampled_from(["q", "k", "v", "lse"]))]
        elif f == "tiles_bad":
            a["tiles"] = draw(st.sampled_from([(-16, 32), (16, -32), (0, 32), (64, 0)]))
    return a, faults


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.function_scoped_fixture])
@given(faulty_call())
def test_any_invalid_argument_set_is_rejected_on_the_host(lib, case):
    a, faults = case
    p = a["ptr"]
    args = (p["q"], p["k"], p["v"], p["o"], p["lse"], a["Bn"], a["H"], a["Sq"], a["Skv"],
            a["d"], a["scale"], a["causal"], a["dtype"], None)
    st_ = lib.attn_fwd(*args) if a["tiles"] is None else lib.attn_fwd_tiles(*args, *a["tiles"])
    assert st_ in (B.ERR_INVALID_ARG, B.ERR_UNSUPPORTED, B.ERR_MISALIGNED), (st_, faults, a)
    assert lib.attn_last_error().decode() != ""
    # the selector agrees on what it can judge (head dim and dtype)
    if a["dtype"] in DIMS and a["d"] > 0 and a["d"] not in DIMS[a["dtype"]]:
        with pytest.raises(B.AttnError):
            B.select_tiles(a["d"], 64, 64, 1, a["dtype"], 0)
