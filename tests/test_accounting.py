"""Host-side work and byte accounting, pinned to the logical-access sweep
printed on "Verify tiled attention" (section "Compare the attention
outputs") and to its access-growth unit check ("Read the executable
checks")."""
import pytest

from pin_checks import golden
from tiled_online_softmax_05_amd import accounting as acc


@pytest.mark.parametrize("row", golden("p1_access_sweep.json")["printed"],
                         ids=lambda r: f"S{r['seq_len']}")
def test_logical_access_model_matches_printed_sweep(row):
    st = golden("p1_access_sweep.json")["setup"]
    m = acc.logical_access_model(row["seq_len"], st["num_heads"], st["head_dim"],
                                 st["bytes_per_elem"], st["block_q"])
    assert round(m["qkvo_bytes"] / 1e6, 2) == row["standard_qkv_o_mb"]
    assert round(m["nxn_matrix_bytes"] / 1e6, 2) == row["standard_nxn_matrix_hbm_mb"]
    assert round(m["standard_total_bytes"] / 1e6, 2) == row["standard_total_hbm_mb"]
    assert round(m["tiled_logical_bytes"] / 1e6, 2) == row["tiled_logical_access_mb_no_cache_reuse"]
    assert m["num_q_blocks"] == row["num_q_blocks"]


def test_access_growth_check():
    c = golden("p1_unit_checks.json")["access_growth"]
    small = acc.logical_access_model(c["seq_len_small"])
    large = acc.logical_access_model(c["seq_len_large"])
    assert small["tiled_logical_bytes"] > small["qkvo_bytes"]
    assert large["tiled_logical_bytes"] / small["tiled_logical_bytes"] > c["large_over_small_greater_than"]


def test_flops_and_pairs():
    # 4*B*H*Sq*Skv*d, halved for causal
    assert acc.attention_flops(1, 32, 4096, 4096, 128, True) == 4 * 32 * 4096 * 4096 * 128 / 2
    assert acc.attention_flops(2, 4, 512, 512, 64, False) == 4 * 2 * 4 * 512 * 512 * 64
    assert acc.visible_pairs(64, 64, True) == 64 * 65 // 2
    assert acc.visible_pairs(8, 5, True) == 1 + 2 + 3 + 4 + 5
    assert acc.visible_pairs(8, 64, True) == sum(57 + i for i in range(8))
    assert acc.tiles_visited(64, 64, 16, 16, True) == 10       # printed on the lab page
    assert acc.tiles_visited(64, 64, 13, 19, True) == 13
    assert acc.tiles_visited(8, 5, 16, 16, True) == 1
    assert acc.compulsory_bytes(1, 32, 4096, 4096, 128, 2, 2) == 4 * 32 * 4096 * 128 * 2 + 32 * 4096 * 4
