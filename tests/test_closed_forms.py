"""Pins for the closed forms, against the values the pages print."""
import json
import os

import pytest

from oracle import closed_forms as cf


@pytest.fixture(scope="module")
def printed(golden_dir):
    return json.load(open(os.path.join(golden_dir, "pages_printed_values.json")))


def test_expected_tokens_reproduces_printed_values(printed):
    e = printed["expected_tokens_k4"]
    for a, v in zip(e["alpha"], e["printed"]):
        assert round(cf.expected_tokens(a, e["k"]), 1) == v
    assert cf.expected_tokens(1.0, e["k"]) == e["cap"]
    assert cf.expected_tokens(0.999999, e["k"]) == pytest.approx(e["cap"], rel=1e-5)
    assert cf.expected_tokens(0.0, e["k"]) == 1.0
    # exact values of the printed roundings
    assert cf.expected_tokens(0.5, 4) == pytest.approx(1.9375, abs=1e-12)
    assert cf.expected_tokens(0.7, 4) == pytest.approx(2.77310, abs=1e-5)
    assert cf.expected_tokens(0.9, 4) == pytest.approx(4.09510, abs=1e-5)


def test_expected_tokens_workload_values():
    assert cf.expected_tokens(0.7, 3) == pytest.approx(2.533, abs=1e-3)
    assert cf.expected_tokens(0.6, 7) == pytest.approx(2.458, abs=1e-3)


def test_kv_cache_sizes_reproduce_printed_values(printed):
    e = printed["kv_per_layer_token"]
    for c in e["cases"]:
        n = cf.kv_elements_per_layer_token(c["H_kv"], e["head_dim"])
        assert n == c["elements"]
        per_token = cf.kv_cache_bytes(e["layers"], c["H_kv"], e["head_dim"], 1, e["bytes_per_value"])
        if "per_token_printed_MB" in c:
            assert per_token / 1e6 == pytest.approx(c["per_token_printed_MB"], rel=0.03)
        else:
            assert round(per_token / 1e3) == c["per_token_printed_KB"]
        total = cf.kv_cache_bytes(e["layers"], c["H_kv"], e["head_dim"], e["context_tokens"],
                                  e["bytes_per_value"])
        assert round(total / 1e9) == c["context_printed_GB"]
    # the reduction factors the pages quote: GQA-8 is 1/16 of MHA, MQA 1/128
    mha = cf.kv_elements_per_layer_token(128, 128)
    assert mha // cf.kv_elements_per_layer_token(8, 128) == 16
    assert mha // cf.kv_elements_per_layer_token(1, 128) == 128


def test_score_table_size(printed):
    e = printed["score_table"]
    n = cf.score_table_entries(e["T"])
    assert round(n / 1e5) * 1e5 == e["entries_printed_approx"]
    assert round(n * e["bytes_per_entry"] / 1e6) == e["bytes_printed_MB"]


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16, 64])
@pytest.mark.parametrize("D", [0, 1, 3, 7, 15, 31])
def test_decode_intensity_is_2G_times_1_plus_D(G, D):
    assert cf.decode_intensity_flops_per_kv_element(G, D) == 2 * G * (1 + D)
    assert cf.decode_intensity_flops_per_kv_element(G, D, hd=64) == 2 * G * (1 + D)


def test_tile_filling_draft_length(printed):
    tile = printed["decode_intensity"]["tile_rows"]
    assert cf.tile_filling_draft_len(8, tile) == 15       # G = 8 -> D = 15
    assert cf.tile_filling_draft_len(4, tile) == 31
    for G in (1, 2, 4, 8, 16, 32, 64, 128):
        D = cf.tile_filling_draft_len(G, tile)
        assert G * (1 + D) == tile
