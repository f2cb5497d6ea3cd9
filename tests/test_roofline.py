"""The byte model reproduces the pages' worked figures and the workload sizes."""
import json
import os

import pytest

import synth
from persistent_runtime_amd import roofline as rf

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_worked_figures.json")))


def test_pages_weight_only_ceiling():
    g = GOLD["weight_ceiling"]
    wbytes = g["params"] * g["bytes_per_param"]
    assert wbytes == pytest.approx(g["weights_bytes"])
    agg = g["n_gpus"] * g["per_gpu_bytes_per_s"]
    assert agg == pytest.approx(g["aggregate_bytes_per_s"])
    assert wbytes / g["n_gpus"] == pytest.approx(g["per_gpu_shard_bytes"])
    ceil = rf.weight_only_ceiling_tok_s(g["params"], g["bytes_per_param"], agg)
    assert ceil == pytest.approx(7478.26, abs=0.01)
    assert g["measured_tok_s"] / ceil == pytest.approx(g["fraction_of_ceiling_about"], abs=0.005)


def test_pages_launch_cap_and_latency():
    g = GOLD["launch_cap"]
    assert rf.launch_bound_tok_s(g["overhead_us_per_token"]) == pytest.approx(g["cap_tok_s_about"], abs=2)
    lat = GOLD["latency"]
    for tps, ms in zip(lat["tok_s"], lat["ms_per_token_about"]):
        assert 1e3 / tps == pytest.approx(ms, abs=0.005)


def test_pages_lane_qkv_outputs():
    g = GOLD["lane_qkv"]
    assert rf.qkv_rows(g["q_heads"], g["kv_heads"], g["head_dim"]) == g["qkv_outputs"]


def test_workload_byte_counts():
    c3 = synth.CONFIGS["dec2b_25l_greedy"]
    # 25 x (7680*2560 + 2560*2560 + 3*2560*6912 + 2*2560) + 32768*2560 + 2560 + 2560 fp16 elements
    assert rf.weight_bytes(c3) == 2 * (25 * (7680 * 2560 + 2560 * 2560 + 3 * 2560 * 6912 + 5120)
                                        + 32768 * 2560 + 5120)
    assert rf.weight_bytes(c3) == 4_132_966_400
    # K and V rows of 20 heads x 128 dims, 25 layers: 256,000 B per cached position
    assert rf.kv_bytes(c3, 0) - rf.kv_bytes(c3, -1) == 25 * 2 * 20 * 128 * 2
    total = rf.bytes_for_steps(c3, 127, 256)
    assert total == 256 * 4_132_966_400 + 256_000 * sum(p + 2 for p in range(127, 383))
    c5 = synth.CONFIGS["dec8b_32l_gqa"]
    assert rf.weight_bytes(c5) == 2 * (32 * (6144 * 4096 + 4096 * 4096 + 3 * 4096 * 14336 + 8192) + 128256 * 4096 + 8192)
    # GQA 32/8 reads a quarter of the KV bytes of MHA at the same head count
    mha = dict(c5, n_kv_heads=32)
    assert rf.kv_bytes(mha, 500) == 4 * rf.kv_bytes(c5, 500)


def test_flops_about_one_per_byte():
    c3 = synth.CONFIGS["dec2b_25l_greedy"]
    ratio = rf.flops_per_token(c3, 255) / rf.bytes_per_token(c3, 255)
    assert 0.95 < ratio < 1.05


def test_windowed_kv_bytes_closed_form():
    """Sliding-window layers read min(pos+1, W) cached rows (plus the row written),
    the other layers pos+1: the LaneFormer-shaped workload at position 2048 has
    10 windowed layers of 1024 + 1 rows and 5 full layers of 2049 + 1 rows of
    2 x 16 heads x 96 dims x 2 bytes each."""
    lfm = synth.CONFIGS["laneformer_15l_swa"]
    row = 2 * 16 * 96 * 2
    assert rf.kv_bytes(lfm, 2048) == row * (10 * (1024 + 1) + 5 * (2049 + 1))
    # before the window fills, windowed and full layers read the same rows
    assert rf.kv_bytes(lfm, 100) == row * 15 * (101 + 1)
    # an all-zero mask is the unwindowed count, whatever the window
    assert rf.kv_bytes(dict(lfm, window_layers=0), 2048) == rf.kv_bytes(dict(lfm, sliding_window=0), 2048)
    assert rf.kv_bytes(dict(lfm, window_layers=0), 2048) == row * 15 * (2049 + 1)
