"""Workload shapes against the report's Table 1 / Sections 2.1 and 3.2 (golden)."""
import json
import os

from sliding_window_sink_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table1_config.json")


def test_constants_match_table1():
    g = json.load(open(GOLDEN))
    assert synth.DQK == g["qk_head_dim"] and synth.DV == g["v_head_dim"]
    assert synth.WINDOW == g["sliding_window"] and synth.ROPE_DIM == g["rope_dims"]
    assert synth.BASE_SWA == g["rope_base_swa"] and synth.BASE_GA == g["rope_base_ga_stage3"]
    w = synth.WORKLOADS
    assert (w[2].Hq, w[2].Hkv) == (g["swa_q_heads"], g["swa_kv_heads"])
    assert (w[3].Hq, w[3].Hkv) == (g["ga_q_heads"], g["ga_kv_heads"])
    assert (w[5].Hq, w[5].Hkv) == (g["swa_q_heads"], g["swa_kv_heads"])
    # 1 GA layer first, then M blocks of N SWA + 1 GA with the first SWA slot
    # taken by that layer: 39 SWA + 9 GA = 48 layers
    total, swa, ga = g["layers_total_swa_ga"]
    M, N = g["hybrid_blocks_M"], g["swa_per_block_N"]
    assert M * (N + 1) == total and M * N - 1 == swa and M + 1 == ga


def test_generators_are_seeded_and_rne():
    q1, k1, v1, s1 = synth.prefill_inputs(7, 1, 16, 8, 1)
    q2, k2, v2, s2 = synth.prefill_inputs(7, 1, 16, 8, 1)
    assert all((a.view(-1) == b.view(-1)).all() for a, b in ((q1, q2), (k1, k2), (v1, v2), (s1, s2)))
    assert q1.shape == (1, 16, 8, 192) and v1.shape == (1, 16, 1, 128) and s1.dtype.is_floating_point
