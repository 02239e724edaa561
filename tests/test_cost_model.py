"""The byte and flop accounting of the benchmark, the FP8 latent row layout and the
input generator against the figures printed on the dsa-indexer diagram's cost box
(tests/golden/dsa_cost_model.txt)."""
import dataclasses
import os

import numpy as np

import bench
import dsa_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dsa_cost_model.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k.strip()] = int(v)
    return vals


def test_golden_figures_are_consistent():
    g = _golden()
    assert g["latent_row_bytes"] + g["indexer_key_bytes"] == g["token_layer_bytes"]
    assert g["token_layer_bytes"] * g["layers"] == g["token_all_layers_bytes"]
    # one FP8 byte per indexer dimension plus one fp32 scale per key
    assert g["indexer_key_bytes"] == g["indexer_head_dim"] + 4
    # 512 FP8 latent values, four fp32 block scales, 64 bf16 rope values
    assert g["latent_row_bytes"] == 512 + 4 * 4 + (g["latent_width"] - 512) * 2


def test_storage_formats_match_the_figures():
    g = _golden()
    assert S.FP8_LATENT_ROW_BYTES == g["latent_row_bytes"]
    cfg = S.CONFIGS["decode_v32"]
    assert (cfg.H_I, cfg.D_I, cfg.k, cfg.H, cfg.Dq) == (g["indexer_heads"], g["indexer_head_dim"],
                                                     g["topk"], g["attention_heads"], g["latent_width"])
    small = dataclasses.replace(cfg, B=1, Lmax=300, lens="ragged:200:300")
    c8 = S.make_case(small, latent_form="fp8")
    assert c8["latent"].shape[-1] == g["latent_row_bytes"]
    assert c8["k_i"].shape[-1] + c8["k_scale"].itemsize == g["indexer_key_bytes"]


def test_benchmark_accounting():
    """Indexer: 132 B per cached key and 2*64*128 flops per visible (row, key); latent
    attention: one row of 1152 B (bf16) or 656 B (FP8) per selected row."""
    g = _golden()
    cfg = S.CONFIGS["decode_v32"]
    lens = S.lengths(cfg)
    bf = bench.algorithmic_costs(cfg, lens)
    f8 = bench.algorithmic_costs(cfg, lens, "fp8")
    rows = cfg.B * cfg.T
    per_row_q = cfg.H_I * cfg.D_I + 8 * cfg.H_I
    assert bf["index_bytes"] == int(np.sum(lens)) * g["indexer_key_bytes"] + rows * per_row_q
    assert bf["index_flops"] == bf["keys"] * 2 * g["indexer_heads"] * g["indexer_head_dim"]
    sel = rows * g["topk"]
    assert bf["selected"] == sel
    assert bf["attention_bytes"] - f8["attention_bytes"] == sel * (cfg.Dq * 2 - g["latent_row_bytes"])
    assert bf["attention_flops"] == f8["attention_flops"] == sel * 2 * g["attention_heads"] * (cfg.Dq + cfg.Dv)
