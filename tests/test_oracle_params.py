"""The pages' printed parameter counts and sizes pin the layer's shapes.

Values come from tests/golden/pages_numbers.json (each entry cites its page
and section).  The MoE count decomposes exactly into 257 SwiGLU experts of
7168x2048, a 256x7168 router weight and a 256-element router bias.
"""
import json
import os

import synth
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def v(name):
    return GOLD[name]["value"]


def test_moe_param_count_full_shape():
    assert oracle.param_count(synth.FULL) == v("moe_params_per_block")


def test_block_and_model_totals():
    block = oracle.param_count(synth.FULL) + v("mla_params_per_block") + 2 * v("rmsnorm_params")
    assert block == v("block_params")
    assert block * v("moe_blocks") == v("all_moe_block_params")


def test_expert_matrix_counts():
    d, I = synth.FULL.d_model, synth.FULL.inter
    assert (d, I) == (v("d_model"), v("expert_d_ff"))
    assert d * I == v("w1_params")
    assert d * I * v("routed_experts") == v("w1_params_all_experts")
    assert d * I * v("routed_experts") * v("moe_blocks") == v("w1_params_all_blocks")


def test_stored_sizes():
    # FP8: one byte per MoE parameter; the printed size is rounded to 0.1 GiB
    assert round(oracle.param_count(synth.FULL) / 2 ** 30, 1) == v("moe_fp8_gib")
    # two float32 RMSNorm gains of d features each
    assert 2 * synth.FULL.d_model * 4 / 1024 == v("two_rmsnorms_fp32_kib")
    share = oracle.param_count(synth.FULL) / v("block_params") * 100
    assert round(share, 1) == v("moe_share_percent")
    assert oracle.BLOCK == v("block_size")


def test_generated_tensors_match_the_count():
    p = synth.make_block(synth.TINY, "normal:0.1", "cpu", 0)
    assert synth.block_tensors_numel(p) == oracle.param_count(synth.TINY)
    # scale tensors: [ceil(out/128), ceil(in/128)] per Linear
    assert tuple(p["s1"].shape) == (16, 1, 4) and tuple(p["s2"].shape) == (16, 4, 1)
