"""Pins of the oracle's bf16-weight expert (Linear layers without scales).

Permutation weights give a closed form that shows the wiring; two-one rows
make the bf16 rounding of the Linear outputs visible; where the FP8 path's
quantisation is exact (activations that are e4m3 numbers with block maximum
448, weights that are e4m3 numbers with unit scales) the first Linear of both
paths must agree; the layer identity for identical experts holds as well.
"""
import numpy as np
import torch

import oracle
import synth

BF16_ONE = 0x3F80
E4M3_ONE = 0x38


def _perm_bf16(perm, bits=BF16_ONE):
    n = len(perm)
    w = np.zeros((n, n), np.uint16)
    w[np.arange(n), perm] = bits          # row o picks input perm[o]
    return w


def _bf16_values(rng, shape, scale=1.0):
    return oracle.bf16_round(rng.standard_normal(shape) * scale)


def test_bf16_expert_closed_form_with_permutation_weights():
    rng = np.random.default_rng(10)
    n = 64
    p1, p3, p2 = rng.permutation(n), rng.permutation(n), rng.permutation(n)
    w1, w3, w2 = _perm_bf16(p1), _perm_bf16(p3, 0x4000), _perm_bf16(p2)      # 0x4000 = 2.0
    x = _bf16_values(rng, (3, n), 3.0)
    o = oracle.expert_ffn_bf16(x, oracle.bf16_weight(w1), oracle.bf16_weight(w3), oracle.bf16_weight(w2), full=True)
    g, u = x[:, p1], 2.0 * x[:, p3]
    assert np.array_equal(o["g"], g) and np.array_equal(o["u"], u)
    assert np.array_equal(o["h"], oracle.bf16_round(g / (1.0 + np.exp(-g)) * u))
    assert np.array_equal(o["o"], o["h"][:, p2])


def test_bf16_expert_saturated_silu_picks_the_gate_branch():
    # g = +-20 saturates SiLU: silu(20) = 20 (to bf16), silu(-20) ~ 0; u = 3
    x = np.array([[20.0, 3.0], [-20.0, 3.0]])
    w1 = np.array([[1.0, 0.0], [1.0, 0.0]])       # g = x0
    w3 = np.array([[0.0, 1.0], [0.0, 1.0]])       # u = x1
    w2 = np.eye(2)
    o = oracle.expert_ffn_bf16(x, w1, w3, w2)
    assert o[0, 0] == 60.0 and o[0, 1] == 60.0
    assert abs(o[1, 0]) < 1e-6 and abs(o[1, 1]) < 1e-6  # SiLU on u instead would give about -57


def test_bf16_expert_linear_outputs_are_rounded_to_bf16():
    rng = np.random.default_rng(11)
    n = 64
    p, q = rng.permutation(n), rng.permutation(n)
    q = np.where(q == p, (q + 1) % n, q)
    w1 = np.zeros((n, n))
    w1[np.arange(n), p] = 1.0
    w1[np.arange(n), q] = 1.0
    x = _bf16_values(rng, (4, n))
    o = oracle.expert_ffn_bf16(x, w1, np.eye(n), np.eye(n), full=True)
    exact = x[:, p] + x[:, q]
    assert np.array_equal(o["g"], oracle.bf16_round(exact))
    assert not np.array_equal(o["g"], exact)


def test_first_linear_agrees_with_the_fp8_path_where_quantisation_is_exact():
    rng = np.random.default_rng(12)
    n = 128
    t = oracle.e4m3_table()[:127]
    vals = np.concatenate([t[40:], -t[40:]])
    x = rng.choice(vals, size=(3, n))
    x[:, 0] = 448.0                                      # block max 448: activation scale 1, exact
    codes = rng.integers(0, 127, size=(2, n, n)).astype(np.uint8)
    codes |= (rng.integers(0, 2, size=codes.shape) << 7).astype(np.uint8)
    one = np.ones((1, 1), np.float32)
    fp8 = oracle.expert_ffn(x, codes[0], one, codes[1], one, codes[0], one, full=True)
    w1 = oracle.e4m3_decode(codes[0])                     # e4m3 values are bf16 numbers
    w3 = oracle.e4m3_decode(codes[1])
    bf = oracle.expert_ffn_bf16(x, w1, w3, w1, full=True)
    assert np.array_equal(fp8["g"], bf["g"]) and np.array_equal(fp8["u"], bf["u"])
    assert np.array_equal(fp8["h"], bf["h"])


def test_layer_identity_with_identical_bf16_experts():
    dims = synth.TINY
    p = {k: (v.view(torch.int16).numpy().view(np.uint16) if v.dtype == torch.bfloat16 else v.numpy())
         for k, v in synth.make_block(dims, "normal:0.1", "cpu", 3, weights="bf16").items()}
    assert "s1" not in p
    for k in ("w1", "w3", "w2"):
        p[k] = np.repeat(p[k][:1], dims.n_experts, axis=0)
    x = oracle.bf16_round(np.random.default_rng(13).standard_normal((6, dims.d_model)))
    r = oracle.moe_forward(x, p, dims)
    ex = oracle.expert_ffn_bf16(x, *(oracle.bf16_weight(p[k][0]) for k in ("w1", "w3", "w2")))
    sh = oracle.expert_ffn_bf16(x, *(oracle.bf16_weight(p["sh_" + k][0]) for k in ("w1", "w3", "w2")))
    assert np.allclose(r["y"], dims.route_scale * ex + sh, rtol=0, atol=1e-12 * (1 + np.abs(r["y"]).max()))
    assert np.array_equal(oracle.moe_forward(np.zeros_like(x), p, dims)["y"], np.zeros_like(x))
