"""Pins of the FP8 block (de)quantisation in the oracle.

The weight layout ("Gate projection", Linear excerpt) is [out, in] with one
float32 scale per 128x128 block, scale tensor [ceil(out/128), ceil(in/128)].
The activation rule (per row, per 128 block, scale = amax/448) is the
oracle's reading of the step the pages omit; its pins are the exact-error
bound of rounding to the nearest e4m3 value and its special cases.
"""
import numpy as np

import oracle


def test_dequant_weight_scale_orientation():
    # out = 256 (two row blocks), in = 384 (three column blocks): each block gets its own scale
    codes = np.full((256, 384), 0x38, dtype=np.uint8)          # every code is 1.0
    scale = np.arange(1, 7, dtype=np.float32).reshape(2, 3)    # [out/128, in/128]
    w = oracle.dequant_weight(codes, scale)
    for ob in range(2):
        for ib in range(3):
            blk = w[ob * 128:(ob + 1) * 128, ib * 128:(ib + 1) * 128]
            assert np.all(blk == scale[ob, ib])


def test_quant_act_zero_and_constant_blocks():
    v = np.zeros((2, 256))
    v[1, 128:] = 3.0
    q, s = oracle.quant_act(v)
    assert s.dtype == np.float32
    assert s[0, 0] == 1.0 and s[0, 1] == 1.0 and s[1, 0] == 1.0
    assert np.all(q[0] == 0) and np.all(q[1, :128] == 0)
    assert s[1, 1] == np.float32(3.0) / np.float32(448.0)
    assert np.all(q[1, 128:] == 0x7E)                          # 3 / (3/448) = 448


def test_quant_act_error_bound_and_amax():
    rng = np.random.default_rng(0)
    v = oracle.bf16_round(rng.standard_normal((16, 512)) * np.exp(rng.uniform(-8, 8, (16, 1))))
    q, s = oracle.quant_act(v)
    d = oracle.dequant_act(q, s)
    blk_v = v.reshape(16, 4, 128)
    blk_d = d.reshape(16, 4, 128)
    ratio = blk_v / s.astype(np.float64)[..., None]
    # |ratio| <= 448 (up to the float32 rounding of the scale) and each code is the nearest e4m3
    assert np.all(np.abs(ratio) <= 448.0 * (1 + 2.0 ** -22))
    a = np.abs(ratio)
    e = np.maximum(np.floor(np.log2(np.maximum(a, 1e-300))), -6)
    half_step = 2.0 ** (e - 3) / 2
    err = np.abs(blk_d - blk_v) / s.astype(np.float64)[..., None]
    # bound: half a step of the e4m3 binade plus the float32 rounding of v/scale
    assert np.all(err <= half_step * (1 + 1e-6) + a * 2.0 ** -24)
    # the largest element of a block maps to +-448
    arg = np.abs(blk_v).argmax(-1)
    top = np.take_along_axis(np.abs(blk_d / s[..., None]), arg[..., None], -1)
    assert np.allclose(top, 448.0)


def test_quant_act_is_scale_equivariant_for_powers_of_two():
    rng = np.random.default_rng(1)
    v = oracle.bf16_round(rng.standard_normal((4, 256)))
    q1, s1 = oracle.quant_act(v)
    q2, s2 = oracle.quant_act(v * 8.0)
    assert np.array_equal(q1, q2)
    assert np.array_equal(s2, s1 * np.float32(8.0))
