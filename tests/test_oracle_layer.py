"""Pins of the oracle's expert, permutation, combine and RMSNorm steps.

Closed forms on hand-built weights (permutation matrices make a transposed or
swapped operand visible), the layer identity that holds when every routed
expert is the same, the invariants of the expert-contiguous permutation, and
the RMSNorm closed form on a constant vector.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth

ONE = 0x38   # e4m3 code of 1.0
TWO = 0x40   # e4m3 code of 2.0


def _perm_weight(perm, code=ONE):
    n = len(perm)
    w = np.zeros((n, n), np.uint8)
    w[np.arange(n), perm] = code          # row o picks input perm[o]
    return w


def test_expert_ffn_closed_form_with_permutation_weights():
    rng = np.random.default_rng(0)
    n = 128
    p1, p3, p2 = rng.permutation(n), rng.permutation(n), rng.permutation(n)
    one = np.ones((1, 1), np.float32)
    w1, w3, w2 = _perm_weight(p1), _perm_weight(p3, TWO), _perm_weight(p2)
    # rows whose values are e4m3 numbers with block max 448: the activation quantiser is exact
    t = oracle.e4m3_table()[:127]
    x = rng.choice(np.concatenate([t[40:], -t[40:]]), size=(3, n))
    x[:, 0] = 448.0
    o = oracle.expert_ffn(x, w1, one, w3, one, w2, one, full=True)
    g = x[:, p1]
    u = 2.0 * x[:, p3]
    assert np.array_equal(o["g"], g) and np.array_equal(o["u"], u)
    h = oracle.bf16_round(g / (1.0 + np.exp(-g)) * u)
    assert np.array_equal(o["h"], h)
    hq, hs = oracle.quant_act(h)
    hd = oracle.dequant_act(hq, hs)
    assert np.array_equal(o["o"], oracle.bf16_round(hd[:, p2]))


def test_expert_ffn_w2_scale_is_linear():
    rng = np.random.default_rng(1)
    dims = synth.Dims(d_model=256, n_experts=2, n_groups=1, topk_groups=1, topk=1, inter=128)
    ew = synth.expert_weights(dims, 1, "cpu", 5, 0)
    a = {k: v[0].numpy() for k, v in ew.items()}
    x = oracle.bf16_round(rng.standard_normal((5, 256)))
    base = oracle.expert_ffn(x, a["w1"], a["s1"], a["w3"], a["s3"], a["w2"], a["s2"])
    dbl = oracle.expert_ffn(x, a["w1"], a["s1"], a["w3"], a["s3"], a["w2"], a["s2"] * 2)
    assert np.array_equal(dbl, 2 * base)


def _tiny_params(seed=0, dims=synth.TINY, bias="normal:0.1"):
    p = synth.make_block(dims, bias, "cpu", seed)
    return {k: v.numpy() for k, v in p.items()}


def test_identical_experts_give_route_scale_times_expert_plus_shared():
    dims = synth.TINY
    p = _tiny_params(1)
    for k in ("w1", "s1", "w3", "s3", "w2", "s2"):
        p[k] = np.repeat(p[k][:1], dims.n_experts, axis=0)
    x = synth.make_x(dims, 32, "cpu", 9).float().numpy().astype(np.float64)
    out = oracle.moe_forward(x, p, dims)
    e = oracle.expert_ffn(x, p["w1"][0], p["s1"][0], p["w3"][0], p["s3"][0], p["w2"][0], p["s2"][0])
    s = oracle.expert_ffn(x, p["sh_w1"][0], p["sh_s1"][0], p["sh_w3"][0], p["sh_s3"][0], p["sh_w2"][0], p["sh_s2"][0])
    assert np.allclose(out["y"], dims.route_scale * e + s, rtol=1e-12, atol=1e-12)


def test_zero_input_gives_zero_update():
    dims = synth.TINY
    p = _tiny_params(2)
    out = oracle.moe_forward(np.zeros((4, dims.d_model)), p, dims)
    assert np.all(out["y"] == 0)


def test_token_subset_matches_full_evaluation():
    dims = synth.TINY
    p = _tiny_params(3)
    x = synth.make_x(dims, 64, "cpu", 3).float().numpy().astype(np.float64)
    full = oracle.moe_forward(x, p, dims)
    sub = oracle.moe_forward(x, p, dims, tokens=[5, 0, 63])
    assert np.array_equal(sub["y"], full["y"][[5, 0, 63]])
    forced = oracle.moe_forward(x, p, dims, idx=full["idx"])
    assert np.array_equal(forced["y"], full["y"])


def test_combine_is_weighted_sum_of_selected_experts():
    # one token, evaluated expert by expert against the layer output
    dims = synth.TINY
    p = _tiny_params(4)
    x = synth.make_x(dims, 8, "cpu", 4).float().numpy().astype(np.float64)
    out = oracle.moe_forward(x, p, dims)
    t = 6
    want = np.zeros(dims.d_model)
    for e, w in zip(out["idx"][t], out["w"][t]):
        o = oracle.expert_ffn(x[t:t + 1], p["w1"][e], p["s1"][e], p["w3"][e], p["s3"][e], p["w2"][e], p["s2"][e])
        want += w * o[0]
    want += oracle.expert_ffn(x[t:t + 1], p["sh_w1"][0], p["sh_s1"][0], p["sh_w3"][0], p["sh_s3"][0],
                              p["sh_w2"][0], p["sh_s2"][0])[0]
    assert np.allclose(out["y"][t], want, rtol=1e-12, atol=1e-12)


def test_combine_adds_choices_in_ascending_expert_id_then_shared():
    # float64 sums whose value depends on the order: the expert-1 row holds 1e16,
    # expert 3 holds 1 and expert 5 holds -1e16.  Ascending expert id gives
    # (1e16 + 1) - 1e16 = 0; the order of the choices as given (5, 1, 3) would give 1
    idx = np.array([[5, 1, 3], [2, 0, 4]])
    w = np.array([[1.0, 1.0, 1.0], [0.5, 2.0, 0.25]])
    outs = np.zeros((2, 3, 2))
    outs[0, :, 0] = [-1e16, 1e16, 1.0]
    outs[1] = [[2.0, 4.0], [1.0, 8.0], [16.0, 32.0]]
    shared = np.array([[10.0, 0.5], [0.0, 0.0]])
    y = oracle.combine(idx, w, outs, shared)
    assert y[0, 0] == 10.0 and y[0, 1] == 0.5
    assert np.array_equal(y[1], [2.0 * 1.0 + 0.5 * 2.0 + 0.25 * 16.0, 2.0 * 8.0 + 0.5 * 4.0 + 0.25 * 32.0])


@pytest.mark.parametrize("T,E,K", [(64, 16, 4), (1000, 256, 8), (1, 8, 8), (0, 16, 4)])
def test_permutation_invariants(T, E, K):
    rng = np.random.default_rng(T + E)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)]) if T else np.zeros((0, K), np.int64)
    r = oracle.permute(idx, E)
    counts, off, rt, pr = r["counts"], r["offsets"], r["row_token"], r["pair_row"]
    # counts by plain counting
    c2 = [0] * E
    for e in idx.ravel().tolist():
        c2[e] += 1
    assert counts.tolist() == c2
    assert counts.sum() == T * K and off[0] == 0 and off[-1] == T * K
    assert sorted(pr.ravel().tolist()) == list(range(T * K))      # bijection
    for t in range(T):
        for k in range(K):
            row = pr[t, k]
            assert rt[row] == t
            assert off[idx[t, k]] <= row < off[idx[t, k] + 1]
    for e in range(E):
        seg = rt[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)                             # ascending tokens


def test_rmsnorm_constant_vector_closed_form():
    d = 7168
    x = np.full((1, d), 1.5)
    res = np.full((1, d), 0.5)
    gain = np.full(d, 1.25, np.float32)
    out, res_new = oracle.add_rmsnorm(x, res, gain)
    c = 2.0
    assert np.all(res_new == 2.0)
    assert np.all(out == oracle.bf16_round(1.25 * c / math.sqrt(c * c + 1e-6)))


def test_rmsnorm_unit_gain_gives_unit_rms_and_library_residual():
    rng = np.random.default_rng(5)
    xt = torch.from_numpy(rng.standard_normal((8, 7168)).astype(np.float32)).to(torch.bfloat16)
    rt = torch.from_numpy(rng.standard_normal((8, 7168)).astype(np.float32) * 3).to(torch.bfloat16)
    x = xt.double().numpy()
    r = rt.double().numpy()
    out, res_new = oracle.add_rmsnorm(x, r, np.ones(7168, np.float32))
    assert np.allclose(np.sqrt((out ** 2).mean(-1)), 1.0, atol=2e-3)
    # the new residual is the float32 sum cast to bf16 (as the rmsnorm excerpt writes it)
    lib = (xt.float() + rt.float()).to(torch.bfloat16).double().numpy()
    assert np.array_equal(res_new, lib)


def test_expert_linear_outputs_are_rounded_to_bf16():
    # two ones per row of W1: g = x[p] + x[q], which needs more than 8 significant bits
    rng = np.random.default_rng(6)
    n = 128
    p, q = rng.permutation(n), rng.permutation(n)
    q = np.where(q == p, (q + 1) % n, q)
    w1 = np.zeros((n, n), np.uint8)
    w1[np.arange(n), p] = ONE
    w1[np.arange(n), q] = ONE
    ident = _perm_weight(np.arange(n))
    one = np.ones((1, 1), np.float32)
    t = oracle.e4m3_table()[:127]
    x = rng.choice(np.concatenate([t[40:], -t[40:]]), size=(2, n))
    x[:, 0] = 448.0
    o = oracle.expert_ffn(x, w1, one, ident, one, ident, one, full=True)
    exact = x[:, p] + x[:, q]
    assert np.array_equal(o["g"], oracle.bf16_round(exact))
    assert not np.array_equal(o["g"], exact)          # the rounding is visible on these inputs


def test_rmsnorm_eps_matters_for_small_vectors():
    d = 256
    c = 2.0 ** -10                                    # c^2 ~ 9.5e-7, comparable to eps = 1e-6
    out, _ = oracle.add_rmsnorm(np.full((1, d), c), np.zeros((1, d)), np.ones(d, np.float32))
    assert np.all(out == oracle.bf16_round(c / math.sqrt(c * c + 1e-6)))
    assert out[0, 0] < 0.75
