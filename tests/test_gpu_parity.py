"""GPU parity of every entry point of the C ABI against the CPU oracle.

Inputs are seeded synthetic tensors from ``synth`` (shapes and value laws of
the named workloads); expected values always come from ``oracle`` run on the
same inputs.  Each entry point is tested alone on oracle-made inputs, then the
fused forward end to end.  Full-shape (7168 x 256 experts) cases compare the
routing of every token and the outputs of sampled tokens (the layer is
token-wise, so a token's output depends on that token alone).
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_bias_amd as moe
import oracle
import synth
from _helpers import (HostView, assert_close, assert_rows_close, cdims, f64, routing_check, sample_tokens, to_numpy,
                      weights_check)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np_params(p):
    return {k: to_numpy(v) for k, v in p.items()}


@pytest.fixture(scope="module")
def tiny_params():
    return synth.make_block(synth.TINY, "normal:0.1", DEV, seed=0)


def run_gate(dims, p, x):
    T = x.shape[0]
    cd = cdims(dims)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=DEV)
    ws = moe.workspace(cd, T)
    moe.moe_gate(cd, T, x, p["gate_w"], p["gate_b"], idx, w, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy().astype(np.int64), w.cpu().numpy()


def run_forward(dims, p, x):
    layer = moe.MoELayer(cdims(dims), p)
    T = x.shape[0]
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=DEV)
    delta = layer(x, idx=idx, w=w)
    torch.cuda.synchronize()
    return delta, idx.cpu().numpy().astype(np.int64), w.cpu().numpy()


# ----------------------------------------------------------------------------
# single entry points
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 37, 300])
def test_activation_quant_bit_exact(T):
    _say(f"moe_permute xq/xs T={T} d=512")
    dims = synth.TINY
    g = torch.Generator().manual_seed(T)
    x = torch.randn((T, dims.d_model), generator=g) * torch.exp2(torch.empty((T, 4, 1)).uniform_(-20, 20, generator=g)
                                                              ).repeat_interleave(128, 1).reshape(T, dims.d_model)
    x[0, 128:256] = 0.0                      # an all-zero block
    if T > 1:
        x[1, :128] = 0.0
        x[1, 5] = -3.0                       # a block with one non-zero element
    xb = x.to(torch.bfloat16).to(DEV)
    idx = torch.stack([torch.randperm(dims.n_experts, generator=g)[:dims.topk] for _ in range(T)]).int().to(DEV)
    cd = cdims(dims)
    K, E = dims.topk, dims.n_experts
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * K + T, dtype=torch.int32, device=DEV)
    pair_row = torch.empty((T, K), dtype=torch.int32, device=DEV)
    xq = torch.empty((T, dims.d_model), dtype=torch.uint8, device=DEV)
    xs = torch.empty((T, dims.d_model // 128), dtype=torch.float32, device=DEV)
    moe.moe_permute(cd, T, idx, xb, counts, offsets, row_token, pair_row, xq, xs, moe.workspace(cd, T))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_act(f64(xb))
    assert np.array_equal(xq.cpu().numpy(), q_ref)
    assert np.array_equal(xs.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("T", [1, 37, 64, 300])
def test_gate_tiny(tiny_params, T):
    _say(f"moe_gate tiny T={T}")
    dims = synth.TINY
    x = synth.make_x(dims, T, DEV, seed=10 + T)
    gi, gw = run_gate(dims, tiny_params, x)
    p = _np_params(tiny_params)
    r = oracle.gate(f64(x), p["gate_w"], p["gate_b"], dims)
    same, ndiff = routing_check(gi, r, dims)
    assert ndiff == 0
    weights_check(gi, gw, r, same)
    # descending biased score on the GPU side too
    for t in range(T):
        b = r["b"][t, gi[t]]
        assert np.all(np.diff(b) <= 1e-6)


def test_gate_exact_ties_go_to_the_lower_index():
    _say("moe_gate hand-built ties")
    # x = 0: every score is exactly 0.5, so biased scores are 0.5 + bias (multiples of 1/64)
    dims = synth.Dims(d_model=128, n_experts=16, n_groups=8, topk_groups=4, topk=4, inter=128)
    bias = torch.tensor([16, 0, 20, -20, 12, 12, 6, 3, 12, 12, -30, -30, 0, 0, 5, 5], dtype=torch.float32) / 64
    p = {"gate_w": torch.ones((16, 128), device=DEV), "gate_b": bias.to(DEV)}
    x = torch.zeros((3, 128), dtype=torch.bfloat16, device=DEV)
    gi, gw = run_gate(dims, p, x)
    r = oracle.gate(np.zeros((3, 128)), np.ones((16, 128), np.float32), bias.numpy(), dims)
    assert np.array_equal(gi, r["idx"])
    assert np.allclose(gw, 2.5 / 4)


@pytest.mark.parametrize("T,E,K", [(64, 16, 4), (300, 16, 4), (1000, 256, 8), (5000, 256, 8)])
def test_permute_exact(T, E, K):
    _say(f"moe_permute T={T} E={E} K={K}")
    dims = synth.Dims(d_model=256, n_experts=E, n_groups=E // 4, topk_groups=E // 4, topk=K, inter=128)
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(E, K, replace=False) for _ in range(T)])
    if T >= 1000:
        idx[: T // 2, 0] = 7                       # one hot expert spanning many chunks
        for t in range(T // 2):
            row = idx[t]
            dup = np.flatnonzero(row[1:] == 7)
            if dup.size:
                row[1 + dup[0]] = [e for e in range(E) if e not in row][0]
    x = torch.zeros((T, 256), dtype=torch.bfloat16, device=DEV)
    cd = cdims(dims)
    counts = torch.empty(E, dtype=torch.int32, device=DEV)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_token = torch.empty(T * K + T, dtype=torch.int32, device=DEV)
    pair_row = torch.empty((T, K), dtype=torch.int32, device=DEV)
    xq = torch.empty((T, 256), dtype=torch.uint8, device=DEV)
    xs = torch.empty((T, 2), dtype=torch.float32, device=DEV)
    moe.moe_permute(cd, T, torch.from_numpy(idx).int().to(DEV), x, counts, offsets, row_token, pair_row, xq, xs,
                    moe.workspace(cd, T))
    torch.cuda.synchronize()
    ref = oracle.permute(idx, E)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    rt = row_token.cpu().numpy()
    assert np.array_equal(rt[: T * K], ref["row_token"])
    assert np.array_equal(rt[T * K:], np.arange(T))
    assert np.array_equal(pair_row.cpu().numpy(), ref["pair_row"])


def _ffn_with_oracle_routing(dims, p, x, with_shared=True):
    """GPU grouped FFN fed with the oracle's routing, permutation and quantised x."""
    T, K, E, d = x.shape[0], dims.topk, dims.n_experts, dims.d_model
    pn = _np_params(p)
    xv = f64(x)
    r = oracle.gate(xv, pn["gate_w"], pn["gate_b"], dims)
    perm = oracle.permute(r["idx"], E)
    xq, xs = oracle.quant_act(xv)
    rows_tok = np.concatenate([perm["row_token"], np.arange(T)]).astype(np.int32)
    cd = cdims(dims)
    out = torch.zeros((T * K + T, d), dtype=torch.bfloat16, device=DEV)
    routed = moe.experts_struct(*(p[k] for k in ("w1", "w3", "w2", "s1", "s3", "s2")))
    shared = moe.experts_struct(*(p["sh_" + k] for k in ("w1", "w3", "w2", "s1", "s3", "s2"))) if with_shared else None
    moe.moe_grouped_ffn(cd, T, routed, shared, torch.from_numpy(perm["offsets"]).int().to(DEV),
                        torch.from_numpy(rows_tok).to(DEV), torch.from_numpy(xq).to(DEV),
                        torch.from_numpy(xs).to(DEV), out, moe.workspace(cd, T))
    torch.cuda.synchronize()
    return out, r, perm, pn, xv


@pytest.mark.parametrize("T", [37, 300])
def test_grouped_ffn_forced_routing_tiny(tiny_params, T):
    _say(f"moe_grouped_ffn tiny T={T}")
    dims = synth.TINY
    x = synth.make_x(dims, T, DEV, seed=20 + T)
    out, r, perm, pn, xv = _ffn_with_oracle_routing(dims, tiny_params, x)
    got = f64(out)
    off = perm["offsets"]
    ref = np.zeros_like(got)
    for e in range(dims.n_experts):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            ref[rows] = oracle.expert_ffn(xv[perm["row_token"][rows]], pn["w1"][e], pn["s1"][e], pn["w3"][e],
                                          pn["s3"][e], pn["w2"][e], pn["s2"][e])
    ref[T * dims.topk:] = oracle.expert_ffn(xv, pn["sh_w1"][0], pn["sh_s1"][0], pn["sh_w3"][0], pn["sh_s3"][0],
                                            pn["sh_w2"][0], pn["sh_s2"][0])
    assert_rows_close(got, ref, f"grouped_ffn tiny T={T}")


def _idx_with_counts(counts, T, K):
    """A [T, K] routing in which expert e is chosen by exactly counts[e] tokens, K distinct experts per token.

    The expert ids, each repeated counts[e] times in ascending order, fill the matrix column by column; an
    expert's copies are at most T consecutive slots, so they land on distinct tokens."""
    ids = np.repeat(np.arange(len(counts)), counts)
    assert ids.size == T * K and max(counts) <= T
    return ids.reshape(K, T).T.copy()


@pytest.mark.parametrize("T,counts", [
    # 32-row tiles (T <= 768): ragged tails and experts cut into two or three equal tiles
    (100, [0, 1, 15, 16, 17, 31, 32, 33, 48, 49, 63, 65, 30, 0, 0, 0]),
    # ... and into up to 15 tiles each
    (300, [0, 1, 15, 16, 17, 47, 49, 63, 65, 127, 128, 129, 144, 160, 193, 46]),
    (600, [0, 1, 33, 95, 96, 97, 192, 193, 257, 300, 385, 451, 300, 0, 0, 0]),
    # 64-row tiles (769..1280 tokens): one to four sub-tiles with ragged tails, 65 / 129 rows cut
    # into two or three tiles, 400..997 rows into 7 to 16
    (1000, [0, 1, 15, 16, 17, 33, 63, 64, 65, 129, 400, 600, 700, 900, 997, 0]),
    # 128-row tiles (more tokens): one to eight sub-tiles over the two wave rows with ragged
    # tails, 129 / 193 rows in two equal 16-row-aligned tiles, 385..1300 rows in 4 to 11
    (1300, [0, 1, 15, 16, 17, 63, 65, 127, 128, 129, 193, 385, 1000, 1300, 1300, 461]),
])
def test_grouped_ffn_tile_edges(tiny_params, T, counts):
    _say(f"moe_grouped_ffn tile edges T={T}")
    dims = synth.TINY
    K, E, d = dims.topk, dims.n_experts, dims.d_model
    idx = _idx_with_counts(np.array(counts), T, K)
    x = synth.make_x(dims, T, DEV, seed=90 + T)
    pn = _np_params(tiny_params)
    xv = f64(x)
    perm = oracle.permute(idx, E)
    assert np.array_equal(perm["counts"], counts)
    xq, xs = oracle.quant_act(xv)
    rows_tok = np.concatenate([perm["row_token"], np.arange(T)]).astype(np.int32)
    cd = cdims(dims)
    out = torch.zeros((T * K + T, d), dtype=torch.bfloat16, device=DEV)
    routed = moe.experts_struct(*(tiny_params[k] for k in ("w1", "w3", "w2", "s1", "s3", "s2")))
    shared = moe.experts_struct(*(tiny_params["sh_" + k] for k in ("w1", "w3", "w2", "s1", "s3", "s2")))
    moe.moe_grouped_ffn(cd, T, routed, shared, torch.from_numpy(perm["offsets"]).int().to(DEV),
                        torch.from_numpy(rows_tok).to(DEV), torch.from_numpy(xq).to(DEV),
                        torch.from_numpy(xs).to(DEV), out, moe.workspace(cd, T))
    torch.cuda.synchronize()
    got = f64(out)
    ref = np.zeros_like(got)
    off = perm["offsets"]
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            ref[rows] = oracle.expert_ffn(xv[perm["row_token"][rows]], pn["w1"][e], pn["s1"][e], pn["w3"][e],
                                          pn["s3"][e], pn["w2"][e], pn["s2"][e])
    ref[T * K:] = oracle.expert_ffn(xv, pn["sh_w1"][0], pn["sh_s1"][0], pn["sh_w3"][0], pn["sh_s3"][0],
                                    pn["sh_w2"][0], pn["sh_s2"][0])
    assert_rows_close(got, ref, f"grouped_ffn tile edges T={T}")


def test_grouped_ffn_without_shared_leaves_shared_rows(tiny_params):
    _say("moe_grouped_ffn shared=NULL")
    dims = synth.TINY
    x = synth.make_x(dims, 20, DEV, seed=3)
    out, *_ = _ffn_with_oracle_routing(dims, tiny_params, x, with_shared=False)
    assert torch.all(out[20 * dims.topk:] == 0)


def test_combine_with_oracle_rows():
    _say("moe_combine oracle rows")
    dims = synth.Dims(d_model=1024, n_experts=64, n_groups=8, topk_groups=4, topk=8, inter=128)
    T, K, d = 50, dims.topk, dims.d_model
    rng = np.random.default_rng(5)
    idx = np.stack([rng.choice(dims.n_experts, K, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, (T, K))
    w = (w / w.sum(1, keepdims=True) * 2.5).astype(np.float32).astype(np.float64)
    perm = oracle.permute(idx, dims.n_experts)
    rows = oracle.bf16_round(rng.standard_normal((T * K + T, d)) * 0.05)
    y = oracle.combine(idx, w, rows[perm["pair_row"]], rows[T * K:])
    delta = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    moe.moe_combine(cdims(dims), T, torch.from_numpy(idx).int().to(DEV), torch.from_numpy(w).float().to(DEV),
                    torch.from_numpy(perm["pair_row"]).int().to(DEV),
                    torch.from_numpy(rows).to(torch.bfloat16).to(DEV), True, delta)
    torch.cuda.synchronize()
    got = f64(delta)
    # fp32 accumulation + one final bf16 rounding: within one bf16 ulp of the exact sum
    assert np.all(np.abs(got - y) <= np.abs(y) * 2.0 ** -8 + 1e-6)


# widths d: 8-element chunks per thread (1, 2, 4 or 8 in the kernel's templates) with
# full and partial last chunks (512: 64 of 256 threads busy; 2176: 272 chunks; 3072;
# 7168; 12928: 1616 chunks; 16384: every thread's eight chunks)
@pytest.mark.parametrize("T,d", [(1, 512), (5, 2176), (37, 3072), (37, 7168), (4096, 7168), (33, 12928),
                                 (9, 16384)])
def test_add_rmsnorm(T, d):
    _say(f"moe_add_rmsnorm T={T} d={d}")
    g = torch.Generator(device=DEV).manual_seed(T + d)
    x = torch.randn((T, d), generator=g, device=DEV).to(torch.bfloat16)
    res = (torch.randn((T, d), generator=g, device=DEV) * 4).to(torch.bfloat16)
    gain = 1 + 0.02 * torch.randn(d, generator=g, device=DEV)
    hn_ref, res_ref = oracle.add_rmsnorm(f64(x), f64(res), gain.cpu().numpy())
    out = torch.empty_like(x)
    moe.moe_add_rmsnorm(d, T, x, res, gain, 1e-6, out)
    torch.cuda.synchronize()
    assert np.array_equal(f64(res), res_ref)                    # new residual: bit-exact
    got = f64(out)
    diff = np.flatnonzero(got != hn_ref)
    if diff.size:
        xv, rv = f64(x).ravel(), f64(res).ravel()
        for i in diff[:8]:
            print(f"[rmsnorm diff] idx={i} gpu={got.ravel()[i]!r} ref={hn_ref.ravel()[i]!r} "
                  f"x={xv[i]!r} res={rv[i]!r}", flush=True)
    print(f"[parity] add_rmsnorm T={T} d={d}: {diff.size} of {got.size} normalised values differ", flush=True)
    assert np.array_equal(got, hn_ref)                          # normalised rows: bit-exact


def test_add_rmsnorm_products_below_float_range():
    """Gains so small that gain * r / rms lies below half the smallest float32
    subnormal (the float conversion gives a signed zero), at the subnormal
    boundary, and in the bf16 subnormal range: each output is the oracle's
    (a signed zero of the product's sign, never NaN)."""
    _say("moe_add_rmsnorm products below the float32 range")
    d, T = 512, 6
    g = torch.Generator(device=DEV).manual_seed(11)
    x = torch.randn((T, d), generator=g, device=DEV).to(torch.bfloat16)
    res = torch.randn((T, d), generator=g, device=DEV).to(torch.bfloat16)
    tiny = np.array([1.4e-45, -1.4e-45, 2.8e-45, -4.2e-45, 1e-42, -1e-40, 3e-39, -1.2e-38], dtype=np.float32)
    gain = torch.from_numpy(np.resize(tiny, d)).to(DEV)
    hn_ref, res_ref = oracle.add_rmsnorm(f64(x), f64(res), gain.cpu().numpy())
    out = torch.empty_like(x)
    moe.moe_add_rmsnorm(d, T, x, res, gain, 1e-6, out)
    torch.cuda.synchronize()
    got = f64(out)
    n_nan = int(np.isnan(got).sum())
    diff = np.flatnonzero(got != hn_ref)
    print(f"[parity] add_rmsnorm tiny gains: {n_nan} NaN, {diff.size} of {got.size} values differ", flush=True)
    assert n_nan == 0 and diff.size == 0
    assert np.array_equal(f64(res), res_ref)
    ref_sign = np.signbit(hn_ref)
    got_sign = np.signbit(got)
    assert np.array_equal(got_sign, ref_sign)                    # zeros keep the product's sign


def test_add_rmsnorm_in_place_output():
    _say("moe_add_rmsnorm out aliases x")
    d, T = 512, 9
    x = torch.randn((T, d), device=DEV).to(torch.bfloat16)
    res = torch.randn((T, d), device=DEV).to(torch.bfloat16)
    gain = torch.ones(d, device=DEV)
    x2, res2 = x.clone(), res.clone()
    out = torch.empty_like(x)
    moe.moe_add_rmsnorm(d, T, x, res, gain, 1e-6, out)
    moe.moe_add_rmsnorm(d, T, x2, res2, gain, 1e-6, x2)
    torch.cuda.synchronize()
    assert torch.equal(out, x2) and torch.equal(res, res2)


# ----------------------------------------------------------------------------
# fused forward, tiny shape
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 37, 64, 1000])
def test_forward_tiny(tiny_params, T):
    _say(f"moe_forward tiny T={T}")
    dims = synth.TINY
    x = synth.make_x(dims, T, DEV, seed=30 + T)
    delta, gi, gw = run_forward(dims, tiny_params, x)
    ref = oracle.moe_forward(f64(x), _np_params(tiny_params), dims)
    same, _ = routing_check(gi, ref["routing"], dims)
    weights_check(gi, gw, ref["routing"], same)
    assert_close(f64(delta)[same], ref["y"][same], f"forward tiny T={T}")


def test_forward_timed_with_null_events(tiny_params):
    """moe_forward_timed records only the events it is given (the timed bench region passes the two
    around the up-projection): the result is moe_forward's bit for bit, and those two time a stage."""
    _say("moe_forward_timed with two of six events")
    from bench import HipEvents
    dims, T = synth.TINY, 300
    cd = cdims(dims)
    x = synth.make_x(dims, T, DEV, seed=61)
    layer = moe.MoELayer(cd, tiny_params)
    ws = moe.workspace(cd, T)
    d0, d1 = torch.empty_like(x), torch.empty_like(x)
    moe.moe_forward(cd, layer.weights, T, x, d0, None, None, ws)
    hev = HipEvents()
    try:
        evs = [None] * moe.MOE_FORWARD_EVENTS
        evs[2], evs[3] = hev.create(2)
        moe.moe_forward_timed(cd, layer.weights, T, x, d1, None, None, ws, evs)
        torch.cuda.synchronize()
        assert hev.ms(evs[2], evs[3]) > 0.0
    finally:
        hev.close()
    assert torch.equal(d0, d1)


def test_forward_is_deterministic(tiny_params):
    _say("moe_forward determinism")
    dims = synth.TINY
    x = synth.make_x(dims, 1000, DEV, seed=4)
    a, *_ = run_forward(dims, tiny_params, x)
    b, *_ = run_forward(dims, tiny_params, x)
    assert torch.equal(a, b)


def test_forward_zero_tokens(tiny_params):
    _say("moe_forward T=0")
    layer = moe.MoELayer(cdims(synth.TINY), tiny_params)
    out = layer(torch.empty((0, synth.TINY.d_model), dtype=torch.bfloat16, device=DEV))
    assert out.shape == (0, synth.TINY.d_model)


def test_forward_all_tokens_on_one_group(tiny_params):
    _say("moe_forward hot group (multi-tile experts)")
    dims = synth.TINY
    p = dict(tiny_params)
    bias = torch.full((dims.n_experts,), -5.0, device=DEV)
    bias[:4] = 5.0                                   # group 0 wins for every token
    bias[4:8] = 4.0                                  # group 1 second
    p["gate_b"] = bias
    T = 300                                          # experts 0..7 get ~300 rows: three 128-row tiles
    x = synth.make_x(dims, T, DEV, seed=6)
    delta, gi, _ = run_forward(dims, p, x)
    assert set(np.unique(gi).tolist()) <= set(range(8))
    ref = oracle.moe_forward(f64(x), _np_params(p), dims)
    same, _ = routing_check(gi, ref["routing"], dims)
    assert_close(f64(delta)[same], ref["y"][same], "forward hot group")


def test_forward_nan_token_is_contained(tiny_params):
    _say("moe_forward NaN input")
    dims = synth.TINY
    x = synth.make_x(dims, 40, DEV, seed=7)
    clean, gi_clean, _ = run_forward(dims, tiny_params, x)
    xn = x.clone()
    xn[3, 17] = float("nan")
    dirty, gi, _ = run_forward(dims, tiny_params, xn)
    assert np.all((gi >= 0) & (gi < dims.n_experts))
    for t in range(40):
        assert len(set(gi[t].tolist())) == dims.topk
    keep = [t for t in range(40) if t != 3]
    assert torch.equal(dirty[keep], clean[keep])
    assert np.array_equal(gi[keep], gi_clean[keep])


# ----------------------------------------------------------------------------
# fused forward, full shape (d 7168, 256 experts, top-8 of 4 groups)
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def full_params():
    _say("generating full-shape weights on the GPU")
    p = synth.make_block(synth.FULL, "normal:0.01", DEV, seed=1)
    torch.cuda.synchronize()
    return p


def _full_case(params, bias, T, seed, n_sample):
    dims = synth.FULL
    p = dict(params)
    p["gate_b"] = bias
    x = synth.make_x(dims, T, DEV, seed=seed)
    delta, gi, gw = run_forward(dims, p, x)
    again, gi2, gw2 = run_forward(dims, p, x)        # no atomics, fixed sum orders: bit-identical
    assert torch.equal(delta, again) and np.array_equal(gi, gi2) and np.array_equal(gw, gw2)
    hv = HostView(p)
    xv = f64(x)
    r = oracle.gate(xv, hv["gate_w"], hv["gate_b"], dims)
    same, ndiff = routing_check(gi, r, dims)
    print(f"[parity] T={T}: {ndiff} near-tie tokens route differently", flush=True)
    weights_check(gi, gw, r, same)
    tok = sample_tokens(gi, dims.n_experts, T, n_sample, seed, bf16=p["w1"].dtype == torch.bfloat16)
    ref = oracle.moe_forward(xv, hv, dims, tokens=tok, routing=r, idx=gi)
    return assert_close(f64(delta)[tok], ref["y"], f"forward full T={T} ({tok.size} sampled tokens)")


# ----------------------------------------------------------------------------
# dense MLP (the blocks before the MoE blocks)
# ----------------------------------------------------------------------------

def run_mlp(p, x, d, inter):
    T = x.shape[0]
    out = torch.full((T, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    ws = moe.mlp_workspace(d, inter, T)
    mlp = moe.experts_struct(*(p[k] for k in ("w1", "w3", "w2", "s1", "s3", "s2")))
    moe.moe_mlp(d, inter, T, mlp, x, out, ws)
    torch.cuda.synchronize()
    return out


def _mlp_ref(pn, xv):
    return oracle.expert_ffn(xv, pn["w1"][0], pn["s1"][0], pn["w3"][0], pn["s3"][0], pn["w2"][0], pn["s2"][0])


@pytest.mark.parametrize("T", [1, 37, 128, 129, 300])
def test_mlp_tiny(T):
    d, inter = 512, 384
    _say(f"moe_mlp d={d} inter={inter} T={T}")
    p = synth.mlp_weights(d, inter, DEV, seed=7)
    x = synth.make_x(synth.Dims(d, 1, 1, 1, 1, inter), T, DEV, seed=70 + T)
    got = f64(run_mlp(p, x, d, inter))
    assert_rows_close(got, _mlp_ref(_np_params(p), f64(x)), f"mlp tiny T={T}")


@pytest.mark.parametrize("T", [1, 37, 64, 128, 129, 300])
def test_mlp_split_k(T):
    # 17 K blocks into the up-projection and 13 into the down-projection, 13
    # h blocks and a ragged last pair of output blocks: at these batch sizes
    # both projections are split over K in slices of 4 blocks, the last one a
    # single block, with 32-row tiles (T <= 128) and 128-row tiles
    d, inter = 2176, 1664
    _say(f"moe_mlp split K d={d} inter={inter} T={T}")
    p = synth.mlp_weights(d, inter, DEV, seed=9)
    x = synth.make_x(synth.Dims(d, 1, 1, 1, 1, inter), T, DEV, seed=90 + T)
    first = run_mlp(p, x, d, inter)
    got = f64(first)
    assert_rows_close(got, _mlp_ref(_np_params(p), f64(x)), f"mlp split K T={T}")
    # the slices' partial sums are added in a fixed order: a second call is bit-identical
    assert torch.equal(run_mlp(p, x, d, inter), first)


@pytest.mark.parametrize("T", [37, 100, 129])
def test_mlp_stream_k(T):
    # inter 18432 (144 h blocks) over d = 3584 (28 K blocks): 144 or 288 items do not fill
    # rounds of 256 workgroups, so the up-projection runs stream-K (runs of 16 or 32 K
    # blocks that cross h blocks; one tile at T = 37, two 64-row tiles at T = 100, 128-row
    # tiles with a one-row tail at T = 129)
    d, inter = 3584, 18432
    _say(f"moe_mlp stream K d={d} inter={inter} T={T}")
    p = synth.mlp_weights(d, inter, DEV, seed=11)
    x = synth.make_x(synth.Dims(d, 1, 1, 1, 1, inter), T, DEV, seed=110 + T)
    first = run_mlp(p, x, d, inter)
    assert_rows_close(f64(first), _mlp_ref(_np_params(p), f64(x)), f"mlp stream K T={T}")
    # each (tile, h block) sums its runs' partial planes in a fixed order
    assert torch.equal(run_mlp(p, x, d, inter), first)


@pytest.mark.slow
@pytest.mark.parametrize("T", [64, 1000])
def test_mlp_full_width_sampled_rows(T):
    # d = 7168 (the pages' model width); inter = 18432, a width the pages leave open, chosen
    # because it needs 144 K blocks in the down-projection
    d, inter = 7168, 18432
    _say(f"moe_mlp d={d} inter={inter} T={T}")
    p = synth.mlp_weights(d, inter, DEV, seed=8)
    x = synth.make_x(synth.Dims(d, 1, 1, 1, 1, inter), T, DEV, seed=80 + T)
    got = f64(run_mlp(p, x, d, inter))
    # first, last and tile-edge rows plus a seeded sample
    rng = np.random.default_rng(T)
    edges = [0, 1, 15, 16, 127, 128, T - 1]
    rows = np.unique(np.concatenate([[r for r in edges if r < T], rng.choice(T, min(T, 16), replace=False)]))
    ref = _mlp_ref(_np_params(p), f64(x)[rows])
    assert_rows_close(got[rows], ref, f"mlp full-width T={T}")
    assert np.isfinite(got).all()


# ----------------------------------------------------------------------------
# bf16 expert weights (Linear layers without scales, no activation quantisation)
# ----------------------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny_params_bf16():
    return synth.make_block(synth.TINY, "normal:0.1", DEV, seed=0, weights="bf16")


def _bf16_expert(pn, pre, i):
    return [oracle.bf16_weight(pn[pre + k][i]) for k in ("w1", "w3", "w2")]


@pytest.mark.parametrize("T", [37, 300])
def test_grouped_ffn_bf16_forced_routing_tiny(tiny_params_bf16, T):
    _say(f"moe_grouped_ffn_bf16 tiny T={T}")
    dims, p = synth.TINY, tiny_params_bf16
    x = synth.make_x(dims, T, DEV, seed=40 + T)
    K, E, d = dims.topk, dims.n_experts, dims.d_model
    pn = _np_params(p)
    xv = f64(x)
    r = oracle.gate(xv, pn["gate_w"], pn["gate_b"], dims)
    perm = oracle.permute(r["idx"], E)
    rows_tok = np.concatenate([perm["row_token"], np.arange(T)]).astype(np.int32)
    cd = cdims(dims)
    out = torch.zeros((T * K + T, d), dtype=torch.bfloat16, device=DEV)
    routed = moe.experts_struct_bf16(p["w1"], p["w3"], p["w2"])
    shared = moe.experts_struct_bf16(p["sh_w1"], p["sh_w3"], p["sh_w2"])
    moe.moe_grouped_ffn_bf16(cd, T, routed, shared, torch.from_numpy(perm["offsets"]).int().to(DEV),
                             torch.from_numpy(rows_tok).to(DEV), x, out, moe.workspace(cd, T))
    torch.cuda.synchronize()
    got = f64(out)
    ref = np.zeros_like(got)
    off = perm["offsets"]
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            ref[rows] = oracle.expert_ffn_bf16(xv[perm["row_token"][rows]], *_bf16_expert(pn, "", e))
    ref[T * K:] = oracle.expert_ffn_bf16(xv, *_bf16_expert(pn, "sh_", 0))
    assert_rows_close(got, ref, f"grouped_ffn_bf16 tiny T={T}")


@pytest.mark.parametrize("T,counts", [
    (100, [0, 1, 15, 16, 17, 31, 32, 33, 48, 49, 63, 65, 30, 0, 0, 0]),
    (300, [0, 1, 15, 16, 17, 31, 33, 63, 127, 129, 144, 160, 193, 200, 71, 0]),
])
def test_grouped_ffn_bf16_tile_edges(tiny_params_bf16, T, counts):
    _say(f"moe_grouped_ffn_bf16 tile edges T={T}")
    dims, p = synth.TINY, tiny_params_bf16
    K, E, d = dims.topk, dims.n_experts, dims.d_model
    idx = _idx_with_counts(np.array(counts), T, K)
    x = synth.make_x(dims, T, DEV, seed=95 + T)
    pn = _np_params(p)
    xv = f64(x)
    perm = oracle.permute(idx, E)
    rows_tok = np.concatenate([perm["row_token"], np.arange(T)]).astype(np.int32)
    cd = cdims(dims)
    out = torch.zeros((T * K + T, d), dtype=torch.bfloat16, device=DEV)
    routed = moe.experts_struct_bf16(p["w1"], p["w3"], p["w2"])
    shared = moe.experts_struct_bf16(p["sh_w1"], p["sh_w3"], p["sh_w2"])
    moe.moe_grouped_ffn_bf16(cd, T, routed, shared, torch.from_numpy(perm["offsets"]).int().to(DEV),
                             torch.from_numpy(rows_tok).to(DEV), x, out, moe.workspace(cd, T))
    torch.cuda.synchronize()
    got = f64(out)
    ref = np.zeros_like(got)
    off = perm["offsets"]
    for e in range(E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size:
            ref[rows] = oracle.expert_ffn_bf16(xv[perm["row_token"][rows]], *_bf16_expert(pn, "", e))
    ref[T * K:] = oracle.expert_ffn_bf16(xv, *_bf16_expert(pn, "sh_", 0))
    assert_rows_close(got, ref, f"grouped_ffn_bf16 tile edges T={T}")


@pytest.mark.parametrize("T", [1, 37, 64, 1000])
def test_forward_bf16_tiny(tiny_params_bf16, T):
    _say(f"moe_forward_bf16 tiny T={T}")
    dims = synth.TINY
    x = synth.make_x(dims, T, DEV, seed=50 + T)
    delta, gi, gw = run_forward(dims, tiny_params_bf16, x)
    ref = oracle.moe_forward(f64(x), _np_params(tiny_params_bf16), dims)
    same, _ = routing_check(gi, ref["routing"], dims)
    weights_check(gi, gw, ref["routing"], same)
    assert_close(f64(delta)[same], ref["y"][same], f"forward_bf16 tiny T={T}")


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [64, 4096])
def test_forward_bf16_full_shape(T):
    _say(f"moe_forward_bf16 full shape T={T}")
    p = synth.make_block(synth.FULL, "normal:0.01", DEV, seed=6, weights="bf16")
    torch.cuda.synchronize()
    _full_case(p, p["gate_b"], T, seed=110 + T, n_sample=64)
    del p
    torch.cuda.empty_cache()


# ----------------------------------------------------------------------------
# one rank's share of an expert-parallel layer (experts [b, e) + fp32 partial)
# ----------------------------------------------------------------------------

def _shard_weights(p, b, e, with_shared):
    keys = ("w1", "w3", "w2", "s1", "s3", "s2")
    routed = moe.experts_struct(*(p[k][b:e] for k in keys))      # views: the rank holds experts b..e-1
    shared = moe.experts_struct(*(p["sh_" + k] for k in keys)) if with_shared else moe.moe_experts()
    return moe.moe_weights(p["gate_w"].data_ptr(), p["gate_b"].data_ptr(), routed, shared)


def _oracle_partial(pv, xv, tok, idx, w, b, e, with_shared):
    """sum over the token's choices with expert in [b, e), ascending expert, of w * expert(x) (+ shared)."""
    y = np.zeros((tok.size, xv.shape[1]))
    for ex in range(b, e):
        rows, ks = np.nonzero(idx[tok] == ex)
        if rows.size:
            o = oracle.expert_ffn(xv[tok[rows]], *(np.asarray(pv[k][ex]) for k in ("w1", "s1", "w3", "s3", "w2", "s2")))
            y[rows] += o * w[tok[rows], ks][:, None].astype(np.float64)
    if with_shared:
        y += oracle.expert_ffn(xv[tok], *(np.asarray(pv["sh_" + k][0]) for k in ("w1", "s1", "w3", "s3", "w2", "s2")))
    return y


def test_shards_sum_to_the_layer_tiny(tiny_params):
    _say("moe_forward_shard tiny: 4 shards of 4 experts, T=300")
    dims, p = synth.TINY, tiny_params
    T = 300
    cd = cdims(dims)
    x = synth.make_x(dims, T, DEV, seed=60)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=DEV)
    ws = moe.workspace(cd, T)
    moe.moe_gate(cd, T, x, p["gate_w"], p["gate_b"], idx, w, ws)
    delta = torch.empty_like(x)
    moe.moe_forward(cd, moe.MoELayer(cd, p).weights, T, x, delta, None, None, ws)
    pn, xv = _np_params(p), f64(x)
    gi, gw = idx.cpu().numpy().astype(np.int64), w.cpu().numpy()
    total = np.zeros((T, dims.d_model))
    for s in range(4):
        b, e = 4 * s, 4 * s + 4
        y = torch.full((T, dims.d_model), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_forward_shard(cd, _shard_weights(p, b, e, s == 0), T, b, e, s == 0, x, idx, w, y, ws)
        torch.cuda.synchronize()
        got = y.cpu().numpy().astype(np.float64)
        assert np.isfinite(got).all()
        ref = _oracle_partial(pn, xv, np.arange(T), gi, gw, b, e, s == 0)
        assert_close(got, ref, f"shard {s} (experts {b}..{e - 1})")
        total += got
    # the cross-rank sum, rounded once, is the layer output (up to the fp32 order of the sum)
    d_sum = torch.from_numpy(total).float().to(torch.bfloat16).double().numpy()
    d_full = f64(delta)
    ulp = np.abs(d_full) * 2.0 ** -7 + 1e-30
    assert (np.abs(d_sum - d_full) <= ulp).mean() > 0.999
    assert_close(total, oracle.moe_forward(xv, pn, dims, idx=gi)["y"], "sum of shards vs oracle layer")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_shard_one_group_full_shape(full_params):
    """One rank holding one group of 32 experts (group 1), no shared expert, T=4096."""
    _say("moe_forward_shard full shape, experts 32..63, T=4096")
    dims, p = synth.FULL, full_params
    T, b, e = 4096, 32, 64
    cd = cdims(dims)
    x = synth.make_x(dims, T, DEV, seed=120)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=DEV)
    ws = moe.workspace(cd, T)
    moe.moe_gate(cd, T, x, p["gate_w"], p["gate_b"], idx, w, ws)
    y = torch.full((T, dims.d_model), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_forward_shard(cd, _shard_weights(p, b, e, False), T, b, e, False, x, idx, w, y, ws)
    torch.cuda.synchronize()
    gi, gw = idx.cpu().numpy().astype(np.int64), w.cpu().numpy()
    got = y.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    hit = np.nonzero(((gi >= b) & (gi < e)).any(1))[0]
    miss = np.nonzero(~((gi >= b) & (gi < e)).any(1))[0]
    assert np.all(got[miss] == 0.0)                        # tokens routed elsewhere get nothing
    rng = np.random.default_rng(7)
    tok = np.sort(rng.choice(hit, min(10, hit.size), replace=False))
    ref = _oracle_partial(HostView(p), f64(x), tok, gi, gw, b, e, False)
    assert_close(got[tok], ref, f"shard experts {b}..{e - 1} full shape ({tok.size} sampled tokens)")
