"""GPU parity of the single-launch forward (moe_forward_fused) against the CPU
oracle, and its agreement with the multi-launch moe_forward.

Inputs are seeded synthetic tensors from ``synth``; expected values come from
``oracle`` on the same inputs.  Every call is followed by a status check: a
wait inside the launch that gave up (MOE_ERR_STALLED) fails the test.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_bias_amd as moe
import oracle
import synth
from _helpers import HostView, assert_close, cdims, f64, routing_check, to_numpy, weights_check

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _np_params(p):
    return {k: to_numpy(v) for k, v in p.items()}


@pytest.fixture(scope="module")
def tiny_params():
    return synth.make_block(synth.TINY, "normal:0.1", DEV, seed=0)


def run_fused(layer, x):
    T = x.shape[0]
    K = layer.dims.topk
    idx = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    delta = layer.forward_fused(x, idx=idx, w=w)
    assert moe.moe_forward_fused_status(layer._fused_ws) == 0, "a wait of the single launch gave up"
    return delta, idx.cpu().numpy().astype(np.int64), w.cpu().numpy()


def check_against_oracle(dims, p, x, delta, gi, gw, what):
    ref = oracle.moe_forward(f64(x), _np_params(p), dims)
    same, _ = routing_check(gi, ref["routing"], dims)
    weights_check(gi, gw, ref["routing"], same)
    return assert_close(f64(delta)[same], ref["y"][same], what)


@pytest.mark.parametrize("T", [1, 7, 37, 64])
def test_fused_tiny(tiny_params, T):
    _say(f"moe_forward_fused tiny T={T}")
    dims = synth.TINY
    layer = moe.MoELayer(cdims(dims), tiny_params)
    x = synth.make_x(dims, T, DEV, seed=40 + T)
    delta, gi, gw = run_fused(layer, x)
    check_against_oracle(dims, tiny_params, x, delta, gi, gw, f"fused tiny T={T}")


def test_fused_calls_in_a_row_reuse_the_workspace(tiny_params):
    _say("moe_forward_fused: T=64, 5, 64, 33 on one workspace")
    dims = synth.TINY
    layer = moe.MoELayer(cdims(dims), tiny_params)
    for i, T in enumerate((64, 5, 64, 33)):
        x = synth.make_x(dims, T, DEV, seed=60 + i)
        delta, gi, gw = run_fused(layer, x)
        check_against_oracle(dims, tiny_params, x, delta, gi, gw, f"fused call {i} T={T}")


def test_fused_is_deterministic(tiny_params):
    _say("moe_forward_fused determinism")
    dims = synth.TINY
    layer = moe.MoELayer(cdims(dims), tiny_params)
    x = synth.make_x(dims, 64, DEV, seed=5)
    a, ia, wa = run_fused(layer, x)
    b, ib, wb = run_fused(layer, x)
    assert torch.equal(a, b) and np.array_equal(ia, ib) and np.array_equal(wa, wb)


def test_fused_matches_multi_launch(tiny_params):
    _say("moe_forward_fused vs moe_forward, tiny T=64")
    dims = synth.TINY
    layer = moe.MoELayer(cdims(dims), tiny_params)
    x = synth.make_x(dims, 64, DEV, seed=8)
    fused, fi, fw = run_fused(layer, x)
    idx = torch.empty((64, dims.topk), dtype=torch.int32, device=DEV)
    w = torch.empty((64, dims.topk), dtype=torch.float32, device=DEV)
    multi = layer(x, idx=idx, w=w)
    torch.cuda.synchronize()
    mi = idx.cpu().numpy().astype(np.int64)
    same = np.all(np.sort(fi, 1) == np.sort(mi, 1), axis=1)
    assert same.sum() >= 62                          # only near-ties may route differently
    # same routing: the FFN is the same code; only the router's last fp32 bits may differ
    np.testing.assert_allclose(fw[same], w.cpu().numpy()[same], rtol=1e-5, atol=1e-6)
    assert_close(f64(fused)[same], f64(multi)[same], "fused vs multi-launch")
    assert np.mean(f64(fused)[same] == f64(multi)[same]) > 0.99    # differences are last-bit flips


def test_fused_hot_group_multi_tile_experts(tiny_params):
    _say("moe_forward_fused hot group: experts with two 32-row tiles")
    dims = synth.TINY
    p = dict(tiny_params)
    bias = torch.full((dims.n_experts,), -5.0, device=DEV)
    bias[:4] = 5.0                                   # group 0 wins for every token
    bias[4:8] = 4.0                                  # group 1 second
    p["gate_b"] = bias
    layer = moe.MoELayer(cdims(dims), p)
    x = synth.make_x(dims, 64, DEV, seed=9)
    delta, gi, gw = run_fused(layer, x)
    assert set(np.unique(gi).tolist()) <= set(range(8))
    check_against_oracle(dims, p, x, delta, gi, gw, "fused hot group")


# int32 index of the "a wait gave up" word in the workspace's control block (kernels.h: DEC_CTL_STALLED)
CTL_STALLED = 192


def test_fused_reports_a_stall_and_recovers(tiny_params):
    """A stall forced from the host: with the stall word set before the call, every bounded
    wait gives up at its first poll, each workgroup still runs to its end, and the last one
    resets the counts.  The status call reports MOE_ERR_STALLED; the next call on the same
    workspace is clean and gives the same bits as before."""
    _say("moe_forward_fused: stall word set from the host")
    dims = synth.TINY
    layer = moe.MoELayer(cdims(dims), tiny_params)
    x = synth.make_x(dims, 64, DEV, seed=12)
    good, gi, gw = run_fused(layer, x)
    ctl = layer._fused_ws[:4096].view(torch.int32)
    ctl[CTL_STALLED] = 1
    torch.cuda.synchronize()
    layer.forward_fused(x)
    assert moe.moe_forward_fused_status(layer._fused_ws) == moe.MOE_ERR_STALLED
    c = ctl.cpu().numpy()
    assert c[CTL_STALLED] == 0 and np.count_nonzero(c) == 1        # only the status word is left set
    again, gi2, gw2 = run_fused(layer, x)                           # asserts status OK
    assert torch.equal(good, again) and np.array_equal(gi, gi2) and np.array_equal(gw, gw2)


def test_fused_rejects_more_than_64_tokens(tiny_params):
    layer = moe.MoELayer(cdims(synth.TINY), tiny_params)
    with pytest.raises(moe.MoeError):
        layer.forward_fused(synth.make_x(synth.TINY, 65, DEV, seed=1))


@pytest.fixture(scope="module")
def full_params():
    _say("generating full-shape weights on the GPU")
    p = synth.make_block(synth.FULL, "normal:0.01", DEV, seed=1)
    torch.cuda.synchronize()
    return p


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_fused_full_decode(full_params):
    _say("moe_forward_fused full shape T=64 (decode)")
    dims = synth.FULL
    p = dict(full_params)
    p["gate_b"] = 0.01 * torch.randn(256, generator=torch.Generator(device=DEV).manual_seed(11), device=DEV)
    layer = moe.MoELayer(cdims(dims), p)
    x = synth.make_x(dims, 64, DEV, seed=101)
    delta, gi, gw = run_fused(layer, x)
    hv = HostView(p)
    xv = f64(x)
    r = oracle.gate(xv, hv["gate_w"], hv["gate_b"], dims)
    same, ndiff = routing_check(gi, r, dims)
    print(f"[parity] fused T=64: {ndiff} near-tie tokens route differently", flush=True)
    weights_check(gi, gw, r, same)
    rng = np.random.default_rng(101)
    tok = np.array(sorted(rng.choice(64, 6, replace=False).tolist()))
    tok = tok[same[tok]]
    ref = oracle.moe_forward(xv, hv, dims, tokens=tok, routing=r)
    assert_close(f64(delta)[tok], ref["y"], f"fused full T=64 ({tok.size} sampled tokens)")
    # every token against the multi-launch path (same FFN code, same routing up to near-ties)
    multi = layer(x)
    torch.cuda.synchronize()
    assert_close(f64(delta)[same], f64(multi)[same], "fused vs multi-launch, full shape")
    assert np.mean(f64(delta)[same] == f64(multi)[same]) > 0.99
