"""GPU parity of the layer forward on the benchmark's own workload instances.

Each case builds its inputs with ``synth.make_workload(name)``: the seeds,
token counts and bias laws that ``bench.py`` times.  It runs the HIP forward,
checks the routing of every token against the oracle (near-tie rule), and
compares the outputs of a token sample with the oracle, evaluated in one call
per layer so that each expert is dequantised once:

* decode (64 tokens): every token;
* prefill (4,096 tokens), skewed (16,384) and the prefill instance at 500,
  1,000 and 65,536 tokens: the first and the last permuted row of every touched expert, both
  sides of every boundary between the FFN tiles of an expert that is cut into
  several tiles (and of the shared expert's tiles), and seeded random tokens up
  to at least 256;
* the stack of four blocks (8,192 tokens): the GPU chain runs free.  Each
  block's new residual and normalised rows are compared bit for bit, on every
  token, with the oracle's RMSNorm of that block's GPU inputs, and the block's
  update with the oracle's layer on the GPU's normalised rows (teacher
  forcing) on a token sample.  The oracle's own four-block chain is evaluated
  on the same tokens and its distance to the free-running GPU chain is
  printed; it is not bounded.

The layer is token-wise ("DeepSeek-V3.2-Exp · MoE update": the forward
flattens the tokens and treats each row on its own), so a token's output
depends only on that token and sampled tokens can be evaluated alone.  The
oracle is evaluated on the GPU's selection: a token that routes differently
must first pass the near-tie rule of the routing check (margin below 1e-5 at
the last kept group or expert, and a valid selection), and its output is
then compared with the oracle run on that selection.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_bias_amd as moe
import oracle
import synth
from _helpers import (NEAR_TIE, HostView, assert_close, cdims, f64, metrics, routing_check, sample_tokens,
                      weights_check)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def _near_ties(r) -> int:
    return int(((r["expert_gap"] < NEAR_TIE) | (r["group_gap"] < NEAR_TIE)).sum())


def _check_layer(name, dims, params, x, delta, gi, gw, tok):
    """Routing of every token, then the outputs of tokens `tok` against the oracle."""
    hv = HostView(params)
    xv = f64(x)
    r = oracle.gate(xv, hv["gate_w"], hv["gate_b"], dims)
    same, ndiff = routing_check(gi, r, dims)
    weights_check(gi, gw, r, same)
    ref = oracle.moe_forward(xv, hv, dims, tokens=tok, routing=r, idx=gi)
    mx, mean = metrics(f64(delta)[tok], ref["y"])
    print(f"[parity] {name}: {tok.size} of {x.shape[0]} tokens compared, max|d|/rms={mx:.3e} mean rel={mean:.3e}; "
          f"near-tie tokens (margin < {NEAR_TIE:g}) {_near_ties(r)}, routed differently {ndiff}", flush=True)
    assert_close(f64(delta)[tok], ref["y"], name)
    return r


def _forward(dims, params, x):
    T = x.shape[0]
    layer = moe.MoELayer(cdims(dims), params)
    gi = torch.empty((T, dims.topk), dtype=torch.int32, device=DEV)
    gw = torch.empty((T, dims.topk), dtype=torch.float32, device=DEV)
    delta = layer(x, idx=gi, w=gw)
    torch.cuda.synchronize()
    return delta, gi.cpu().numpy().astype(np.int64), gw.cpu().numpy()


@pytest.mark.timeout(900)
def test_decode_workload_every_token():
    _say("decode workload (T=64, bench instance): every token")
    data = synth.make_workload("decode", device=DEV)
    dims, p, x = data["dims"], data["blocks"][0], data["x"]
    delta, gi, gw = _forward(dims, p, x)
    again, gi2, _ = _forward(dims, p, x)
    assert torch.equal(delta, again) and np.array_equal(gi, gi2)
    _check_layer("decode T=64", dims, p, x, delta, gi, gw, np.arange(x.shape[0]))


@pytest.fixture(scope="module")
def prefill_block():
    data = synth.make_workload("prefill", device=DEV, tokens=1)
    torch.cuda.synchronize()
    yield data["blocks"][0]
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_prefill_workload_sampled_tokens(prefill_block):
    _say("prefill workload (T=4096, bench instance)")
    w = synth.WORKLOADS["prefill"]
    x = synth.make_x(w.dims, w.tokens, DEV, w.seed)
    delta, gi, gw = _forward(w.dims, prefill_block, x)
    tok = sample_tokens(gi, w.dims.n_experts, w.tokens, 256, seed=1)
    _check_layer("prefill T=4096", w.dims, prefill_block, x, delta, gi, gw, tok)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T", [500, 1000])
def test_prefill_weights_at_mid_batch_sizes(prefill_block, T):
    """The prefill instance's weights at batch sizes between decode and
    prefill: 32-row tiles at 500 tokens (experts of ~16 rows, some cut in
    two), 64-row tiles at 1000."""
    _say(f"prefill weights at T={T}")
    w = synth.WORKLOADS["prefill"]
    x = synth.make_x(w.dims, T, DEV, w.seed + T)
    delta, gi, gw = _forward(w.dims, prefill_block, x)
    tok = sample_tokens(gi, w.dims.n_experts, T, 256, seed=4)
    _check_layer(f"prefill weights T={T}", w.dims, prefill_block, x, delta, gi, gw, tok)


@pytest.mark.timeout(1200)
def test_prefill_weights_at_65536_tokens(prefill_block):
    """The prefill instance's weights at 65,536 tokens (524,288 routed rows,
    ~16 tiles per expert): grids, tile counts and row offsets far beyond those
    of the named workloads."""
    _say("prefill weights at T=65536")
    w = synth.WORKLOADS["prefill"]
    x = synth.make_x(w.dims, 65536, DEV, w.seed)
    delta, gi, gw = _forward(w.dims, prefill_block, x)
    tok = sample_tokens(gi, w.dims.n_experts, 65536, 256, seed=2)
    _check_layer("prefill weights T=65536", w.dims, prefill_block, x, delta, gi, gw, tok)


@pytest.mark.timeout(900)
def test_skewed_workload_sampled_tokens():
    _say("skewed workload (T=16384, Zipf-like bias, bench instance)")
    data = synth.make_workload("skewed", device=DEV)
    dims, p, x = data["dims"], data["blocks"][0], data["x"]
    delta, gi, gw = _forward(dims, p, x)
    tok = sample_tokens(gi, dims.n_experts, x.shape[0], 256, seed=3)
    _check_layer("skewed T=16384", dims, p, x, delta, gi, gw, tok)
    del data, p
    torch.cuda.empty_cache()


@pytest.mark.timeout(1500)
def test_stack4_workload_teacher_forced():
    _say("stack of 4 blocks (T=8192, bench instance): free-running GPU chain, teacher-forced oracle")
    data = synth.make_workload("stack4", device=DEV)
    dims, T, d = data["dims"], data["tokens"], data["dims"].d_model
    cd = cdims(dims)
    res = data["residual"].clone()
    src = data["x"]
    h = torch.empty_like(src)
    tok = None
    chain_x, chain_res = None, None               # the oracle's own chain on the sampled tokens
    for b in range(4):
        gain = data["gains"][b]
        x_in, res_in = f64(src), f64(res)         # this block's GPU inputs
        moe.moe_add_rmsnorm(d, T, src, res, gain, 1e-6, h)
        gi = torch.empty((T, dims.topk), dtype=torch.int32, device=DEV)
        gw = torch.empty((T, dims.topk), dtype=torch.float32, device=DEV)
        out = moe.MoELayer(cd, data["blocks"][b])(h, idx=gi, w=gw)
        torch.cuda.synchronize()
        g = gain.cpu().numpy()
        # a0 on every token: the oracle's RMSNorm of the GPU's block inputs
        hn_ref, res_ref = oracle.add_rmsnorm(x_in, res_in, g)
        assert np.array_equal(f64(res), res_ref), f"block {b}: new residual differs"
        hv_rows = f64(h)
        n_bad = int((hv_rows != hn_ref).sum())
        assert n_bad == 0, f"block {b}: {n_bad} normalised values differ"
        del x_in, res_in, hn_ref, res_ref
        # routing of every token on the GPU's normalised rows
        hv = HostView(data["blocks"][b])
        gi_np, gw_np = gi.cpu().numpy().astype(np.int64), gw.cpu().numpy()
        r = oracle.gate(hv_rows, hv["gate_w"], hv["gate_b"], dims)
        same, ndiff = routing_check(gi_np, r, dims)
        weights_check(gi_np, gw_np, r, same)
        if tok is None:
            tok = sample_tokens(gi_np, dims.n_experts, T, 96, seed=4)[::4]   # every 4th: >= 64 tokens
            assert tok.size >= 64
            chain_x, chain_res = f64(data["x"])[tok], f64(data["residual"])[tok]
        # one oracle call: the teacher-forced rows (GPU inputs, GPU selection)
        # and the oracle's own chain (its own inputs and selection) side by side
        chain_hn, chain_res = oracle.add_rmsnorm(chain_x, chain_res, g)
        chain_idx = oracle.gate(chain_hn, hv["gate_w"], hv["gate_b"], dims)["idx"]
        xs = np.concatenate([hv_rows[tok], chain_hn])
        ref = oracle.moe_forward(xs, hv, dims, idx=np.concatenate([gi_np[tok], chain_idx]))
        n = tok.size
        got = f64(out)[tok]
        mx, mean = metrics(got, ref["y"][:n])
        print(f"[parity] stack block {b} (T={T}, teacher-forced): {n} tokens compared, max|d|/rms={mx:.3e} "
              f"mean rel={mean:.3e}; near-tie tokens {_near_ties(r)}, routed differently {ndiff}", flush=True)
        assert_close(got, ref["y"][:n], f"stack block {b} teacher-forced")
        chain_x = ref["delta"][n:]
        del hv_rows, r
        src = out
    cmx, cmean = metrics(f64(src)[tok], chain_x)
    print(f"[report] free-running 4-block GPU chain vs the oracle's own chain on {tok.size} tokens: "
          f"max|d|/rms={cmx:.3e} mean rel={cmean:.3e}", flush=True)
    assert np.all(np.isfinite(f64(src)))
    del data
    torch.cuda.empty_cache()
