"""The allocation-free forward (moe_forward_no_workspace) against moe_forward.

It runs the same kernels on the library's own per-GPU array instead of a
caller workspace, so its outputs must equal moe_forward's bit for bit.  Two
calls in a row, the second on a smaller batch (the array keeps the first
call's contents), on full-shape decode weights.
"""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_bias_amd as moe
import synth
from _helpers import cdims

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _run(fn, cd, layer, x, T, K):
    delta = torch.full_like(x, float("nan"))
    idx = torch.full((T, K), -1, dtype=torch.int32, device=DEV)
    w = torch.full((T, K), float("nan"), dtype=torch.float32, device=DEV)
    fn(delta, idx, w)
    torch.cuda.synchronize()
    return delta, idx, w


def test_no_workspace_forward_matches_moe_forward_on_two_calls():
    print("[case] moe_forward_no_workspace vs moe_forward, full-shape decode weights, T=64 then T=17", flush=True)
    data = synth.make_workload("decode", device=DEV)
    dims, p = data["dims"], data["blocks"][0]
    cd = cdims(dims)
    layer = moe.MoELayer(cd, p)
    K = dims.topk
    for T, seed in ((64, 1), (17, 5)):
        x = synth.make_x(dims, T, DEV, seed)
        ws = moe.workspace(cd, T)
        ref = _run(lambda d, i, w: moe.moe_forward(cd, layer.weights, T, x, d, i, w, ws), cd, layer, x, T, K)
        got = _run(lambda d, i, w: moe.moe_forward_no_workspace(cd, layer.weights, T, x, d, i, w), cd, layer, x, T, K)
        assert torch.equal(got[0], ref[0]), f"T={T}: update differs"
        assert torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[2]), f"T={T}: routing differs"
        assert torch.isfinite(got[0].float()).all()
        print(f"[parity] no-workspace forward T={T}: bit-identical to moe_forward", flush=True)


def test_no_workspace_forward_rejects_batches_beyond_its_array():
    dims = synth.FULL
    cd = cdims(dims)
    T = 4096
    assert moe.moe_workspace_size(cd, T) > moe.MOE_STATIC_WORKSPACE_BYTES
    x = torch.zeros((T, dims.d_model), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        moe.moe_forward_no_workspace(cd, moe.moe_weights(), T, x, x, None, None)
    assert e.value.code == -2
