"""C ABI checks that need no GPU: the library loads, exports every function
include/moe.h declares, and rejects bad arguments on the host before it
touches the device (each call below returns before any HIP call)."""
import ctypes
import os
import re

import pytest

import mixture_experts_ffn_bias_amd as moe
from mixture_experts_ffn_bias_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(moe.LIB_PATH), reason="libmoe.so not built")

FULL = dict(d_model=7168, n_experts=256, n_groups=8, topk_groups=4, topk=8, inter=2048, route_scale=2.5)
FAKE = 1 << 20          # a 256-byte aligned non-null address; never dereferenced on these paths


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(moe_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted(moe.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = moe.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert moe.status_string(0) == "ok"
    for c in (-1, -2, -3, -4, -5, -6):
        assert moe.status_string(c) not in ("ok", "unknown status")


def dims(**kw):
    d = dict(FULL)
    d.update(kw)
    return moe.make_dims(**d)


def ws_size(**kw):
    return moe.moe_workspace_size(dims(**kw), 64)


def test_workspace_size_full_shape_decode():
    n = ws_size()
    assert n > 64 * 7168 * 9 * 2            # at least the bf16 expert-output rows
    assert moe.moe_workspace_size(dims(), 0) >= 0


@pytest.mark.parametrize("bad", [
    dict(d_model=7000), dict(inter=2000), dict(n_experts=300), dict(n_experts=24, n_groups=8),
    dict(topk=33, topk_groups=8), dict(n_groups=128, n_experts=256),
])
def test_unsupported_dims_have_no_workspace(bad):
    assert ws_size(**bad) == 0


@pytest.mark.parametrize("bad", [
    dict(topk_groups=9), dict(topk=0), dict(n_experts=256, n_groups=7), dict(topk=130, topk_groups=4),
    dict(route_scale=float("inf")), dict(d_model=-128),
])
def test_invalid_dims_are_rejected(bad):
    rc = B.lib().moe_gate(ctypes.byref(dims(**bad)), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == -1


def test_unsupported_dims_code():
    rc = B.lib().moe_gate(ctypes.byref(dims(d_model=7000)), 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == -2


def test_null_dims_and_negative_tokens():
    L = B.lib()
    assert L.moe_gate(None, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_gate(ctypes.byref(dims()), -1, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1


def test_zero_tokens_is_a_noop_everywhere():
    L = B.lib()
    d = ctypes.byref(dims())
    assert L.moe_gate(d, 0, None, None, None, None, None, None, 0, None) == 0
    assert L.moe_permute(d, 0, None, None, None, None, None, None, None, None, None, 0, None) == 0
    assert L.moe_grouped_ffn(d, 0, None, None, None, None, None, None, None, None, 0, None) == 0
    assert L.moe_combine(d, 0, None, None, None, None, 1, None, None) == 0
    assert L.moe_forward(d, None, 0, None, None, None, None, None, 0, None) == 0
    assert L.moe_add_rmsnorm(7168, 0, None, None, None, 1e-6, None, None) == 0
    assert L.moe_mlp(7168, 18432, 0, None, None, None, None, 0, None) == 0
    assert L.moe_grouped_ffn_bf16(d, 0, None, None, None, None, None, None, None, 0, None) == 0
    assert L.moe_forward_bf16(d, None, 0, None, None, None, None, None, 0, None) == 0


def test_null_pointers_rejected():
    L = B.lib()
    d = ctypes.byref(dims())
    assert L.moe_gate(d, 4, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_combine(d, 4, FAKE, FAKE, None, FAKE, 1, FAKE, None) == -1
    ex = moe.moe_experts(FAKE, FAKE, None, FAKE, FAKE, FAKE)
    assert L.moe_grouped_ffn(d, 4, ctypes.byref(ex), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_forward(d, None, 4, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == -1


def test_workspace_too_small():
    L = B.lib()
    d = dims()
    need = moe.moe_workspace_size(d, 64)
    assert L.moe_gate(ctypes.byref(d), 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == -3
    assert L.moe_gate(ctypes.byref(d), 64, FAKE, FAKE, FAKE, FAKE, FAKE, None, need, None) == -3


def test_misaligned_pointers():
    L = B.lib()
    d = ctypes.byref(dims())
    assert L.moe_gate(d, 4, FAKE + 2, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -4
    assert L.moe_gate(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 16, 1 << 30, None) == -4
    ex = moe.moe_experts(FAKE + 8, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_grouped_ffn(d, 4, ctypes.byref(ex), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -4
    assert L.moe_add_rmsnorm(7168, 4, FAKE + 2, FAKE, FAKE, 1e-6, FAKE, None) == -4


def test_rmsnorm_argument_checks():
    L = B.lib()
    assert L.moe_add_rmsnorm(7000, 4, FAKE, FAKE, FAKE, 1e-6, FAKE, None) == -2
    assert L.moe_add_rmsnorm(32768, 4, FAKE, FAKE, FAKE, 1e-6, FAKE, None) == -2
    assert L.moe_add_rmsnorm(7168, 4, FAKE, FAKE, FAKE, -1.0, FAKE, None) == -1
    assert L.moe_add_rmsnorm(0, 4, FAKE, FAKE, FAKE, 1e-6, FAKE, None) == -1


def test_python_binding_raises_on_error_codes():
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_gate(dims(topk_groups=9), 4, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert ei.value.code == -1


def test_mlp_argument_checks():
    L = B.lib()
    ex = moe.moe_experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    need = moe.moe_mlp_workspace_size(7168, 18432, 64)
    # xq + xs + h, at least
    assert need >= 64 * 7168 + 64 * 56 * 4 + 64 * 18432
    assert moe.moe_mlp_workspace_size(7168, 18432 + 64, 64) == 0
    assert moe.moe_mlp_workspace_size(7168, 32768 + 128, 64) == 0
    assert moe.moe_mlp_workspace_size(0, 2048, 64) == 0
    assert L.moe_mlp(7168, 18432 + 64, 64, ctypes.byref(ex), FAKE, FAKE, FAKE, 1 << 30, None) == -2
    assert L.moe_mlp(-128, 2048, 64, ctypes.byref(ex), FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_mlp(7168, 2048, -1, ctypes.byref(ex), FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_mlp(7168, 2048, 64, None, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_mlp(7168, 2048, 64, ctypes.byref(ex), None, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_mlp(7168, 2048, 64, ctypes.byref(ex), FAKE + 2, FAKE, FAKE, 1 << 30, None) == -4
    assert L.moe_mlp(7168, 2048, 64, ctypes.byref(ex), FAKE, FAKE, FAKE + 16, 1 << 30, None) == -4
    small = moe.moe_mlp_workspace_size(7168, 2048, 64)
    assert L.moe_mlp(7168, 2048, 64, ctypes.byref(ex), FAKE, FAKE, FAKE, small - 1, None) == -3
    assert L.moe_mlp(7168, 2048, 64, ctypes.byref(ex), FAKE, FAKE, None, small, None) == -3


def test_bf16_entry_points_reject_bad_arguments():
    L = B.lib()
    d = ctypes.byref(dims())
    ex = moe.moe_experts_bf16(FAKE, FAKE, FAKE)
    assert L.moe_grouped_ffn_bf16(d, 4, None, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_grouped_ffn_bf16(d, 4, ctypes.byref(moe.moe_experts_bf16(FAKE, None, FAKE)), None, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, 1 << 30, None) == -1
    assert L.moe_grouped_ffn_bf16(d, 4, ctypes.byref(moe.moe_experts_bf16(FAKE + 2, FAKE, FAKE)), None, FAKE, FAKE,
                                  FAKE, FAKE, FAKE, 1 << 30, None) == -4
    assert L.moe_grouped_ffn_bf16(d, 4, ctypes.byref(ex), None, FAKE, FAKE, FAKE + 2, FAKE, FAKE, 1 << 30, None) == -4
    assert L.moe_grouped_ffn_bf16(d, 4, ctypes.byref(ex), None, FAKE, FAKE, FAKE, FAKE, None, 1 << 30, None) == -3
    w = moe.moe_weights_bf16(FAKE, FAKE, ex, ex)
    assert L.moe_forward_bf16(d, None, 4, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == -1
    assert L.moe_forward_bf16(d, ctypes.byref(w), 4, None, FAKE, None, None, FAKE, 1 << 30, None) == -1
    assert L.moe_forward_bf16(d, ctypes.byref(w), 4, FAKE, FAKE, None, None, FAKE, 16, None) == -3
    assert L.moe_forward_bf16_timed(d, ctypes.byref(w), 4, FAKE, FAKE, None, None, FAKE, 1 << 30, None, None) == -1
    bad = moe.moe_weights_bf16(FAKE, FAKE, moe.moe_experts_bf16(FAKE, FAKE, FAKE + 8), ex)
    assert L.moe_forward_bf16(d, ctypes.byref(bad), 4, FAKE, FAKE, None, None, FAKE, 1 << 30, None) == -4
    # permute: xq and xs must be given together or not at all
    assert L.moe_permute(d, 4, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 1 << 30, None) == -1


def test_shard_argument_checks():
    L = B.lib()
    d = ctypes.byref(dims())
    ex = moe.moe_experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    w = moe.moe_weights(FAKE, FAKE, ex, ex)
    call = lambda b, e, sh, x=FAKE, idx=FAKE, y=FAKE, ws=1 << 30, T=4, wt=ctypes.byref(w): L.moe_forward_shard(
        d, wt, T, b, e, sh, x, idx, FAKE, y, FAKE if ws else None, ws, None)
    assert call(0, 0, 1) == -1           # empty range
    assert call(32, 16, 1) == -1         # reversed range
    assert call(-1, 16, 1) == -1
    assert call(0, 257, 1) == -1         # past the last expert
    assert call(0, 32, 1, T=0) == 0      # no tokens: no-op
    assert call(0, 32, 1, idx=None) == -1
    assert call(0, 32, 1, wt=None) == -1
    assert call(0, 32, 1, y=FAKE + 4) == -4
    assert call(0, 32, 1, ws=0) == -3
    noshared = moe.moe_weights(FAKE, FAKE, ex, moe.moe_experts(None, None, None, None, None, None))
    assert call(0, 32, 1, wt=ctypes.byref(noshared)) == -1   # the shared expert is required with with_shared


def test_fused_workspace_sizes():
    d = dims()
    assert moe.moe_forward_fused_workspace_size(d, 0) == 0
    assert moe.moe_forward_fused_workspace_size(d, 65) == 0          # single launch: at most 64 tokens
    assert moe.moe_forward_fused_workspace_size(d, -1) == 0
    small, full = moe.moe_forward_fused_workspace_size(d, 1), moe.moe_forward_fused_workspace_size(d, 64)
    assert 4096 < small < full
    assert full > 64 * 7168 * 9 * 2                                   # the bf16 expert-output rows
    assert moe.moe_forward_fused_workspace_size(dims(d_model=7000), 8) == 0


def test_fused_argument_checks():
    L = B.lib()
    d = ctypes.byref(dims())
    ex = moe.moe_experts(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    w = moe.moe_weights(FAKE, FAKE, ex, ex)
    need = moe.moe_forward_fused_workspace_size(dims(), 16)
    call = lambda T=16, wt=ctypes.byref(w), x=FAKE, out=FAKE, ws=FAKE, n=need: L.moe_forward_fused(
        d, wt, T, x, out, None, None, ws, n, None)
    assert call(T=0) == 0                # no tokens: no-op
    assert call(T=65) == -2              # beyond the single-launch batch
    assert call(T=-1) == -1
    assert call(wt=None) == -1
    assert call(x=None) == -1
    assert call(out=FAKE + 2) == -4
    assert call(ws=FAKE + 64) == -4
    assert call(n=need - 1) == -3
    assert call(ws=None) == -3
    nobias = moe.moe_weights(FAKE, None, ex, ex)
    assert call(wt=ctypes.byref(nobias)) == -1
    noshared = moe.moe_weights(FAKE, FAKE, ex, moe.moe_experts(None, None, None, None, None, None))
    assert call(wt=ctypes.byref(noshared)) == -1
    assert L.moe_forward_fused_status(None, None) == -1


def test_no_workspace_forward_argument_checks():
    # checked on the host before the device array is looked up or anything runs
    L = moe.lib()
    w = B.moe_weights()
    assert L.moe_forward_no_workspace(None, ctypes.byref(w), 4, FAKE, FAKE, None, None, None) == -1
    assert L.moe_forward_no_workspace(ctypes.byref(dims()), ctypes.byref(w), -1, FAKE, FAKE, None, None, None) == -1
    assert L.moe_forward_no_workspace(ctypes.byref(dims()), ctypes.byref(w), 0, FAKE, FAKE, None, None, None) == 0
    big = 1
    while moe.moe_workspace_size(dims(), big) <= moe.MOE_STATIC_WORKSPACE_BYTES:
        big *= 2
    assert L.moe_forward_no_workspace(ctypes.byref(dims()), ctypes.byref(w), big, FAKE, FAKE, None, None, None) == -2
    assert moe.moe_workspace_size(dims(), 64) <= moe.MOE_STATIC_WORKSPACE_BYTES
