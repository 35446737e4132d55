"""Shared pieces of the GPU parity tests: dims conversion, host views of
device parameters for the oracle, routing comparison with the near-tie rule,
and the output metrics with their bounds.

Bounds (from the layer's accuracy target): routing sets are bit-exact except
tokens whose oracle margin at the K-th expert or the topk_groups-th group is
below 1e-5; on the other tokens max|gpu - ref| / rms(ref) <= 2e-2 and
mean|gpu - ref| / mean|ref| <= 5e-3, with ref the oracle's unrounded float64
output.
"""
from __future__ import annotations

import numpy as np
import torch

import mixture_experts_ffn_bias_amd as moe
import oracle

NEAR_TIE = 1e-5
MAX_REL = 2e-2
MEAN_REL = 5e-3


def cdims(d) -> "moe.moe_dims":
    return moe.make_dims(d.d_model, d.n_experts, d.n_groups, d.topk_groups, d.topk, d.inter, d.route_scale)


def f64(t: torch.Tensor) -> np.ndarray:
    """bf16 / fp32 tensor (any device) -> float64 numpy values (exact)."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def to_numpy(t):
    """Host copy of a tensor; bf16 comes back as its uint16 bit patterns."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class HostView:
    """Read-only mapping over device parameters that copies one expert at a time."""

    class _Rows:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, e):
            return to_numpy(self.t[e])

    def __init__(self, params):
        self.p = params
        self.small = {k: params[k].cpu().numpy() for k in ("gate_w", "gate_b")}

    def __contains__(self, k):
        return k in self.p

    def __getitem__(self, k):
        if k in self.small:
            return self.small[k]
        return HostView._Rows(self.p[k])


def routing_check(gpu_idx: np.ndarray, r: dict, dims, tol: float = NEAR_TIE):
    """Compare GPU routing with the oracle's.  Returns (same_mask, n_near_tie_diffs).

    A differing token must be a near-tie, and the GPU's choice must still be a
    valid selection: K distinct experts in at most topk_groups groups, whose
    total biased score is within K*tol of the oracle's best.
    """
    T, K = gpu_idx.shape
    ref = np.sort(r["idx"], axis=1)
    got = np.sort(gpu_idx, axis=1)
    same = np.all(ref == got, axis=1)
    near = (r["expert_gap"] < tol) | (r["group_gap"] < tol)
    bad = np.flatnonzero(~same & ~near)
    assert bad.size == 0, f"{bad.size} tokens route differently without a near-tie, e.g. token {bad[:5]}"
    epg = dims.n_experts // dims.n_groups
    for t in np.flatnonzero(~same):
        sel = gpu_idx[t]
        assert len(set(sel.tolist())) == K and np.all((sel >= 0) & (sel < dims.n_experts))
        assert len(set((sel // epg).tolist())) <= dims.topk_groups
        b = r["b"][t]
        assert b[sel].sum() >= b[r["idx"][t]].sum() - K * tol
    return same, int((~same).sum())


def weights_check(gpu_idx, gpu_w, r, same, rtol=2e-5):
    for t in np.flatnonzero(same)[:4096]:
        want = dict(zip(r["idx"][t].tolist(), r["w"][t].tolist()))
        got = dict(zip(gpu_idx[t].tolist(), gpu_w[t].tolist()))
        for e, v in want.items():
            assert abs(got[e] - v) <= rtol * abs(v), (t, e, got[e], v)


def metrics(gpu: np.ndarray, ref: np.ndarray):
    diff = np.abs(gpu - ref)
    rms = np.sqrt(np.mean(ref * ref))
    return float(diff.max() / rms), float(diff.mean() / np.abs(ref).mean())


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str):
    mx, mean = metrics(gpu, ref)
    print(f"[parity] {what}: max|d|/rms={mx:.3e} mean rel={mean:.3e}", flush=True)
    assert mx <= MAX_REL and mean <= MEAN_REL, f"{what}: max {mx:.3e} (<= {MAX_REL}), mean {mean:.3e} (<= {MEAN_REL})"
    return mx, mean


def assert_rows_close(gpu: np.ndarray, ref: np.ndarray, what: str, within_ulp: float = 0.99):
    """Bound for single expert rows (bf16 values on both sides).

    Rows are compared before the router-weighted combine averages them, so a
    single bf16 rounding flip on a large element is already several percent
    of the rms; the bound is therefore element-wise: at least `within_ulp` of
    the elements within one bf16 ulp of the oracle, and mean |d| / mean |ref|
    <= 5e-3.
    """
    ulp = np.maximum(np.abs(ref), 1e-30) * 2.0 ** -7
    frac = float(np.mean(np.abs(gpu - ref) <= ulp))
    _, mean = metrics(gpu, ref)
    print(f"[parity] {what}: within 1 ulp {frac:.5f}, mean rel={mean:.3e}", flush=True)
    assert frac >= within_ulp and mean <= MEAN_REL, f"{what}: within-ulp {frac:.4f}, mean {mean:.3e}"


def tile_rows(T: int, bf16: bool = False) -> int:
    """Rows per FFN tile of the routed layer for a batch of T tokens (the
    library's choice): with e4m3 expert weights 32 up to 768 tokens, 64 up to
    1280, then 128; with bf16 weights 32 up to 128 tokens, then 128."""
    if bf16:
        return 32 if T <= 128 else 128
    return 32 if T <= 768 else (64 if T <= 1280 else 128)


def tile_starts(count: int, T: int, bf16: bool = False):
    """First rows (relative to the expert's first row) of the FFN tiles after
    the first, for an expert with `count` permuted rows in a batch of T tokens:
    an expert with more rows than one tile holds is cut into ceil(count / rows)
    tiles of equal size, rounded up to 16 rows (the library's tile plan)."""
    nt_rows = tile_rows(T, bf16)
    n = -(-count // nt_rows)
    if n <= 1:
        return []
    rt = min(nt_rows, -(-(-(-count // n)) // 16) * 16)
    return [j * rt for j in range(1, n)]


def sample_tokens(idx: np.ndarray, n_experts: int, T: int, at_least: int, seed: int,
                  bf16: bool = False) -> np.ndarray:
    """First and last permuted row of every touched expert, both sides of every
    tile boundary of multi-tile experts and of the shared expert, plus seeded
    random tokens up to `at_least`."""
    perm = oracle.permute(idx, n_experts)
    off, rt = perm["offsets"], perm["row_token"]
    pick = set()
    for e in range(n_experts):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        pick.update((int(rt[lo]), int(rt[hi - 1])))
        for b in tile_starts(hi - lo, T, bf16):
            pick.update((int(rt[lo + b - 1]), int(rt[lo + b])))
    nt_rows = tile_rows(T, bf16)
    for j in range(1, -(-T // nt_rows)):          # the shared expert's tiles: rows in token order
        pick.update((j * nt_rows - 1, j * nt_rows))
    rng = np.random.default_rng(seed)
    rest = np.setdiff1d(np.arange(T), np.fromiter(pick, dtype=np.int64))
    need = max(0, min(at_least - len(pick), rest.size))
    pick.update(rng.choice(rest, need, replace=False).tolist())
    return np.array(sorted(pick), dtype=np.int64)
