"""Plain fp64 CPU oracle of one DeepSeek-V3.2-Exp MoE layer forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package entry's smoke
check and the benchmark's CPU-baseline leg, never by the product path.  It
shares no code, table or helper with the HIP library.

What it computes, and where each step comes from (page titles as printed):

* "DeepSeek-V3.2-Exp · MoE update", moe-forward excerpt: tokens are
  flattened to [N, d]; the gate returns routing weights and expert indices;
  an fp32 accumulator y; a count of the tokens per selected expert; a loop
  over experts in ascending id
  that gathers the tokens routed to the expert in ascending token order,
  runs the expert and adds its output times the router weight; then the
  shared expert's output for every token; finally y is cast back to the
  input dtype (the page's output expression).
* "DeepSeek-V3.2-Exp · Add shared output", formula: the update is the routed
  sum plus the shared-expert output.
* "DeepSeek-V3.2-Exp · Gate projection", expert excerpt: an expert applies
  w1 and w3, takes SiLU of the first times the second in float32, casts the
  product back to the input dtype and applies w2; Linear excerpt: weights
  are [out, in], FP8 weights carry one float32 scale per 128x128 block, wider
  (bf16) weights carry none, no bias.
* "DeepSeek-V3.2-Exp · MoE update", rmsnorm excerpt: with a residual, the
  residual is added in float32, the sum (cast back) becomes the new residual,
  and the output is the gain times the sum divided by the root of its mean
  square plus eps, eps 1e-6.
* "MoE transformer block", parameter accounting table: the MoE of one block
  has 11,320,164,608 parameters; with 256 routed + 1 shared expert of shape
  7168->2048->7168 the remainder is exactly a 256x7168 router weight plus a
  256-element router bias.

The pages show only the gate's call site.  The router used here is the plain
reading of the layer's description: sigmoid scores of x.Wg^T, a per-expert
bias added for selection only, groups scored by the sum of their two largest
biased scores, the top topk_groups groups kept (the others excluded), the
top topk biased scores among kept experts selected, and weights equal to
the unbiased scores of the selected experts normalised to sum 1 and multiplied
by route_scale.  Ties go to the lower group / expert index.

The pages also omit how an FP8 Linear multiplies (the Linear excerpt skips
that part of the file).  The reading used here: the bf16 activation row is
quantised per 128-element block to e4m3 with scale = block amax / 448 (the
same rule the weights use), the block products are summed exactly, and the
Linear output is rounded to bfloat16 (it returns the activation dtype, which
is why the expert converts it to float32 before SiLU).

Every floating-point step is evaluated in float64.  The Linear layers multiply
the dequantised operands (e4m3 value times its float32 scale, exact in
float64) with BLAS matrix products: each product of two dequantised values
has up to 56 significant bits and is rounded to float64's 53, and the
summation order is BLAS's own, so a Linear output carries a relative error
of about 1e-16 before it is rounded to bfloat16.  The roundings the pages
place (bf16 Linear outputs, bf16 h, float32 scale arithmetic of the
quantiser) are applied explicitly.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

BLOCK = 128          # "Gate projection", Linear excerpt: the FP8 scale block edge
E4M3_MAX = 448.0     # largest finite e4m3fn value (OCP 8-bit floating point, E4M3)
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127
RMS_EPS = 1e-6       # "MoE update", rmsnorm excerpt: eps default

__all__ = [
    "BLOCK", "E4M3_MAX", "RMS_EPS",
    "e4m3_table", "e4m3_decode", "e4m3_encode", "bf16_round", "bf16_bits_to_f64",
    "f64_to_bf16_bits", "dequant_weight", "quant_act", "dequant_act", "gate", "permute",
    "silu", "expert_ffn", "expert_ffn_bf16", "bf16_weight", "combine", "moe_forward", "add_rmsnorm", "param_count",
    "weights_for",
]


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def e4m3_table() -> np.ndarray:
    """Value of each of the 256 e4m3fn codes (OCP OFP8 E4M3: sign, 4-bit exponent
    with bias 7, 3-bit mantissa, subnormals m * 2^-9, S.1111.111 is NaN, no inf)."""
    c = np.arange(256)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = sign * mag
    v[(e == 15) & (m == 7)] = np.nan
    return v


_E4M3 = e4m3_table()
_E4M3_POS = _E4M3[:127]  # codes 0x00..0x7E: 0 .. 448, strictly increasing
_E4M3_T = torch.from_numpy(_E4M3)


def e4m3_decode(codes) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(v) -> np.ndarray:
    """Nearest e4m3fn code, ties to even, magnitudes above 448 saturate to 448.

    The sign is kept (a negative value that rounds to zero gives 0x80).  NaN
    gives 0x7F.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = f * 2^ex, f in [0.5, 1)
    e = np.maximum(ex - 1, -6)               # binade; subnormals share the 2^-6 binade spacing
    step = np.ldexp(1.0, e - 3)              # 3 stored mantissa bits
    with np.errstate(invalid="ignore"):
        r = np.rint(a / step) * step         # rint rounds half to even
        r = np.minimum(r, E4M3_MAX)
    code = np.searchsorted(_E4M3_POS, np.nan_to_num(r, nan=0.0)).astype(np.uint8)
    code = code | (np.signbit(v).astype(np.uint8) << 7)
    code[np.isnan(v)] = 0x7F
    return code


def bf16_round(v) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126)
    step = np.ldexp(1.0, e - 7)              # 7 stored mantissa bits
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.rint(a / step) * step
        r = np.where(r > BF16_MAX, np.inf, r)
    return np.copysign(r, v)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v) -> np.ndarray:
    """Bits of values that are already bfloat16 numbers (e.g. bf16_round output)."""
    return (np.asarray(v, dtype=np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# FP8 block quantisation ("Gate projection", Linear excerpt)
# --------------------------------------------------------------------------

def dequant_weight(codes, scale) -> np.ndarray:
    """W[o, i] = e4m3(codes[o, i]) * scale[o // 128, i // 128], float64 [out, in].

    (The table lookup and the scaling run as multi-threaded torch CPU ops;
    both are exact in float64.)
    """
    codes = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
    scale = np.asarray(scale, dtype=np.float32).astype(np.float64)
    O, I = codes.shape
    assert O % BLOCK == 0 and I % BLOCK == 0, "the oracle takes whole 128x128 blocks"
    w = torch.take(_E4M3_T, torch.from_numpy(codes).long()).view(O // BLOCK, BLOCK, I // BLOCK, BLOCK)
    w = w * torch.from_numpy(scale)[:, None, :, None]
    return w.reshape(O, I).numpy()


def quant_act(v):
    """Per-row, per-128-block e4m3 quantisation of bfloat16 activations.

    For each block: a = max |v_j| (exact); scale = fl32(a / 448); codes =
    e4m3(fl32(v_j / scale)) with float32 correctly rounded division; an
    all-zero block gets scale 1.  Returns (codes uint8 [n, L], scale float32
    [n, L/128]).
    """
    v = np.asarray(v, dtype=np.float64)
    n, L = v.shape
    assert L % BLOCK == 0
    blk = v.reshape(n, L // BLOCK, BLOCK)
    with np.errstate(invalid="ignore"):
        amax = np.abs(blk).max(axis=-1)
    scale = (amax.astype(np.float32) / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = blk.astype(np.float32) / scale[..., None]
    codes = e4m3_encode(ratio.astype(np.float64)).reshape(n, L)
    return codes, scale


def dequant_act(codes, scale) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    n, L = codes.shape
    v = e4m3_decode(codes).reshape(n, L // BLOCK, BLOCK)
    v = v * np.asarray(scale, dtype=np.float32).astype(np.float64)[..., None]
    return v.reshape(n, L)


# --------------------------------------------------------------------------
# Router ("MoE update", moe-forward excerpt: the gate call, which returns the
# routing weights and the expert indices)
# --------------------------------------------------------------------------

def gate(x, gate_w, gate_b, dims) -> Dict[str, np.ndarray]:
    """Group-limited top-k sigmoid router with a selection-only bias.

    x: float64 [T, d] (bf16 values); gate_w: float32 [E, d]; gate_b: float32 [E].
    Returns idx [T, K] (descending biased score), w [T, K] float64, the scores,
    group scores, and the two selection margins used to flag near-ties:
    expert_gap = K-th minus (K+1)-th biased score among kept experts,
    group_gap  = TG-th minus (TG+1)-th group score.
    """
    x = np.asarray(x, dtype=np.float64)
    T = x.shape[0]
    E, G, TG, K = dims.n_experts, dims.n_groups, dims.topk_groups, dims.topk
    epg = E // G
    rows = np.arange(T)[:, None]

    z = x @ np.asarray(gate_w, dtype=np.float32).astype(np.float64).T     # logits [T, E]
    s = 1.0 / (1.0 + np.exp(-z))                                          # sigmoid scores
    b = s + np.asarray(gate_b, dtype=np.float32).astype(np.float64)       # biased scores

    two_largest = np.sort(b.reshape(T, G, epg), axis=-1)[:, :, -2:]
    gscore = two_largest.sum(axis=-1)                                     # [T, G]
    gorder = np.argsort(-gscore, axis=-1, kind="stable")                  # ties: lower group first
    keep = np.zeros((T, G), dtype=bool)
    keep[rows, gorder[:, :TG]] = True
    b_kept = np.where(np.repeat(keep, epg, axis=1), b, -np.inf)           # other groups excluded

    eorder = np.argsort(-b_kept, axis=-1, kind="stable")                  # ties: lower expert first
    idx = eorder[:, :K]
    sel = s[rows, idx]
    w = sel / sel.sum(axis=-1, keepdims=True) * dims.route_scale

    b_sorted = b_kept[rows, eorder]
    expert_gap = b_sorted[:, K - 1] - b_sorted[:, K] if K < E else np.full(T, np.inf)
    g_sorted = gscore[rows, gorder]
    group_gap = g_sorted[:, TG - 1] - g_sorted[:, TG] if TG < G else np.full(T, np.inf)
    return {"idx": idx.astype(np.int64), "w": w, "z": z, "s": s, "b": b,
            "group_score": gscore, "groups": np.sort(gorder[:, :TG], axis=-1),
            "expert_gap": expert_gap, "group_gap": group_gap}


def weights_for(s_rows, idx, route_scale) -> np.ndarray:
    """Router weights for a given selection: unbiased scores normalised, times route_scale."""
    sel = np.take_along_axis(s_rows, idx, axis=-1)
    return sel / sel.sum(axis=-1, keepdims=True) * route_scale


# --------------------------------------------------------------------------
# Token counting and expert-contiguous order ("MoE update", moe-forward excerpt:
# a count per expert, then each expert's tokens gathered in ascending order)
# --------------------------------------------------------------------------

def permute(idx, n_experts: int) -> Dict[str, np.ndarray]:
    """counts[e]; rows of expert e are the tokens choosing e in ascending order,
    experts laid out in ascending id.  pair_row[t, k] is the row of (t, k)."""
    idx = np.asarray(idx, dtype=np.int64)
    T, K = idx.shape
    counts = np.bincount(idx.ravel(), minlength=n_experts)
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_token = np.empty(T * K, dtype=np.int64)
    pair_row = np.empty((T, K), dtype=np.int64)
    for e in range(n_experts):
        t, k = np.nonzero(idx == e)          # row-major: ascending token
        pos = offsets[e] + np.arange(t.size)
        row_token[pos] = t
        pair_row[t, k] = pos
    return {"counts": counts, "offsets": offsets, "row_token": row_token, "pair_row": pair_row}


# --------------------------------------------------------------------------
# Expert ("Gate projection", expert excerpt)
# --------------------------------------------------------------------------

def silu(v):
    return v / (1.0 + np.exp(-v))


def expert_ffn(x_rows, w1, s1, w3, s3, w2, s2, full: bool = False):
    """w2((silu(w1 x) * w3 x)) with FP8 Linear layers, for bf16 rows x [n, d].

    g = bf16(Q(x) . W1^T), u = bf16(Q(x) . W3^T), h = bf16(silu(g) * u),
    o = bf16(Q(h) . W2^T); Q is quant_act, W the block-dequantised weight.
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    xq, xs = quant_act(x_rows)
    xd = dequant_act(xq, xs)
    with np.errstate(over="ignore"):
        g = bf16_round(xd @ dequant_weight(w1, s1).T)
        u = bf16_round(xd @ dequant_weight(w3, s3).T)
        h = bf16_round(silu(g) * u)
    hq, hs = quant_act(h)
    o = bf16_round(dequant_act(hq, hs) @ dequant_weight(w2, s2).T)
    if full:
        return {"o": o, "g": g, "u": u, "h": h, "xq": xq, "xs": xs, "hq": hq, "hs": hs}
    return o


def expert_ffn_bf16(x_rows, w1, w3, w2, full: bool = False):
    """The same expert with bf16 weights: w2((silu(w1 x) * w3 x)) without scales.

    "Gate projection", Linear excerpt: a weight whose elements are wider
    than one byte gets no scale parameter.  The Linear forward is not on the
    pages; read plainly, it multiplies the bf16 activation by the bf16
    weight [out, in] (no activation quantisation) and returns bf16:
    g = bf16(x . W1^T), u = bf16(x . W3^T), h = bf16(silu(g) * u),
    o = bf16(h . W2^T), each dot product exact in float64 before its rounding.
    """
    x_rows = np.asarray(x_rows, dtype=np.float64)
    W1 = np.asarray(w1, dtype=np.float64)
    W3 = np.asarray(w3, dtype=np.float64)
    W2 = np.asarray(w2, dtype=np.float64)
    with np.errstate(over="ignore"):
        g = bf16_round(x_rows @ W1.T)
        u = bf16_round(x_rows @ W3.T)
        h = bf16_round(silu(g) * u)
        o = bf16_round(h @ W2.T)
    if full:
        return {"o": o, "g": g, "u": u, "h": h}
    return o


def _expert(params, e: Optional[int]):
    if e is None:  # the shared expert
        names = ("sh_w1", "sh_s1", "sh_w3", "sh_s3", "sh_w2", "sh_s2")
        return [np.asarray(params[n][0]) for n in names]
    names = ("w1", "s1", "w3", "s3", "w2", "s2")
    return [np.asarray(params[n][e]) for n in names]


def _run_expert(params, e: Optional[int], x_rows):
    """Expert e (None: the shared one) on x_rows, FP8 or bf16 by the weights it holds."""
    if "s1" not in params:  # bf16 weights: no scales
        pre, i = ("sh_", 0) if e is None else ("", e)
        return expert_ffn_bf16(x_rows, bf16_weight(params[pre + "w1"][i]), bf16_weight(params[pre + "w3"][i]),
                               bf16_weight(params[pre + "w2"][i]))
    return expert_ffn(x_rows, *_expert(params, e))


def bf16_weight(w) -> np.ndarray:
    """A bf16 weight given as raw bit patterns (uint16 / int16) or as values -> float64."""
    a = np.asarray(w)
    if a.dtype in (np.uint16, np.int16):
        return bf16_bits_to_f64(a.view(np.uint16))
    return a.astype(np.float64)


# --------------------------------------------------------------------------
# Layer forward ("MoE update" moe-forward excerpt + output expression;
# "Add shared output" formula)
# --------------------------------------------------------------------------

def combine(idx, w, outs, shared) -> np.ndarray:
    """Router-weighted sum of a token's expert outputs plus the shared output.

    idx [n, K] selected experts, w [n, K] router weights, outs [n, K, d] the
    output of expert idx[t, k] on token t, shared [n, d] the shared expert's
    output.  y[t] = sum over the K choices, taken in ascending expert id, of
    w[t, k] * outs[t, k], then + shared[t] ("MoE update", moe-forward excerpt:
    experts are visited in ascending id into a float32 accumulator and the
    shared expert's output comes last; here float64).
    """
    idx = np.asarray(idx, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    n, K = idx.shape
    y = np.zeros((n, outs.shape[-1]), dtype=np.float64)
    order = np.argsort(idx, axis=1, kind="stable")          # each token's choices by ascending expert id
    at = np.arange(n)
    for j in range(K):
        k = order[:, j]
        y += w[at, k][:, None] * outs[at, k]
    return y + np.asarray(shared, dtype=np.float64)


def moe_forward(x, params, dims, tokens: Optional[Sequence[int]] = None,
                idx: Optional[np.ndarray] = None, routing: Optional[Dict] = None) -> Dict[str, np.ndarray]:
    """Forward of one MoE layer on bf16 x [T, d] (given as float64 values).

    params: mapping with gate_w [E, d], gate_b [E] and per-expert indexable
    w1/s1/w3/s3/w2/s2 (routed, [E, ...]) and sh_w1/... (shared, [1, ...]);
    without s1/s3/s2 the expert weights are bf16 (expert_ffn_bf16).
    tokens: evaluate the expert part only for these tokens (routing is always
    computed for all).  idx: force this selection [T, K] (weights then come
    from the oracle's own scores).  routing: a gate() result to reuse.
    Returns routing, y (float64, unrounded) and delta = bf16(y) for the
    evaluated tokens.

    The update of token t is the sum over its K choices, taken in ascending
    expert id, of the router weight times the expert's output on x[t], plus
    the shared expert's output on x[t] ("MoE update", moe-forward excerpt:
    experts are visited in ascending id and the shared expert comes last;
    "Add shared output", formula).  The expert outputs are evaluated one
    expert at a time over all rows that chose it, so each expert's weights
    are dequantised once.
    """
    x = np.asarray(x, dtype=np.float64)
    T, d = x.shape
    r = routing if routing is not None else gate(x, params["gate_w"], params["gate_b"], dims)
    sel_idx = r["idx"] if idx is None else np.asarray(idx, dtype=np.int64)
    w_all = r["w"] if idx is None else weights_for(r["s"], sel_idx, dims.route_scale)
    tok = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    n, K = tok.size, sel_idx.shape[1]

    choice = sel_idx[tok]                                   # [n, K] expert of each choice
    outs = np.zeros((n, K, d), dtype=np.float64)            # expert output of each (token, choice)
    for e in np.unique(choice):
        tt, kk = np.nonzero(choice == e)
        outs[tt, kk] = _run_expert(params, int(e), x[tok[tt]])
    y = combine(choice, w_all[tok], outs, _run_expert(params, None, x[tok]))
    return {"idx": sel_idx, "w": w_all, "routing": r, "tokens": tok, "y": y, "delta": bf16_round(y)}


def add_rmsnorm(x, residual, gain, eps: float = RMS_EPS):
    """Fused residual add + RMSNorm ("MoE update", rmsnorm excerpt, residual branch).

    r = x + residual; new residual = bf16(r); out = bf16(gain * r / sqrt(mean(r^2) + eps)).
    """
    r = np.asarray(x, dtype=np.float64) + np.asarray(residual, dtype=np.float64)
    res_new = bf16_round(r)
    var = np.mean(r * r, axis=-1, keepdims=True)
    g = np.asarray(gain, dtype=np.float32).astype(np.float64)
    out = bf16_round(g * (r / np.sqrt(var + eps)))
    return out, res_new


def param_count(dims, n_shared: int = 1) -> int:
    """Learned elements of one MoE layer: (routed + shared) SwiGLU experts of three
    d x inter matrices, the router weight [E, d] and the router bias [E]
    ("MoE transformer block", parameter accounting table; FP8 scales are not counted)."""
    return (dims.n_experts + n_shared) * 3 * dims.d_model * dims.inter + dims.n_experts * dims.d_model + dims.n_experts
