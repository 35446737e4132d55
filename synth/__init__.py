"""Seeded synthetic inputs for the DeepSeek-V3.2-Exp MoE layer.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the CPU oracle and the HIP path consume exactly the
bytes produced here, so a parity check compares the two on identical inputs.

Shapes follow the pages: the MoE forward takes x [tokens, d] and returns a
tensor of the same shape ("DeepSeek-V3.2-Exp · MoE update", output shape);
every expert is a SwiGLU MLP whose three Linear layers hold FP8 weights
[out, in] with one float32 scale per 128x128 block ("Gate projection",
Linear excerpt).  Expert weights are drawn in float32 from N(0, 1/in) (a
variance, i.e. fan-in scaling) and quantised per 128x128 block with
scale = block amax / 448, then stored as e4m3fn codes (uint8) plus the scale.

The recipe of each named workload (seed, bias law, token count) is in
``WORKLOADS``; all randomness comes from ``torch.Generator`` seeded with the
workload seed plus a per-tensor tag, on the device the tensors are made on.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import torch

E4M3_MAX = 448.0
BLOCK = 128


@dataclasses.dataclass(frozen=True)
class Dims:
    d_model: int
    n_experts: int
    n_groups: int
    topk_groups: int
    topk: int
    inter: int
    route_scale: float = 2.5

    @property
    def experts_per_group(self) -> int:
        return self.n_experts // self.n_groups


FULL = Dims(d_model=7168, n_experts=256, n_groups=8, topk_groups=4, topk=8, inter=2048)
TINY = Dims(d_model=512, n_experts=16, n_groups=4, topk_groups=2, topk=4, inter=128)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    tokens: int
    bias: str            # "normal:<sigma>", "zero", "zipf"
    seed: int
    blocks: int = 1      # >1: stacked blocks with fused residual-add RMSNorm in front
    gain_sigma: float = 0.0


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", TINY, 64, "normal:0.1", seed=0),
    "decode": Workload("decode", FULL, 64, "normal:0.01", seed=1),
    "prefill": Workload("prefill", FULL, 4096, "zero", seed=2),
    "skewed": Workload("skewed", FULL, 16384, "zipf", seed=3),
    "stack4": Workload("stack4", FULL, 8192, "normal:0.01", seed=4, blocks=4, gain_sigma=0.02),
}


def _gen(device, seed: int, tag: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + tag * 7919 + 17) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _normal(shape, std: float, device, seed: int, tag: int) -> torch.Tensor:
    g = _gen(device, seed, tag)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def quantize_blocks_e4m3(w: torch.Tensor):
    """Store a float32 [..., out, in] weight as e4m3fn codes + float32 [..., out/128, in/128] scales.

    scale = amax of the 128x128 block / 448 (a zero block gets scale 1).
    Used only to *produce* FP8 weights from the float32 draw.
    """
    *lead, o, i = w.shape
    assert o % BLOCK == 0 and i % BLOCK == 0
    b = w.reshape(*lead, o // BLOCK, BLOCK, i // BLOCK, BLOCK)
    amax = b.abs().amax(dim=(-3, -1))
    scale = amax / E4M3_MAX
    scale = torch.where(amax == 0, torch.ones_like(scale), scale)
    q = (b / scale[..., :, None, :, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, o, i)
    return codes.contiguous(), scale.contiguous()


def expert_weights(dims: Dims, n: int, device, seed: int, tag0: int) -> Dict[str, torch.Tensor]:
    """n SwiGLU experts: w1, w3 [n, inter, d]; w2 [n, d, inter] (+ s1, s3, s2 scales)."""
    d, I = dims.d_model, dims.inter
    out = {
        "w1": torch.empty((n, I, d), dtype=torch.uint8, device=device),
        "w3": torch.empty((n, I, d), dtype=torch.uint8, device=device),
        "w2": torch.empty((n, d, I), dtype=torch.uint8, device=device),
        "s1": torch.empty((n, I // BLOCK, d // BLOCK), dtype=torch.float32, device=device),
        "s3": torch.empty((n, I // BLOCK, d // BLOCK), dtype=torch.float32, device=device),
        "s2": torch.empty((n, d // BLOCK, I // BLOCK), dtype=torch.float32, device=device),
    }
    for e in range(n):  # one expert at a time keeps the float32 temporaries small
        for j, (wn, sn, shape, fan_in) in enumerate(
            (("w1", "s1", (I, d), d), ("w3", "s3", (I, d), d), ("w2", "s2", (d, I), I))
        ):
            w = _normal(shape, math.sqrt(1.0 / fan_in), device, seed, tag0 + 3 * e + j)
            q, s = quantize_blocks_e4m3(w)
            out[wn][e].copy_(q)
            out[sn][e].copy_(s)
            del w, q, s
    return out


def expert_weights_bf16(dims: Dims, n: int, device, seed: int, tag0: int) -> Dict[str, torch.Tensor]:
    """n SwiGLU experts with bf16 weights (no scales): w1, w3 [n, inter, d]; w2 [n, d, inter].

    Same normal laws (and seeds) as expert_weights, rounded to bf16 instead of block-quantised.
    """
    d, I = dims.d_model, dims.inter
    out = {
        "w1": torch.empty((n, I, d), dtype=torch.bfloat16, device=device),
        "w3": torch.empty((n, I, d), dtype=torch.bfloat16, device=device),
        "w2": torch.empty((n, d, I), dtype=torch.bfloat16, device=device),
    }
    for e in range(n):
        for j, (wn, shape, fan_in) in enumerate((("w1", (I, d), d), ("w3", (I, d), d), ("w2", (d, I), I))):
            out[wn][e].copy_(_normal(shape, math.sqrt(1.0 / fan_in), device, seed, tag0 + 3 * e + j))
    return out


def gate_bias(dims: Dims, law: str, device, seed: int, tag: int) -> torch.Tensor:
    E = dims.n_experts
    if law == "zero":
        return torch.zeros(E, dtype=torch.float32, device=device)
    if law.startswith("normal:"):
        return _normal((E,), float(law.split(":")[1]), device, seed, tag)
    if law == "zipf":
        # bias[e] = 0.5 * ln(1 / (rank(e) + 1)), rank from a seeded permutation of 0..E-1
        g = _gen("cpu", seed, tag)
        rank = torch.randperm(E, generator=g).to(torch.float64)
        return (0.5 * torch.log(1.0 / (rank + 1.0))).to(torch.float32).to(device)
    raise ValueError(law)


def make_block(dims: Dims, bias_law: str, device, seed: int, block: int = 0,
               weights: str = "e4m3") -> Dict[str, torch.Tensor]:
    """Parameters of one MoE layer: router weight/bias, routed + 1 shared expert.

    weights: "e4m3" (block-quantised with scales) or "bf16" (no scales).
    """
    t = 1000 + block * 100_000
    p = {
        "gate_w": _normal((dims.n_experts, dims.d_model), math.sqrt(1.0 / dims.d_model), device, seed, t + 1),
        "gate_b": gate_bias(dims, bias_law, device, seed, t + 2),
    }
    make = {"e4m3": expert_weights, "bf16": expert_weights_bf16}[weights]
    routed = make(dims, dims.n_experts, device, seed, t + 10)
    shared = make(dims, 1, device, seed, t + 10 + 3 * dims.n_experts + 5)
    p.update({k: v for k, v in routed.items()})
    p.update({"sh_" + k: v for k, v in shared.items()})
    return p


def mlp_weights(d_model: int, inter: int, device, seed: int) -> Dict[str, torch.Tensor]:
    """One dense SwiGLU MLP (d_model -> inter -> d_model) in the experts' FP8 form, leading dim 1."""
    dims = Dims(d_model=d_model, n_experts=1, n_groups=1, topk_groups=1, topk=1, inter=inter)
    return expert_weights(dims, 1, device, seed, 500)


def make_x(dims: Dims, tokens: int, device, seed: int, tag: int = 1) -> torch.Tensor:
    return _normal((tokens, dims.d_model), 1.0, device, seed, tag).to(torch.bfloat16)


def make_workload(name: str, device="cpu", tokens: Optional[int] = None, seed: Optional[int] = None,
                  blocks: Optional[int] = None, weights: str = "e4m3") -> Dict[str, object]:
    """All inputs of a named workload.  Returns {"x", "blocks": [params...], ...}.

    weights: "e4m3" (the layer's FP8 experts) or "bf16" (the same laws, bf16 without scales).
    """
    w = WORKLOADS[name]
    T = w.tokens if tokens is None else tokens
    s = w.seed if seed is None else seed
    nb = w.blocks if blocks is None else blocks
    out: Dict[str, object] = {"workload": w, "dims": w.dims, "tokens": T, "seed": s}
    out["x"] = make_x(w.dims, T, device, s)
    out["blocks"] = [make_block(w.dims, w.bias, device, s, b, weights=weights) for b in range(nb)]
    if w.blocks > 1:
        out["residual"] = _normal((T, w.dims.d_model), 1.0, device, s, 2).to(torch.bfloat16)
        out["gains"] = [1.0 + _normal((w.dims.d_model,), w.gain_sigma, device, s, 3 + 10 * b) for b in range(nb)]
    return out


_SCALE_KEYS = {"s1", "s2", "s3", "sh_s1", "sh_s2", "sh_s3"}


def block_tensors_numel(p: Dict[str, torch.Tensor]) -> int:
    """Learned elements of one layer (FP8 block scales are metadata and not counted)."""
    return sum(v.numel() for k, v in p.items() if k not in _SCALE_KEYS)
