"""Benchmark of the DeepSeek-V3.2-Exp MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skewed|stack4|tiny]
                    [--extra prefill,skewed,stack4|none] [--tokens T] [--weights e4m3|bf16]
                    [--ep-share N] [--fused] [--mlp INTER] [--no-cpu-baseline]

A step is one pass of the whole layer (router, permutation, grouped expert
FFN, combine; for the stacked workload four blocks of fused residual-add
RMSNorm + layer) over one batch of synthetic, seeded inputs that are resident
in HBM before timing starts.  Prints one JSON line: the headline workload's
tokens/s, the roofline position of its dominant kernel (timed with HIP events
on the library's stream inside the timed region, which records only the two
events around that kernel; every stage's time comes from an instrumented
pass before it) and the CPU oracle's
throughput on a sample of the same workload (with the parity of the timed
GPU output against that oracle call), plus one record per extra workload
(the compute-bound ones by default) with the same measurements.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s (the expert GEMMs run bf16 MFMAs)
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense fp8 matrix peak, TFLOP/s (the figure the metric names)
STAGES = ("gate", "permute", "ffn_up", "ffn_down", "combine")


class HipEvents:
    """hipEvent_t handles from the HIP runtime already loaded by torch."""

    def __init__(self):
        path = None
        for m in re.findall(r"(/\S*libamdhip64\S*)", open("/proc/self/maps").read()):
            path = m
            break
        self.hip = ctypes.CDLL(path or "libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(ev))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
            out.append(ev.value)
        self.made.extend(out)
        return out

    def ms(self, a, b) -> float:
        v = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(v), ctypes.c_void_p(a), ctypes.c_void_p(b))
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(v.value)

    def record(self, ev, stream):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        rc = self.hip.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def close(self):
        for e in self.made:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))
        self.made = []


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = tuple("mixture_experts_ffn_bias_amd/csrc/" + f for f in ("ffn.hip", "ffn_tile.h", "plan.h", "common.h"))


def kernel_source_digest() -> str:
    """SHA-256 of the FFN kernel sources' code.

    Comments are removed and whitespace collapsed first, so that an edit of a
    comment leaves the digest, and the counters taken with the same code,
    valid.  (None of these sources has a comment marker inside a string.)
    """
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        src = open(os.path.join(ROOT, f)).read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counters, or None.

    profiles/traffic.json holds FETCH_SIZE and WRITE_SIZE (KiB per dispatch) per
    workload and kernel, the factors that turn them into bytes (what the same
    counters read for a plain device copy of known size) and the digest of the
    kernel sources they were taken with; a different digest means the kernels
    changed since, and no traffic is reported.
    """
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    e = t.get("kernels", {}).get(f"{workload}/{kernel}")
    if not e:
        return None
    return int((e["fetch_kib"] * t["fetch_factor"] + e["write_kib"] * t["write_factor"]) * 1024)


def algorithmic_work(dims, T, touched, bf16=False):
    """Bytes and FLOPs the method must move / compute, per kernel and per layer.

    touched: number of routed experts with at least one row (the shared expert
    comes on top).  A projection kernel's algorithmic bytes are the weights
    (and block scales) of the experts it runs, plus, for the up-projection,
    x read once (its e4m3 codes and scales; bf16 with bf16 weights).  h and
    the expert output rows o are intermediate buffers of this implementation
    and are reported apart ("h_bytes", "o_bytes": each written once and read
    once).  The layer's bytes are every touched expert's weights, the router
    weight and bias, x in and the update out (bf16).
    bf16: bf16 expert weights without scales and bf16 activations.
    """
    d, I, K = dims.d_model, dims.inter, dims.topk
    R = T * K + T                                  # routed rows + shared rows
    ne = touched + 1
    if bf16:
        up_w, dn_w = 2 * (2 * I * d), 2 * I * d
        x_bytes, h_bytes = T * d * 2, R * I * 2
    else:
        up_w = 2 * I * d + 2 * (I // 128) * (d // 128) * 4
        dn_w = I * d + (d // 128) * (I // 128) * 4
        x_bytes, h_bytes = T * d + T * (d // 128) * 4, R * (I + (I // 128) * 4)
    return {
        "ffn_up": {"bytes": ne * up_w + x_bytes, "flops": 2 * R * d * 2 * I},
        "ffn_down": {"bytes": ne * dn_w, "flops": 2 * R * I * d},
        "h_bytes": h_bytes,
        "o_bytes": R * d * 2,
        "layer_bytes": ne * (up_w + dn_w) + dims.n_experts * d * 4 + dims.n_experts * 4 + 2 * T * d * 2,
        "layer_flops": 2 * R * 3 * d * I,
    }


def roofline_position(alg_bytes, alg_flops, seconds):
    """Achieved HBM rate and matrix rate of a kernel or step, each as a fraction of
    its MI355X peak (bf16 MFMA, which the expert GEMMs use, and the fp8 figure),
    and which of HBM and bf16 MFMA binds (the larger fraction)."""
    gbs = alg_bytes / seconds / 1e9
    tfs = alg_flops / seconds / 1e12
    hbm, bf16, fp8 = gbs / HBM_PEAK_GBS, tfs / BF16_MFMA_PEAK_TFLOPS, tfs / FP8_MFMA_PEAK_TFLOPS
    if hbm >= bf16:
        head = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(hbm, 4)}
    else:
        head = {"bound": "mfma", "achieved": round(tfs, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(bf16, 4)}
    head.update({"hbm_GBps": round(gbs, 1), "hbm_frac": round(hbm, 4), "TFLOPs": round(tfs, 1),
                 "bf16_mfma_frac": round(bf16, 4), "fp8_mfma_frac": round(fp8, 4)})
    return head


def _host(t):
    """Host numpy copy; bf16 comes back as its uint16 bit patterns (the oracle's bf16 weight form)."""
    import numpy as np
    import torch
    t = t.detach().cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def host_threads() -> int:
    """Host threads for the oracle: the process's CPU share (OMP_NUM_THREADS when set), at most the cores."""
    n = os.cpu_count() or 1
    try:
        return max(1, min(n, int(os.environ.get("OMP_NUM_THREADS", n))))
    except ValueError:
        return n


def cpu_baseline(x, params, dims, threads, tokens, residual=None, gain=None, gpu_delta=None, gpu_idx=None):
    """The oracle on host cores: ONE call over the token sample `tokens`.

    The weights of the experts the sample selects are copied to host memory
    before the timed call; the call itself runs the router, dequantises each
    of those experts once, evaluates them and the shared expert in float64
    and combines.  With a residual and gain, the fused residual-add RMSNorm in
    front of the layer is in the timed call too.  When the GPU's output and
    routing of the same layer are given, the parity of the GPU output on the
    sample against this call's result comes back as well (tokens whose oracle
    selection margin is below 1e-5 and that the GPU routes differently are
    left out of the output figures and counted).
    """
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import oracle

    torch.set_num_threads(threads)
    tok = np.asarray(tokens, dtype=np.int64)
    names = ("w1", "s1", "w3", "s3", "w2", "s2") if "s1" in params else ("w1", "w3", "w2")
    xv = x[torch.from_numpy(tok).to(x.device)].float().cpu().numpy().astype(np.float64)
    rv = residual[torch.from_numpy(tok).to(x.device)].float().cpu().numpy().astype(np.float64) \
        if residual is not None else None
    gv = gain.cpu().numpy() if gain is not None else None
    host = {"gate_w": params["gate_w"].cpu().numpy(), "gate_b": params["gate_b"].cpu().numpy()}
    for n in names:
        host["sh_" + n] = _host(params["sh_" + n])
    with threadpool_limits(limits=threads):
        xin = oracle.add_rmsnorm(xv, rv, gv)[0] if rv is not None else xv
        sel = oracle.gate(xin, host["gate_w"], host["gate_b"], dims)["idx"]
        need = sorted(set(sel.ravel().tolist()))
        for n in names:                            # untimed: host copies of the selected experts' weights
            full = params[n]
            host[n] = {e: _host(full[e]) for e in need}
        t0 = time.perf_counter()
        if rv is not None:
            xin = oracle.add_rmsnorm(xv, rv, gv)[0]
        ref = oracle.moe_forward(xin, host, dims)
        elapsed = time.perf_counter() - t0
    what = "fused residual-add RMSNorm + layer" if residual is not None else "layer"
    base = {"value": round(tok.size / elapsed, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{tok.size} of {x.shape[0]} tokens in one oracle call ({what}: router, the {len(need)} "
                      f"experts the sample selects, each dequantised once, and the shared expert, float64), "
                      f"{elapsed:.1f} s on {threads} host threads"}
    parity = None
    if gpu_delta is not None and gpu_idx is not None:
        r = ref["routing"]
        gi = np.sort(gpu_idx[tok], axis=1)
        same = np.all(gi == np.sort(r["idx"], axis=1), axis=1)
        near = (r["expert_gap"] < 1e-5) | (r["group_gap"] < 1e-5)
        got = gpu_delta[torch.from_numpy(tok).to(gpu_delta.device)].float().cpu().numpy().astype(np.float64)
        y = ref["y"]
        diff = np.abs(got[same] - y[same])
        parity = {"tokens": int(tok.size), "routing_identical": int(same.sum()),
                  "routed_differently_near_tie": int((~same & near).sum()),
                  "routed_differently_not_near_tie": int((~same & ~near).sum()),
                  "near_tie_tokens": int(near.sum()),
                  "max_abs_over_rms": float(diff.max() / np.sqrt(np.mean(y[same] ** 2))),
                  "mean_rel": float(diff.mean() / np.abs(y[same]).mean()),
                  "bounds": {"max_abs_over_rms": 2e-2, "mean_rel": 5e-3}}
    return base, parity


def gpu_info(torch):
    """Device name and clocks (best effort: rocm-smi's current clocks when it answers)."""
    import subprocess
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
            "hbm_GiB": round(p.total_memory / 2 ** 30, 1)}
    if "rocprof" in os.environ.get("LD_PRELOAD", ""):
        info["clocks"] = None  # under the profiler a child may not start another program (rocm-smi)
        return info
    try:
        out = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=10).stdout
        clk = {}
        for m in re.finditer(r"(sclk|mclk|fclk|socclk) clock level: \d+: \((\d+)Mhz\)", out):
            clk.setdefault(m.group(1) + "_MHz", int(m.group(2)))
        info["clocks"] = clk or None
    except (OSError, subprocess.SubprocessError):
        info["clocks"] = None
    return info


def bench_layer(name, args, moe, synth, torch, np, dev, tokens=0):
    """Warm-up, then `args.steps` timed steps of workload `name`.

    Returns (record, ctx): the record holds the step time, tokens/s, the touched
    experts, each stage's time (HIP events on the library's stream) and the
    roofline position of the dominant kernel; ctx holds the data the CPU
    baseline needs (freed by the caller)."""
    wl = synth.WORKLOADS[name]
    dims = wl.dims
    bf16 = args.weights == "bf16"
    data = synth.make_workload(name, device=dev, weights=args.weights, tokens=tokens or None)
    T = data["tokens"]
    cd = moe.make_dims(dims.d_model, dims.n_experts, dims.n_groups, dims.topk_groups, dims.topk, dims.inter,
                       dims.route_scale)
    layers = [moe.MoELayer(cd, p) for p in data["blocks"]]
    nb = len(layers)
    x0 = data["x"]
    ws = layers[0].workspace(T)
    stream = torch.cuda.current_stream()
    delta = torch.empty_like(x0)
    idx = [torch.empty((T, dims.topk), dtype=torch.int32, device=dev) for _ in range(nb)]
    w = [torch.empty((T, dims.topk), dtype=torch.float32, device=dev) for _ in range(nb)]
    if nb > 1:
        res0 = data["residual"]
        res = torch.empty_like(res0)
        h = torch.empty_like(x0)
        cur = torch.empty_like(x0)
    hev = HipEvents()
    torch.cuda.synchronize()

    fwd = moe.moe_forward_bf16 if bf16 else moe.moe_forward
    fwd_timed = moe.moe_forward_bf16_timed if bf16 else moe.moe_forward_timed

    def step(events=None):
        if nb == 1:
            if events is None:
                fwd(cd, layers[0].weights, T, x0, delta, idx[0], w[0], ws, stream)
            else:
                fwd_timed(cd, layers[0].weights, T, x0, delta, idx[0], w[0], ws, events[0], stream)
            return
        res.copy_(res0)
        src = x0
        for b in range(nb):
            moe.moe_add_rmsnorm(dims.d_model, T, src, res, data["gains"][b], 1e-6, h, stream)
            out = delta if b == nb - 1 else cur
            if events is None:
                fwd(cd, layers[b].weights, T, h, out, idx[b], w[b], ws, stream)
            else:
                fwd_timed(cd, layers[b].weights, T, h, out, idx[b], w[b], ws, events[b], stream)
            src = out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    launches = K * nb

    def stage_times(evs, stages):
        out = {}
        for i, s in enumerate(STAGES):
            if s in stages:
                out[s] = sum(hev.ms(evs[k][b][i], evs[k][b][i + 1]) for k in range(K) for b in range(nb)) / launches
        return out

    # every stage's time, from K instrumented steps before the timed region
    # (each recorded event adds about 3.5 us to a step)
    evs = [[hev.create(moe.MOE_FORWARD_EVENTS) for _ in range(nb)] for _ in range(K)]
    for k in range(K):
        step(evs[k])
    torch.cuda.synchronize()
    stage_avg = stage_times(evs, STAGES)
    dom = max(("ffn_up", "ffn_down"), key=lambda s: stage_avg[s])
    # the timed region records only the two events around the dominant kernel
    di = STAGES.index(dom)

    def dom_events():
        row = [None] * moe.MOE_FORWARD_EVENTS
        row[di], row[di + 1] = hev.create(2)
        return row

    evs = [[dom_events() for _ in range(nb)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_avg[dom] = stage_times(evs, (dom,))[dom]
    hev.close()

    counts = [np.bincount(i.cpu().numpy().ravel(), minlength=dims.n_experts) for i in idx]
    touched = [int((c > 0).sum()) for c in counts]
    work = [algorithmic_work(dims, T, t, bf16) for t in touched]
    bytes_per = sum(wk[dom]["bytes"] for wk in work) / nb      # per launch (the blocks of the stack are alike)
    flops_per = sum(wk[dom]["flops"] for wk in work) / nb
    roof = roofline_position(bytes_per, flops_per, stage_avg[dom] * 1e-3)
    traffic_key = name + ("_bf16" if bf16 else "")
    roof.update({"kernel": dom, "traffic": measured_traffic(traffic_key, dom), "launch_ms": round(stage_avg[dom], 4),
                 "alg_bytes": int(bytes_per), "alg_flops": int(flops_per),
                 "h_bytes": int(sum(wk["h_bytes"] for wk in work) / nb),
                 "o_bytes": int(sum(wk["o_bytes"] for wk in work) / nb)})
    step_s = wall / K
    layer_bytes = sum(wk["layer_bytes"] for wk in work)
    layer_flops = sum(wk["layer_flops"] for wk in work)
    layer = roofline_position(layer_bytes, layer_flops, step_s)
    layer.update({"alg_bytes_per_step": int(layer_bytes), "alg_flops_per_step": int(layer_flops),
                  "stage_ms": {s: round(v, 4) for s, v in stage_avg.items()}})
    rec = {"workload": name, "tokens": T, "blocks": nb, "steps": K, "ms_per_step": round(step_s * 1e3, 4),
           "tokens_per_s": round(T * K / wall, 2), "touched_experts": touched, "roofline": roof, "layer": layer}
    ctx = {"data": data, "dims": dims, "delta": delta, "idx": idx, "layers": layers, "ws": ws}
    return rec, ctx


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode", choices=["tiny", "decode", "prefill", "skewed", "stack4"],
                    help="the headline workload (its figures are the line's value and roofline)")
    ap.add_argument("--extra", default="prefill,skewed,stack4",
                    help="comma-separated workloads timed after the headline and reported under 'workloads' "
                         "('none' for none)")
    ap.add_argument("--tokens", type=int, default=0,
                    help="token count of the headline workload (default: the workload's own); with --mlp: "
                         "the MLP's batch")
    ap.add_argument("--weights", default="e4m3", choices=["e4m3", "bf16"],
                    help="expert weights: FP8 e4m3 with 128x128 block scales (the layer's), or bf16 without scales")
    ap.add_argument("--ep-share", type=int, default=0, metavar="N",
                    help="time one rank's share of an N-way expert-parallel layer instead: experts [0, E/N) "
                         "plus the shared expert over all tokens (moe_forward_shard, fp32 partial output)")
    ap.add_argument("--fused", action="store_true",
                    help="time the single-launch forward (moe_forward_fused: one kernel for the whole layer, "
                         "at most 64 tokens, e4m3 weights) instead of the per-step kernels")
    ap.add_argument("--mlp", type=int, default=0, metavar="INTER",
                    help="time the dense SwiGLU MLP of the blocks before the MoE blocks instead (moe_mlp, FP8 "
                         "weights d_model -> INTER -> d_model, e.g. 18432) over the workload's tokens")
    ap.add_argument("--cpu-tokens", type=int, default=64,
                    help="tokens in the CPU baseline's one oracle call (the whole batch when it is smaller)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the layer runs on a single GPU here, and a rank's expert "
              "share on one GPU is timed with --ep-share N (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mixture_experts_ffn_bias_amd as moe
    import synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_copy": n, "bytes_written_per_copy": n, "copies": 3}))
        return
    if args.ep_share:
        return bench_share(args, moe, synth, torch, np, dev)
    if args.fused:
        return bench_fused(args, moe, synth, torch, np, dev)
    if args.mlp:
        return bench_mlp(args, moe, synth, torch, np, dev)
    bf16 = args.weights == "bf16"
    rec, ctx = bench_layer(args.workload, args, moe, synth, torch, np, dev, tokens=args.tokens)
    dims = ctx["dims"]
    out = {
        "metric": "MoE layer tokens/s (d7168,256e,top8) + % of fp8 MFMA / HBM roofline",
        "value": rec["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "tokens": rec["tokens"], "blocks": rec["blocks"],
                   "d_model": dims.d_model, "experts": dims.n_experts, "groups": dims.n_groups,
                   "topk_groups": dims.topk_groups, "topk": dims.topk, "inter": dims.inter,
                   "weights": "bf16, no scales" if bf16 else "e4m3 + fp32 128x128 block scales",
                   "touched_experts": rec["touched_experts"]},
        "roofline": rec["roofline"],
        "layer": rec["layer"],
        "gpu": gpu_info(torch),
    }
    if not args.no_cpu_baseline:
        data, T = ctx["data"], rec["tokens"]
        n = min(T, args.cpu_tokens)
        tok = np.sort(np.random.default_rng(0).choice(T, n, replace=False)) if n < T else np.arange(T)
        threads = host_threads()
        if rec["blocks"] > 1:
            base, parity = cpu_baseline(data["x"], data["blocks"][0], dims, threads, tok,
                                        residual=data["residual"], gain=data["gains"][0])
            base["sample"] += "; the first block of the stack, so tokens/s per block"
        else:
            base, parity = cpu_baseline(data["x"], data["blocks"][0], dims, threads, tok, gpu_delta=ctx["delta"],
                                        gpu_idx=ctx["idx"][0].cpu().numpy())
        out["cpu_baseline"] = base
        if parity is not None:
            out["parity"] = parity
    del ctx
    torch.cuda.empty_cache()
    extra = [] if args.extra in ("", "none") else [w for w in args.extra.split(",") if w != args.workload]
    if extra:
        out["workloads"] = {}
        for name in extra:
            r, c = bench_layer(name, args, moe, synth, torch, np, dev)
            del c
            torch.cuda.empty_cache()
            out["workloads"][name] = r
    print(json.dumps(out), flush=True)


def bench_share(args, moe, synth, torch, np, dev):
    """One rank's share of an N-way expert-parallel layer: permutation, FFN of experts
    [0, E/N) and of the shared expert, fp32 partial combine (the routing comes from the
    gate, outside the timed region, as it would from the token's home rank)."""
    wl = synth.WORKLOADS[args.workload]
    dims = wl.dims
    n = args.ep_share
    if wl.blocks != 1 or dims.n_experts % n or args.weights != "e4m3":
        sys.exit("--ep-share takes a single-block workload, a divisor of the expert count and e4m3 weights")
    data = synth.make_workload(args.workload, device=dev)
    T, p = data["tokens"], data["blocks"][0]
    cd = moe.make_dims(dims.d_model, dims.n_experts, dims.n_groups, dims.topk_groups, dims.topk, dims.inter,
                       dims.route_scale)
    e_hi = dims.n_experts // n
    keys = ("w1", "w3", "w2", "s1", "s3", "s2")
    wts = moe.moe_weights(p["gate_w"].data_ptr(), p["gate_b"].data_ptr(),
                          moe.experts_struct(*(p[k][:e_hi] for k in keys)),
                          moe.experts_struct(*(p["sh_" + k] for k in keys)))
    x = data["x"]
    ws = moe.workspace(cd, T, device=dev)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=dev)
    moe.moe_gate(cd, T, x, p["gate_w"], p["gate_b"], idx, w, ws)
    y = torch.empty((T, dims.d_model), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        moe.moe_forward_shard(cd, wts, T, 0, e_hi, True, x, idx, w, y, ws, stream)
    hev = HipEvents()
    K = args.steps
    ev = hev.create(2 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        hev.record(ev[2 * k], stream.cuda_stream)
        moe.moe_forward_shard(cd, wts, T, 0, e_hi, True, x, idx, w, y, ws, stream)
        hev.record(ev[2 * k + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = sum(hev.ms(ev[2 * k], ev[2 * k + 1]) for k in range(K)) / K
    hev.close()
    gi = idx.cpu().numpy()
    touched = int((np.bincount(gi.ravel(), minlength=dims.n_experts)[:e_hi] > 0).sum())
    d, I = dims.d_model, dims.inter
    rows = int(((gi >= 0) & (gi < e_hi)).sum()) + T
    wbytes = (touched + 1) * (3 * I * d + 3 * (I // 128) * (d // 128) * 4)
    alg = wbytes + T * d * 2 + T * dims.topk * 8 + T * d * 4
    flops = 2 * rows * 3 * d * I
    roof = roofline_position(alg, flops, step_ms * 1e-3)
    roof.update({"kernel": "share step (permute + FFN + partial combine)", "traffic": None,
                 "launch_ms": round(step_ms, 4), "alg_bytes": int(alg), "alg_flops": int(flops)})
    out = {
        "metric": "MoE layer tokens/s (d7168,256e,top8): one rank's expert share",
        "value": round(T * K / wall, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "ep_share": f"experts 0..{e_hi - 1} of "
                   f"{dims.n_experts} + shared ({n}-way split)", "rows": rows, "touched_experts": touched},
        "roofline": roof, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def bench_fused(args, moe, synth, torch, np, dev):
    """The whole layer as one kernel launch (moe_forward_fused), timed launch by launch."""
    wl = synth.WORKLOADS[args.workload]
    dims = wl.dims
    if wl.blocks != 1 or args.weights != "e4m3":
        sys.exit("--fused takes a single-block workload and e4m3 weights")
    data = synth.make_workload(args.workload, device=dev, tokens=args.tokens or None)
    T = data["tokens"]
    if T > moe.FUSED_MAX_TOKENS:
        sys.exit(f"--fused runs at most {moe.FUSED_MAX_TOKENS} tokens (workload has {T})")
    cd = moe.make_dims(dims.d_model, dims.n_experts, dims.n_groups, dims.topk_groups, dims.topk, dims.inter,
                       dims.route_scale)
    layer = moe.MoELayer(cd, data["blocks"][0])
    x = data["x"]
    ws = moe.fused_workspace(cd, T, device=dev)
    delta = torch.empty_like(x)
    idx = torch.empty((T, dims.topk), dtype=torch.int32, device=dev)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        moe.moe_forward_fused(cd, layer.weights, T, x, delta, idx, w, ws, stream)
    if moe.moe_forward_fused_status(ws, stream) != 0:
        sys.exit("moe_forward_fused: a wait gave up (status MOE_ERR_STALLED)")
    hev = HipEvents()
    K = args.steps
    ev = hev.create(2 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        hev.record(ev[2 * k], stream.cuda_stream)
        moe.moe_forward_fused(cd, layer.weights, T, x, delta, idx, w, ws, stream)
        hev.record(ev[2 * k + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = sum(hev.ms(ev[2 * k], ev[2 * k + 1]) for k in range(K)) / K
    hev.close()
    status = moe.moe_forward_fused_status(ws, stream)
    touched = int((np.bincount(idx.cpu().numpy().ravel(), minlength=dims.n_experts) > 0).sum())
    work = algorithmic_work(dims, T, touched)
    gbs = work["layer_bytes"] / (launch_ms * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": "decode_kernel (whole layer, one launch)",
            "traffic": None, "launch_ms": round(launch_ms, 4), "alg_bytes": int(work["layer_bytes"]),
            "alg_flops": int(work["layer_flops"])}
    out = {
        "metric": "MoE layer tokens/s (d7168,256e,top8) + % of fp8 MFMA / HBM roofline",
        "value": round(T * K / wall, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "path": "single launch (moe_forward_fused)",
                   "touched_experts": touched, "status": "ok" if status == 0 else "stalled"},
        "roofline": roof, "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)
    if status != 0:
        sys.exit("moe_forward_fused: a wait gave up during the timed launches")


def bench_mlp(args, moe, synth, torch, np, dev):
    """The dense MLP (moe_mlp) over the workload's tokens, timed launch by launch."""
    wl = synth.WORKLOADS[args.workload]
    d, inter = wl.dims.d_model, args.mlp
    if args.weights != "e4m3":
        sys.exit("--mlp takes e4m3 weights")
    T = args.tokens or wl.tokens
    x = synth.make_x(wl.dims, T, dev, wl.seed)
    p = synth.mlp_weights(d, inter, dev, wl.seed)
    mlp = moe.experts_struct(*(p[k] for k in ("w1", "w3", "w2", "s1", "s3", "s2")))
    ws = moe.mlp_workspace(d, inter, T, device=dev)
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        moe.moe_mlp(d, inter, T, mlp, x, out, ws, stream)
    hev = HipEvents()
    K = args.steps
    ev = hev.create(2 * K)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(K):
        hev.record(ev[2 * k], stream.cuda_stream)
        moe.moe_mlp(d, inter, T, mlp, x, out, ws, stream)
        hev.record(ev[2 * k + 1], stream.cuda_stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = sum(hev.ms(ev[2 * k], ev[2 * k + 1]) for k in range(K)) / K
    hev.close()
    wbytes = 3 * d * inter + 3 * (d // 128) * (inter // 128) * 4
    alg_bytes = wbytes + 2 * T * d * 2                      # weights once, x in, out
    alg_flops = 6 * T * d * inter
    roof = roofline_position(alg_bytes, alg_flops, launch_ms * 1e-3)
    roof.update({"kernel": "dense MLP (quantisation + up- and down-projection)", "traffic": None,
                 "launch_ms": round(launch_ms, 4), "alg_bytes": int(alg_bytes), "alg_flops": int(alg_flops)})
    res = {
        "metric": "dense MLP tokens/s (d7168, FP8 SwiGLU) + % of bf16 MFMA / HBM roofline",
        "value": round(T * K / wall, 2), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": args.workload, "tokens": T, "path": "dense MLP (moe_mlp)", "d_model": d,
                   "inter": inter, "weights": "e4m3 + fp32 128x128 block scales"},
        "roofline": roof, "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
