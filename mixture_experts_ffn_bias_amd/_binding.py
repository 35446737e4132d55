"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
of the library.  torch provides device memory and the current stream.  If
the library has not been built, loading it raises instead of falling back to
anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK = 0
SYMBOLS = ("moe_workspace_size", "moe_gate", "moe_permute", "moe_grouped_ffn", "moe_grouped_ffn_bf16", "moe_combine",
           "moe_forward", "moe_forward_timed", "moe_forward_bf16", "moe_forward_bf16_timed", "moe_forward_shard",
           "moe_forward_fused_workspace_size", "moe_forward_fused", "moe_forward_fused_status", "moe_add_rmsnorm",
           "moe_mlp_workspace_size", "moe_mlp", "moe_forward_no_workspace", "moe_status_string")
MOE_ERR_STALLED = -6
FUSED_MAX_TOKENS = 64
MOE_FORWARD_EVENTS = 6
MOE_STATIC_WORKSPACE_BYTES = 32 << 20


class MoeError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what} failed: {status_string(code)} ({code})")
        self.code = code


class moe_dims(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("topk", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("route_scale", ctypes.c_float)]


class moe_experts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2", "s1", "s3", "s2")]


class moe_weights(ctypes.Structure):
    _fields_ = [("gate_w", ctypes.c_void_p), ("gate_b", ctypes.c_void_p), ("routed", moe_experts),
                ("shared", moe_experts)]


class moe_experts_bf16(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w1", "w3", "w2")]


class moe_weights_bf16(ctypes.Structure):
    _fields_ = [("gate_w", ctypes.c_void_p), ("gate_b", ctypes.c_void_p), ("routed", moe_experts_bf16),
                ("shared", moe_experts_bf16)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with `python -m mixture_experts_ffn_bias_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        dp = ctypes.POINTER(moe_dims)
        L.moe_workspace_size.argtypes = [dp, i64]
        L.moe_workspace_size.restype = sz
        L.moe_gate.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [dp, i64, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_grouped_ffn.argtypes = [dp, i64, ctypes.POINTER(moe_experts), ctypes.POINTER(moe_experts), vp, vp, vp,
                                      vp, vp, vp, sz, vp]
        L.moe_grouped_ffn_bf16.argtypes = [dp, i64, ctypes.POINTER(moe_experts_bf16), ctypes.POINTER(moe_experts_bf16),
                                           vp, vp, vp, vp, vp, sz, vp]
        L.moe_combine.argtypes = [dp, i64, vp, vp, vp, vp, i32, vp, vp]
        L.moe_forward.argtypes = [dp, ctypes.POINTER(moe_weights), i64, vp, vp, vp, vp, vp, sz, vp]
        L.moe_forward_timed.argtypes = [dp, ctypes.POINTER(moe_weights), i64, vp, vp, vp, vp, vp, sz, vp,
                                        ctypes.POINTER(ctypes.c_void_p)]
        L.moe_forward_bf16.argtypes = [dp, ctypes.POINTER(moe_weights_bf16), i64, vp, vp, vp, vp, vp, sz, vp]
        L.moe_forward_bf16_timed.argtypes = [dp, ctypes.POINTER(moe_weights_bf16), i64, vp, vp, vp, vp, vp, sz, vp,
                                             ctypes.POINTER(ctypes.c_void_p)]
        L.moe_forward_shard.argtypes = [dp, ctypes.POINTER(moe_weights), i64, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_forward_fused_workspace_size.argtypes = [dp, i64]
        L.moe_forward_fused_workspace_size.restype = sz
        L.moe_forward_fused.argtypes = [dp, ctypes.POINTER(moe_weights), i64, vp, vp, vp, vp, vp, sz, vp]
        L.moe_forward_fused_status.argtypes = [vp, vp]
        L.moe_add_rmsnorm.argtypes = [i32, i64, vp, vp, vp, ctypes.c_float, vp, vp]
        L.moe_mlp_workspace_size.argtypes = [i32, i32, i64]
        L.moe_mlp_workspace_size.restype = sz
        L.moe_mlp.argtypes = [i32, i32, i64, ctypes.POINTER(moe_experts), vp, vp, vp, sz, vp]
        L.moe_forward_no_workspace.argtypes = [dp, ctypes.POINTER(moe_weights), i64, vp, vp, vp, vp, vp]
        for n in ("moe_gate", "moe_permute", "moe_grouped_ffn", "moe_grouped_ffn_bf16", "moe_combine", "moe_forward",
                  "moe_forward_timed", "moe_forward_bf16", "moe_forward_bf16_timed", "moe_forward_shard",
                  "moe_forward_fused", "moe_forward_fused_status", "moe_add_rmsnorm", "moe_mlp",
                  "moe_forward_no_workspace"):
            getattr(L, n).restype = ctypes.c_int
        L.moe_status_string.argtypes = [ctypes.c_int]
        L.moe_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().moe_status_string(int(code)).decode()


def _p(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, what: str):
    if rc != MOE_OK:
        raise MoeError(rc, what)


def make_dims(d_model, n_experts, n_groups, topk_groups, topk, inter, route_scale=2.5) -> moe_dims:
    return moe_dims(d_model, n_experts, n_groups, topk_groups, topk, inter, route_scale)


def experts_struct(w1, w3, w2, s1, s3, s2) -> moe_experts:
    return moe_experts(_p(w1), _p(w3), _p(w2), _p(s1), _p(s3), _p(s2))


def moe_workspace_size(dims: moe_dims, tokens: int) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(dims), int(tokens)))


def workspace(dims: moe_dims, tokens: int, device="cuda") -> torch.Tensor:
    n = moe_workspace_size(dims, tokens)
    if n == 0 and tokens > 0:
        raise MoeError(-1, "moe_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_gate(dims, tokens, x, gate_w, gate_b, idx, w, ws, stream=None):
    _check(lib().moe_gate(ctypes.byref(dims), int(tokens), _p(x), _p(gate_w), _p(gate_b), _p(idx), _p(w), _p(ws),
                          ws.numel() if ws is not None else 0, _stream(stream)), "moe_gate")


def moe_permute(dims, tokens, idx, x, counts, offsets, row_token, pair_row, xq, xs, ws, stream=None):
    _check(lib().moe_permute(ctypes.byref(dims), int(tokens), _p(idx), _p(x), _p(counts), _p(offsets),
                             _p(row_token), _p(pair_row), _p(xq), _p(xs), _p(ws),
                             ws.numel() if ws is not None else 0, _stream(stream)), "moe_permute")


def moe_grouped_ffn(dims, tokens, routed: moe_experts, shared: Optional[moe_experts], offsets, row_token, xq, xs,
                    out, ws, stream=None):
    _check(lib().moe_grouped_ffn(ctypes.byref(dims), int(tokens), ctypes.byref(routed),
                                 ctypes.byref(shared) if shared is not None else None, _p(offsets), _p(row_token),
                                 _p(xq), _p(xs), _p(out), _p(ws), ws.numel() if ws is not None else 0,
                                 _stream(stream)), "moe_grouped_ffn")


def experts_struct_bf16(w1, w3, w2) -> moe_experts_bf16:
    return moe_experts_bf16(_p(w1), _p(w3), _p(w2))


def moe_grouped_ffn_bf16(dims, tokens, routed: moe_experts_bf16, shared: Optional[moe_experts_bf16], offsets,
                         row_token, x, out, ws, stream=None):
    _check(lib().moe_grouped_ffn_bf16(ctypes.byref(dims), int(tokens), ctypes.byref(routed),
                                      ctypes.byref(shared) if shared is not None else None, _p(offsets),
                                      _p(row_token), _p(x), _p(out), _p(ws), ws.numel() if ws is not None else 0,
                                      _stream(stream)), "moe_grouped_ffn_bf16")


def moe_combine(dims, tokens, idx, w, pair_row, rows, has_shared, delta, stream=None):
    _check(lib().moe_combine(ctypes.byref(dims), int(tokens), _p(idx), _p(w), _p(pair_row), _p(rows),
                             1 if has_shared else 0, _p(delta), _stream(stream)), "moe_combine")


def moe_forward(dims, weights: moe_weights, tokens, x, delta, idx_out, w_out, ws, stream=None):
    _check(lib().moe_forward(ctypes.byref(dims), ctypes.byref(weights), int(tokens), _p(x), _p(delta), _p(idx_out),
                             _p(w_out), _p(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_forward")


def moe_forward_no_workspace(dims, weights: moe_weights, tokens, x, delta, idx_out, w_out, stream=None):
    """moe_forward with the library's own per-GPU array as its workspace (allocates nothing;
    calls that overlap on one GPU race)."""
    _check(lib().moe_forward_no_workspace(ctypes.byref(dims), ctypes.byref(weights), int(tokens), _p(x), _p(delta),
                                          _p(idx_out), _p(w_out), _stream(stream)), "moe_forward_no_workspace")


def moe_forward_timed(dims, weights: moe_weights, tokens, x, delta, idx_out, w_out, ws, events, stream=None):
    """events: MOE_FORWARD_EVENTS hipEvent_t handles (ints, e.g. from HipEvents); None entries are not recorded."""
    arr = (ctypes.c_void_p * MOE_FORWARD_EVENTS)(*events)
    _check(lib().moe_forward_timed(ctypes.byref(dims), ctypes.byref(weights), int(tokens), _p(x), _p(delta),
                                   _p(idx_out), _p(w_out), _p(ws), ws.numel() if ws is not None else 0,
                                   _stream(stream), arr), "moe_forward_timed")


def moe_forward_bf16(dims, weights: moe_weights_bf16, tokens, x, delta, idx_out, w_out, ws, stream=None):
    _check(lib().moe_forward_bf16(ctypes.byref(dims), ctypes.byref(weights), int(tokens), _p(x), _p(delta),
                                  _p(idx_out), _p(w_out), _p(ws), ws.numel() if ws is not None else 0,
                                  _stream(stream)), "moe_forward_bf16")


def moe_forward_bf16_timed(dims, weights: moe_weights_bf16, tokens, x, delta, idx_out, w_out, ws, events,
                           stream=None):
    arr = (ctypes.c_void_p * MOE_FORWARD_EVENTS)(*events)
    _check(lib().moe_forward_bf16_timed(ctypes.byref(dims), ctypes.byref(weights), int(tokens), _p(x), _p(delta),
                                        _p(idx_out), _p(w_out), _p(ws), ws.numel() if ws is not None else 0,
                                        _stream(stream), arr), "moe_forward_bf16_timed")


def moe_forward_shard(dims, weights: moe_weights, tokens, expert_begin, expert_end, with_shared, x, idx, w, y_partial,
                      ws, stream=None):
    _check(lib().moe_forward_shard(ctypes.byref(dims), ctypes.byref(weights), int(tokens), int(expert_begin),
                                   int(expert_end), 1 if with_shared else 0, _p(x), _p(idx), _p(w), _p(y_partial),
                                   _p(ws), ws.numel() if ws is not None else 0, _stream(stream)), "moe_forward_shard")


def moe_add_rmsnorm(d, tokens, x, residual, gain, eps, out, stream=None):
    _check(lib().moe_add_rmsnorm(int(d), int(tokens), _p(x), _p(residual), _p(gain), float(eps), _p(out),
                                 _stream(stream)), "moe_add_rmsnorm")


def moe_mlp_workspace_size(d_model: int, inter: int, tokens: int) -> int:
    return int(lib().moe_mlp_workspace_size(int(d_model), int(inter), int(tokens)))


def mlp_workspace(d_model: int, inter: int, tokens: int, device="cuda") -> torch.Tensor:
    n = moe_mlp_workspace_size(d_model, inter, tokens)
    if n == 0 and tokens > 0:
        raise MoeError(-1, "moe_mlp_workspace_size")
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def moe_forward_fused_workspace_size(dims: moe_dims, tokens: int) -> int:
    return int(lib().moe_forward_fused_workspace_size(ctypes.byref(dims), int(tokens)))


def fused_workspace(dims: moe_dims, tokens: int, device="cuda") -> torch.Tensor:
    """Workspace of moe_forward_fused for up to `tokens` tokens, zeroed (its
    leading control block must start at zero; each call leaves it so)."""
    n = moe_forward_fused_workspace_size(dims, tokens)
    if n == 0:
        raise MoeError(-2, "moe_forward_fused_workspace_size")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def moe_forward_fused(dims, weights: moe_weights, tokens, x, delta, idx_out, w_out, ws, stream=None):
    _check(lib().moe_forward_fused(ctypes.byref(dims), ctypes.byref(weights), int(tokens), _p(x), _p(delta),
                                   _p(idx_out), _p(w_out), _p(ws), ws.numel() if ws is not None else 0,
                                   _stream(stream)), "moe_forward_fused")


def moe_forward_fused_status(ws, stream=None) -> int:
    """MOE_OK, or MOE_ERR_STALLED if a wait of the last call on `ws` gave up (synchronises the stream)."""
    return int(lib().moe_forward_fused_status(_p(ws), _stream(stream)))


def moe_mlp(d_model, inter, tokens, mlp: moe_experts, x, out, ws, stream=None):
    _check(lib().moe_mlp(int(d_model), int(inter), int(tokens), ctypes.byref(mlp), _p(x), _p(out), _p(ws),
                         ws.numel() if ws is not None else 0, _stream(stream)), "moe_mlp")


_EXPERT_KEYS = ("w1", "w3", "w2", "s1", "s3", "s2")


class MoELayer:
    """One MoE layer whose parameters live in device memory.

    params: gate_w fp32 [E, d], gate_b fp32 [E], w1/w3 uint8 [E, I, d],
    w2 uint8 [E, d, I], s1/s3 fp32 [E, I/128, d/128], s2 fp32 [E, d/128, I/128],
    and the same with an ``sh_`` prefix for the shared expert (leading dim 1).
    With bf16 w1/w3/w2 (and no scales) the layer runs moe_forward_bf16.

    The layer keeps one workspace (grown on demand) that every call uses: calls
    on different streams must be ordered by the caller (an event or a sync),
    as must a call that grows the workspace after a call on another stream.
    """

    def __init__(self, dims: moe_dims, params: Dict[str, torch.Tensor]):
        self.dims = dims
        E, d, I = dims.n_experts, dims.d_model, dims.inter
        self.bf16 = params["w1"].dtype == torch.bfloat16
        wdt = torch.bfloat16 if self.bf16 else torch.uint8
        want = {"gate_w": ((E, d), torch.float32), "gate_b": ((E,), torch.float32)}
        for pre, n in (("", E), ("sh_", 1)):
            want[pre + "w1"] = ((n, I, d), wdt)
            want[pre + "w3"] = ((n, I, d), wdt)
            want[pre + "w2"] = ((n, d, I), wdt)
            if not self.bf16:
                want[pre + "s1"] = ((n, I // 128, d // 128), torch.float32)
                want[pre + "s3"] = ((n, I // 128, d // 128), torch.float32)
                want[pre + "s2"] = ((n, d // 128, I // 128), torch.float32)
        for k, (shape, dt) in want.items():
            t = params[k]
            if tuple(t.shape) != shape or t.dtype != dt or not t.is_contiguous() or t.device.type != "cuda":
                raise ValueError(f"{k}: expected contiguous {dt} {shape} on the GPU, got {t.dtype} "
                                 f"{tuple(t.shape)} on {t.device}")
        self.params = params
        if self.bf16:
            self.weights = moe_weights_bf16(
                _p(params["gate_w"]), _p(params["gate_b"]),
                experts_struct_bf16(*(params[k] for k in ("w1", "w3", "w2"))),
                experts_struct_bf16(*(params["sh_" + k] for k in ("w1", "w3", "w2"))))
        else:
            self.weights = moe_weights(
                _p(params["gate_w"]), _p(params["gate_b"]),
                experts_struct(*(params[k] for k in _EXPERT_KEYS)),
                experts_struct(*(params["sh_" + k] for k in _EXPERT_KEYS)))
        self._ws: Optional[torch.Tensor] = None
        self._fused_ws: Optional[torch.Tensor] = None

    def workspace(self, tokens: int) -> torch.Tensor:
        n = moe_workspace_size(self.dims, tokens)
        if self._ws is None or self._ws.numel() < n:
            self._ws = workspace(self.dims, tokens, device=self.params["gate_w"].device)
        return self._ws

    def forward(self, x: torch.Tensor, delta=None, idx=None, w=None, stream=None) -> torch.Tensor:
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != self.dims.d_model or not x.is_contiguous():
            raise ValueError("x must be a contiguous bf16 [tokens, d_model] tensor")
        T = x.shape[0]
        if delta is None:
            delta = torch.empty_like(x)
        run = moe_forward_bf16 if self.bf16 else moe_forward
        run(self.dims, self.weights, T, x, delta, idx, w, self.workspace(T), stream)
        return delta

    def forward_fused(self, x: torch.Tensor, delta=None, idx=None, w=None, stream=None) -> torch.Tensor:
        """forward() as one kernel launch (moe_forward_fused): e4m3 weights, at most 64 tokens."""
        if self.bf16:
            raise ValueError("the single-launch forward takes e4m3 expert weights")
        if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != self.dims.d_model or not x.is_contiguous():
            raise ValueError("x must be a contiguous bf16 [tokens, d_model] tensor")
        T = x.shape[0]
        if delta is None:
            delta = torch.empty_like(x)
        n = moe_forward_fused_workspace_size(self.dims, T)
        if self._fused_ws is None or self._fused_ws.numel() < n:
            self._fused_ws = fused_workspace(self.dims, T, device=self.params["gate_w"].device)
        moe_forward_fused(self.dims, self.weights, T, x, delta, idx, w, self._fused_ws, stream)
        return delta

    __call__ = forward
