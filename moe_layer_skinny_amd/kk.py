"""ctypes binding of libkk.so (include/kk.h).  Argument marshalling only.

Every step of the layer runs in the library's HIP kernels; PyTorch is used here only to
hand over device pointers and streams.  There is no fallback: if libkk.so is missing the
import of a Layer raises.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkk.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "kk.h")

KK_OK, KK_ERR_INVALID_ARG, KK_ERR_UNSUPPORTED, KK_ERR_WORKSPACE, KK_ERR_HIP = range(5)
KK_F32, KK_BF16 = 0, 1
KK_PATH_GEMV, KK_PATH_SPLITK_MFMA = 0, 1
KK_GRAPH = 1
KK_TWO_STREAM = 2
KK_PREFETCH = 4
PATH_NAMES = {KK_PATH_GEMV: "gemv", KK_PATH_SPLITK_MFMA: "splitk_mfma"}


class KKConfig(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("oproj_in", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("routed_scale", ctypes.c_float),
                ("norm_eps", ctypes.c_float)]


class KKWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_o", "w_r", "router_bias", "w13", "w2", "ws13", "ws2",
                                               "norm_weight")]


class KKPlan(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("path", "forced", "oproj_splitk", "router_splitk",
                                              "kernels_per_step", "streams")]


class KKError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_string(status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded libkk.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(there is no fallback implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32
        sig = {
            "kk_validate": (i32, [ctypes.POINTER(KKConfig), i32]),
            "kk_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(KKConfig), i32]),
            "kk_create": (i32, [ctypes.POINTER(KKConfig), ctypes.POINTER(KKWeights), i32,
                                ctypes.POINTER(vp)]),
            "kk_destroy": (i32, [vp]),
            "kk_query_plan": (i32, [vp, i32, ctypes.POINTER(KKPlan)]),
            "kk_oproj_residual": (i32, [vp, i32, vp, vp, vp, vp, vp, vp]),
            "kk_router_topk": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp]),
            "kk_moe_decode": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]),
            "kk_routing_status": (i32, [vp, vp, vp]),
            "kk_layer_decode": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, vp, u32]),
            "kk_layer_decode_static": (i32, [vp, i32, vp, vp, vp, vp, vp, vp, u32]),
            "kk_chain_decode": (i32, [ctypes.POINTER(vp), i32, i32, ctypes.POINTER(vp), vp,
                                      ctypes.POINTER(vp), vp, vp, u32]),
            "kk_set_stream_delay": (i32, [vp, i32, ctypes.c_float]),
            "kk_set_kernel_timing": (i32, [vp, i32]),
            "kk_read_kernel_timing": (i32, [vp, ctypes.POINTER(ctypes.c_char_p),
                                            ctypes.POINTER(ctypes.c_float), i32,
                                            ctypes.POINTER(i32)]),
            "kk_status_string": (ctypes.c_char_p, [i32]),
            "kk_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/kk.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(kk_[a-z_]+)\s*\(", text, re.M)))


def status_string(s: int) -> str:
    return lib().kk_status_string(s).decode()


def last_error() -> str:
    return lib().kk_last_error().decode()


def _check(status: int) -> None:
    if status != KK_OK:
        raise KKError(status, last_error())


def make_config(hidden, oproj_in, n_experts, top_k, inter, shared_inter, dtype, routed_scale=1.0,
                norm_eps=1e-6):
    """norm_eps applies only to a layer created with a norm weight ("norm_w")."""
    dt = {"f32": KK_F32, "bf16": KK_BF16}.get(dtype, dtype)
    return KKConfig(hidden, oproj_in, n_experts, top_k, inter, shared_inter, dt, routed_scale,
                    norm_eps)


def validate(cfg: KKConfig, max_batch: int) -> int:
    return lib().kk_validate(ctypes.byref(cfg), max_batch)


def workspace_bytes(cfg: KKConfig, max_batch: int) -> int:
    return lib().kk_workspace_bytes(ctypes.byref(cfg), max_batch)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


class Layer:
    """One decode layer bound to device-resident weights (torch tensors, out-major); an optional
    "norm_w" [H] adds the RMSNorm before the router and the experts."""

    def __init__(self, cfg: KKConfig, weights: dict, max_batch: int):
        self.cfg, self.max_batch = cfg, max_batch
        self._weights = weights  # keep the tensors alive
        w = KKWeights(*(weights[n].data_ptr() for n in
                        ("w_o", "w_r", "router_bias", "w13", "w2", "ws13", "ws2")),
                      _ptr(weights.get("norm_w")))
        h = ctypes.c_void_p()
        _check(lib().kk_create(ctypes.byref(cfg), ctypes.byref(w), max_batch, ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None):
            lib().kk_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace_bytes(self) -> int:
        return workspace_bytes(self.cfg, self.max_batch)

    def new_workspace(self, device="cuda"):
        import torch
        return torch.empty(self.workspace_bytes(), dtype=torch.uint8, device=device)

    def query_plan(self, B: int) -> dict:
        p = KKPlan()
        _check(lib().kk_query_plan(self._h, B, ctypes.byref(p)))
        d = {n: getattr(p, n) for n, _ in KKPlan._fields_}
        d["path_name"] = PATH_NAMES.get(p.path, str(p.path))
        return d

    def oproj_residual(self, B, x, resid, h32, ws, h_out=None, stream=None):
        _check(lib().kk_oproj_residual(self._h, B, _ptr(x), _ptr(resid), _ptr(h32), _ptr(h_out),
                                       _ptr(ws), _stream(stream)))

    def router_topk(self, B, h32, topk_idx, topk_gate, expert_offsets, perm, ws, stream=None):
        _check(lib().kk_router_topk(self._h, B, _ptr(h32), _ptr(topk_idx), _ptr(topk_gate),
                                    _ptr(expert_offsets), _ptr(perm), _ptr(ws), _stream(stream)))

    def moe_decode(self, B, h32, topk_idx, topk_gate, expert_offsets, perm, out, ws, stream=None):
        _check(lib().kk_moe_decode(self._h, B, _ptr(h32), _ptr(topk_idx), _ptr(topk_gate),
                                   _ptr(expert_offsets), _ptr(perm), _ptr(out), _ptr(ws),
                                   _stream(stream)))

    def routing_status(self, ws, stream=None):
        """Raises KKError(KK_ERR_INVALID_ARG) if the last moe_decode on ws was given invalid
        routing tables (waits for the stream)."""
        _check(lib().kk_routing_status(self._h, _ptr(ws), _stream(stream)))

    def layer_decode(self, B, x, resid, out, ws, topk_idx=None, topk_gate=None, stream=None,
                     graph=False, two_stream=False):
        flags = (KK_GRAPH if graph else 0) | (KK_TWO_STREAM if two_stream else 0)
        _check(lib().kk_layer_decode(self._h, B, _ptr(x), _ptr(resid), _ptr(out), _ptr(topk_idx),
                                     _ptr(topk_gate), _ptr(ws), _stream(stream), flags))

    def layer_decode_static(self, B, x, resid, out, topk_idx=None, topk_gate=None, stream=None,
                            two_stream=False):
        """kk_layer_decode_static: the step with the library's static scratch (no workspace)."""
        flags = KK_TWO_STREAM if two_stream else 0
        _check(lib().kk_layer_decode_static(self._h, B, _ptr(x), _ptr(resid), _ptr(out),
                                            _ptr(topk_idx), _ptr(topk_gate), _stream(stream), flags))

    def set_stream_delay(self, which: int, microseconds: float):
        """Test hook: a bounded wait first on the main (0) or auxiliary (1) stream of each step."""
        _check(lib().kk_set_stream_delay(self._h, which, float(microseconds)))

    def set_kernel_timing(self, enable: bool):
        _check(lib().kk_set_kernel_timing(self._h, 1 if enable else 0))

    def read_kernel_timing(self, cap: int = 4096) -> list[tuple[str, float]]:
        names = (ctypes.c_char_p * cap)()
        ms = (ctypes.c_float * cap)()
        n = ctypes.c_int32()
        _check(lib().kk_read_kernel_timing(self._h, names, ms, cap, ctypes.byref(n)))
        return [(names[i].decode(), ms[i]) for i in range(min(n.value, cap))]


def chain_decode(layers, B, xs, resid, outs, ws, stream=None, graph=False, prefetch=False):
    """kk_chain_decode over Layer objects: layer l reads xs[l] and the previous layer's output
    (resid for the first) and writes outs[l]."""
    n = len(layers)
    if not (len(xs) == len(outs) == n):
        raise ValueError("one x and one out per layer")
    ctxs = (ctypes.c_void_p * n)(*[layer._h.value for layer in layers])
    xa = (ctypes.c_void_p * n)(*[t.data_ptr() for t in xs])
    oa = (ctypes.c_void_p * n)(*[t.data_ptr() for t in outs])
    flags = (KK_GRAPH if graph else 0) | (KK_PREFETCH if prefetch else 0)
    _check(lib().kk_chain_decode(ctxs, n, B, xa, _ptr(resid), oa, _ptr(ws), _stream(stream), flags))
