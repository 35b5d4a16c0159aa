"""Seeded synthetic inputs for the MoE decode-layer step (shared by tests, bench and smoke).

This module is the only code that both the fp64 oracle's callers and the HIP path's
callers use.  It draws numbers and lays them out; it holds none of the layer's arithmetic
(no projection, routing or activation function).

Generator: Philox4x32-10 (Salmon et al., SC'11), implemented twice from its published
definition -- in C for the host (``philox_host.c``) and in HIP for the device
(``fill_device.hip``) -- so that the ~34 GB of routed-expert weights can be filled in HBM
while the oracle regenerates exactly the experts it needs on the host.  Element n of the
stream (key0, key1) is one normal draw N(0, sigma^2): the Box-Muller transform (Box and
Muller, 1958) of two uniforms taken from the Philox words of counter (n, 0, 0), with its
logarithm, square root and cosine written out from single IEEE double operations in the same
order on both sides (no fused multiply-add), so host and device give the same bits; the draw
is rounded RNE to fp32 and, for bf16 tensors, RNE to bf16.

Workload shapes follow the layer description (hidden 7168, 384 experts top-8, SwiGLU
intermediate 2048, a tensor-parallel rank's share with o-proj slice 448 and intermediate 128,
and a tiny fp32 layer); the per-token resample attempts that keep the top-k boundary gap
>= 1e-3 are stored in ``tests/golden/attempts.json`` (written by a script that calls the
oracle).
"""
from __future__ import annotations

import ctypes
import json
import math
import os
import subprocess
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_HERE)
HOST_LIB = os.path.join(_HERE, "libsynth_host.so")
DEV_LIB = os.path.join(_HERE, "libsynth_dev.so")
ATTEMPTS_JSON = os.path.join(_ROOT, "tests", "golden", "attempts.json")

# Tensor stream ids (key1) for weights; key0 is the layer seed.
T_WO, T_WR, T_BIAS, T_W13, T_W2, T_WS13, T_WS2, T_PERM, T_NORM = 1, 2, 3, 4, 5, 6, 7, 8, 9
# Token streams: key0 = token seed, key1 = TOKEN_BASE + 16 * attempt + kind (+ LAYER_STRIDE *
# layer for the attention-output stand-in x of layer >= 1 of a chain).
TOKEN_BASE = 0x100
KIND_X, KIND_R = 0, 1
LAYER_STRIDE = 0x1000
# Speculative-verify tokens (one sequence): a component shared by all tokens, stream
# (VERIFY_SEED, TOKEN_BASE + kind), mixed with each token's own stream as
# sqrt(VERIFY_RHO) * shared + sqrt(1 - VERIFY_RHO) * own.
VERIFY_SEED = 0x5EED
VERIFY_RHO = 0.9

WEIGHT_SIGMA = 0.02
ACT_SIGMA = 1.0
BIAS_SIGMA = 0.1
# RMSNorm weight: 1 + a draw of this standard deviation per channel
NORM_SIGMA = 0.1
NORM_EPS = 1e-6
ZIPF_S = 1.2


def scale_for(sigma: float) -> float:
    """The generators' scale argument: the standard deviation of the normal draw itself."""
    return float(sigma)


@dataclass(frozen=True)
class LayerConfig:
    name: str
    hidden: int
    oproj_in: int
    n_experts: int
    top_k: int
    inter: int
    shared_inter: int
    dtype: str  # "f32" or "bf16" (weights, x, r, out)
    batches: tuple
    bias: str  # "normal" | "zero" | "zipf"
    gap_space: str  # "key" | "logit"
    layer_seed: int = 0
    description: str = ""
    tokens: str = "independent"  # "independent" | "verify" (correlated tokens of one sequence)
    norm: bool = False  # RMSNorm (weight [H], eps NORM_EPS) between the residual add and experts
    layers: int = 1  # > 1: a chain of layers, layer l with weights of layer seed layer_seed + l

    @property
    def wbytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def max_batch(self) -> int:
        return max(self.batches)


CONFIGS = {
    c.name: c
    for c in [
        LayerConfig("tiny_fp32", 256, 256, 16, 2, 128, 128, "f32", (1,), "normal", "key",
                    description="tiny fp32 layer, batch 1"),
        LayerConfig("full_b1", 7168, 7168, 384, 8, 2048, 2048, "bf16", (1,), "normal", "key",
                    description="full-size layer, batch 1 (GEMV path)"),
        LayerConfig("full_b8", 7168, 7168, 384, 8, 2048, 2048, "bf16", (8,), "normal", "key",
                    description="full-size layer, batch 8, token seeds 0-7"),
        LayerConfig("full_b64", 7168, 7168, 384, 8, 2048, 2048, "bf16", (64,), "zero", "logit",
                    description="full-size layer, batch 64, uniform router bias"),
        LayerConfig("tp_rank", 7168, 448, 384, 8, 128, 128, "bf16", (1, 2, 8, 64), "zipf", "key",
                    description="one TP16 rank's share, Zipf(1.2) router bias, batch sweep"),
        LayerConfig("verify_b8", 7168, 7168, 384, 8, 2048, 2048, "bf16", (8,), "normal", "key",
                    description="full-size layer, speculative-verify batch: 8 correlated tokens "
                                "of one sequence (shared component, rho 0.9)",
                    tokens="verify"),
        LayerConfig("tiny_norm", 256, 256, 16, 2, 128, 128, "f32", (1, 2), "normal", "key",
                    description="tiny fp32 layer with RMSNorm before router and experts",
                    norm=True),
        LayerConfig("full_norm", 7168, 7168, 384, 8, 2048, 2048, "bf16", (1, 8), "normal", "key",
                    description="full-size layer with RMSNorm before router and experts",
                    norm=True),
        LayerConfig("tp_norm", 7168, 448, 384, 8, 128, 128, "bf16", (1, 2, 8, 64), "zipf", "key",
                    description="one TP16 rank's share with RMSNorm before router and experts",
                    norm=True),
        LayerConfig("tp_max", 7168, 448, 512, 16, 128, 128, "bf16", (1, 2, 64), "zipf", "key",
                    description="the largest routing the kernels take: 512 experts, top-16, "
                                "up to 64 tokens (1024 slots), TP16-rank expert shapes"),
        # chained layers carry the RMSNorm: without it the residual stream of random layers
        # grows layer by layer until the sigmoid scores saturate
        LayerConfig("chain_tp", 7168, 448, 384, 8, 128, 128, "bf16", (1, 2, 8), "zipf", "key",
                    description="four consecutive TP16-rank layers with distinct weights, "
                                "RMSNorm before router and experts", norm=True, layers=4),
        LayerConfig("chain_full", 7168, 7168, 384, 8, 2048, 2048, "bf16", (1, 8), "normal",
                    "key", description="two consecutive full-size layers with distinct weights, "
                                       "RMSNorm before router and experts", norm=True, layers=2),
    ]
}


def layer_of(cfg: LayerConfig, l: int) -> LayerConfig:
    """Layer l of a chain as a one-layer config (its own weights: layer seed + l)."""
    if not 0 <= l < cfg.layers:
        raise ValueError(f"{cfg.name} has {cfg.layers} layers")
    return replace(cfg, name=f"{cfg.name}.{l}", layer_seed=cfg.layer_seed + l, layers=1)


# ----------------------------------------------------------------------------- host library
_host = None


def _build_host_lib() -> None:
    src = os.path.join(_HERE, "philox_host.c")
    tmp = HOST_LIB + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC", src,
                           "-o", tmp])
    os.replace(tmp, HOST_LIB)


def build(force: bool = True) -> None:
    """Compile the host generator (gcc) and the device fill (hipcc, gfx950)."""
    if force or not os.path.exists(HOST_LIB):
        _build_host_lib()
    if force or not os.path.exists(DEV_LIB):
        src = os.path.join(_HERE, "fill_device.hip")
        tmp = DEV_LIB + ".tmp"
        subprocess.check_call(["hipcc", "--offload-arch=gfx950", "-O3", "-shared", "-fPIC",
                               "-ffp-contract=off",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               src, "-o", tmp], stderr=subprocess.DEVNULL)
        os.replace(tmp, DEV_LIB)


def _lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_LIB):
            _build_host_lib()
        lib = ctypes.CDLL(HOST_LIB)
        lib.synth_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                   ctypes.c_uint32, ctypes.c_uint32, ctypes.c_double]
        lib.synth_fill.restype = None
        lib.synth_u32.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint64,
                                  ctypes.c_uint32, ctypes.c_uint32]
        lib.synth_u32.restype = None
        lib.synth_philox4x32_10.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_philox4x32_10.restype = None
        _host = lib
    return _host


def philox4x32_10(counter, key):
    """Raw Philox4x32-10 block: 4 counter words, 2 key words -> 4 output words."""
    c = np.asarray(counter, dtype=np.uint32).copy()
    k = np.asarray(key, dtype=np.uint32).copy()
    out = np.zeros(4, dtype=np.uint32)
    _lib().synth_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def host_stream(count: int, key0: int, key1: int, sigma: float, dtype: str, first: int = 0):
    """Elements first..first+count-1 of stream (key0, key1): float32 array or bf16 bits (uint16)."""
    if dtype == "f32":
        out = np.empty(count, dtype=np.float32)
        code = 0
    elif dtype == "bf16":
        out = np.empty(count, dtype=np.uint16)
        code = 1
    else:
        raise ValueError(dtype)
    if count:
        _lib().synth_fill(out.ctypes.data, code, first, count, key0 & 0xFFFFFFFF, key1 & 0xFFFFFFFF,
                          scale_for(sigma))
    return out


def host_u32(count: int, key0: int, key1: int, first: int = 0):
    out = np.empty(count, dtype=np.uint32)
    if count:
        _lib().synth_u32(out.ctypes.data, first, count, key0, key1)
    return out


# ----------------------------------------------------------------------------- layer tensors
def weight_spec(cfg: LayerConfig):
    """name -> (shape, stream id, sigma).  Out-major layouts (each output row contiguous)."""
    H, Ko, E, I, Is = cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.inter, cfg.shared_inter
    return {
        "w_o": ((H, Ko), T_WO, WEIGHT_SIGMA),
        "w_r": ((E, H), T_WR, WEIGHT_SIGMA),
        "w13": ((E, 2 * I, H), T_W13, WEIGHT_SIGMA),
        "w2": ((E, H, I), T_W2, WEIGHT_SIGMA),
        "ws13": ((2 * Is, H), T_WS13, WEIGHT_SIGMA),
        "ws2": ((H, Is), T_WS2, WEIGHT_SIGMA),
    }


def host_weight(cfg: LayerConfig, name: str):
    shape, tid, sigma = weight_spec(cfg)[name]
    n = int(np.prod(shape))
    return host_stream(n, cfg.layer_seed, tid, sigma, cfg.dtype).reshape(shape)


def host_expert(cfg: LayerConfig, e: int):
    """(w13_e [2I][H], w2_e [H][I]) of routed expert e, generated on the host."""
    H, I = cfg.hidden, cfg.inter
    n13, n2 = 2 * I * H, H * I
    w13 = host_stream(n13, cfg.layer_seed, T_W13, WEIGHT_SIGMA, cfg.dtype, first=e * n13)
    w2 = host_stream(n2, cfg.layer_seed, T_W2, WEIGHT_SIGMA, cfg.dtype, first=e * n2)
    return w13.reshape(2 * I, H), w2.reshape(H, I)


def host_norm_weight(cfg: LayerConfig):
    """RMSNorm weight [H] in the config dtype: 1 + NORM_SIGMA-scaled draw, fp64 -> fp32 -> dtype."""
    if not cfg.norm:
        return None
    d = host_stream(cfg.hidden, cfg.layer_seed, T_NORM, NORM_SIGMA, "f32").astype(np.float64)
    v = (1.0 + d).astype(np.float32)
    return f32_to_bf16_bits(v) if cfg.dtype == "bf16" else v


def host_bias(cfg: LayerConfig):
    """Router bias, fp32 [E]."""
    E = cfg.n_experts
    if cfg.bias == "normal":
        return host_stream(E, cfg.layer_seed, T_BIAS, BIAS_SIGMA, "f32")
    if cfg.bias == "zero":
        return np.zeros(E, dtype=np.float32)
    if cfg.bias == "zipf":
        # Zipf(s) probability mass over ranks 1..E, placed through a random permutation of
        # the experts (rank r -> expert perm[r-1]); permutation = experts ordered by a
        # Philox draw, ties by index.
        u = host_u32(E, cfg.layer_seed, T_PERM)
        perm = np.lexsort((np.arange(E), u))
        ranks = np.arange(1, E + 1, dtype=np.float64)
        pmf = ranks ** (-ZIPF_S)
        pmf /= pmf.sum()
        b = np.empty(E, dtype=np.float64)
        b[perm] = pmf
        return b.astype(np.float32)
    raise ValueError(cfg.bias)


def token_key(attempt: int, kind: int, layer: int = 0) -> int:
    return TOKEN_BASE + LAYER_STRIDE * int(layer) + 16 * int(attempt) + kind


def f32_to_bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return np.where(nan, ((u >> 16) | 0x40).astype(np.uint16), r)


def host_token(cfg: LayerConfig, t: int, attempt: int):
    """(x_t [Ko], r_t [H]) for token seed t, resample attempt `attempt`.

    Independent tokens draw each vector from the token's own stream.  Verify tokens mix a
    component shared by the whole batch with the token's own stream (fp32 draws, mixed in
    fp64, rounded to fp32 and then to the config dtype); a resample redraws only the token's
    own part.
    """
    if cfg.tokens == "independent":
        x = host_stream(cfg.oproj_in, t, token_key(attempt, KIND_X), ACT_SIGMA, cfg.dtype)
        r = host_stream(cfg.hidden, t, token_key(attempt, KIND_R), ACT_SIGMA, cfg.dtype)
        return x, r
    if cfg.tokens != "verify":
        raise ValueError(cfg.tokens)
    out = []
    for n, kind in ((cfg.oproj_in, KIND_X), (cfg.hidden, KIND_R)):
        shared = host_stream(n, VERIFY_SEED, token_key(0, kind), ACT_SIGMA, "f32")
        own = host_stream(n, t, token_key(attempt, kind), ACT_SIGMA, "f32")
        v = (np.sqrt(VERIFY_RHO) * shared.astype(np.float64) +
             np.sqrt(1.0 - VERIFY_RHO) * own.astype(np.float64)).astype(np.float32)
        out.append(f32_to_bf16_bits(v) if cfg.dtype == "bf16" else v)
    return out[0], out[1]


def host_chain_x(cfg: LayerConfig, l: int, t: int, attempt: int):
    """x_l [Ko] of token seed t for layer l >= 1 of a chain (the stand-in for that layer's
    attention output), resample attempt `attempt`."""
    if cfg.tokens != "independent" or l < 1:
        raise ValueError("chain inputs past layer 0 are independent per-layer draws")
    return host_stream(cfg.oproj_in, t, token_key(attempt, KIND_X, l), ACT_SIGMA, cfg.dtype)


def host_chain_tokens(cfg: LayerConfig, B: int, table: dict | None = None):
    """([x_0 .. x_{L-1}] each [B][Ko], r_0 [B][H]) of a chain for token seeds 0..B-1."""
    x0, r0 = host_tokens(cfg, B, attempts_for(cfg, B, table))
    xs = [x0]
    table = load_attempts() if table is None else table
    per_layer = table["configs"][cfg.name]["layer_attempts"]
    for l in range(1, cfg.layers):
        xs.append(np.stack([host_chain_x(cfg, l, t, per_layer[l - 1][t]) for t in range(B)]))
    return xs, r0


def load_attempts(path: str = ATTEMPTS_JSON) -> dict:
    with open(path) as f:
        return json.load(f)


def attempts_for(cfg: LayerConfig, B: int, table: dict | None = None):
    table = load_attempts() if table is None else table
    ent = table["configs"][cfg.name]["attempts"]
    if B > len(ent):
        raise ValueError(f"{cfg.name}: attempts stored for {len(ent)} tokens, asked for {B}")
    return [int(a) for a in ent[:B]]


def host_tokens(cfg: LayerConfig, B: int, attempts=None):
    """x [B][Ko], r [B][H] for token seeds 0..B-1 (attempts from the stored table by default)."""
    if attempts is None:
        attempts = attempts_for(cfg, B)
    xs, rs = zip(*(host_token(cfg, t, attempts[t]) for t in range(B)))
    return np.stack(xs), np.stack(rs)


def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------- device fill
_dev = None


def _dev_lib():
    global _dev
    if _dev is None:
        if not os.path.exists(DEV_LIB):
            raise RuntimeError(f"{DEV_LIB} is not built: run __graft_entry__.build()")
        lib = ctypes.CDLL(DEV_LIB)
        lib.synth_dev_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                       ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_double, ctypes.c_void_p]
        lib.synth_dev_fill.restype = ctypes.c_int
        _dev = lib
    return _dev


def device_stream(ptr: int, count: int, key0: int, key1: int, sigma: float, dtype: str,
                  first: int = 0, stream: int = 0) -> None:
    """Fill `count` elements at device address `ptr` with elements first.. of stream (key0, key1)."""
    code = {"f32": 0, "bf16": 1}[dtype]
    rc = _dev_lib().synth_dev_fill(ptr, code, first, count, key0 & 0xFFFFFFFF, key1 & 0xFFFFFFFF,
                                   scale_for(sigma), stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_fill failed: hip error {rc}")


def device_weight(cfg: LayerConfig, name: str, ptr: int, stream: int = 0) -> None:
    shape, tid, sigma = weight_spec(cfg)[name]
    device_stream(ptr, int(np.prod(shape)), cfg.layer_seed, tid, sigma, cfg.dtype, stream=stream)
