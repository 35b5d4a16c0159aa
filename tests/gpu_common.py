"""Shared set-up for the GPU parity tests: device layers, oracle results, tolerance checks.

Inputs come only from synth (device fill for weights, host draws for tokens); expected
values come only from the fp64 oracle run on host-generated copies of the same inputs.
"""
from __future__ import annotations

import functools
import sys

import numpy as np

import oracle as O
import synth

# Tolerance of the layer's outputs (bf16 out, fp32 accumulation): elementwise
# |gpu - ref| <= ABS + REL * |ref|  (max relative 2e-2 / max absolute 1e-2, allclose form).
TOL_ABS, TOL_REL = 1e-2, 2e-2
GATE_TOL = 1e-5

_layers: dict = {}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def gpu_layer(name: str, cfg=None):
    """(cfg, weights dict, kk.Layer) for a workload (or a given one-layer config under `name`);
    workloads with the same shapes and layer seed share weight tensors."""
    if name in _layers:
        return _layers[name]
    import synth.device as sd
    from moe_layer_skinny_amd import kk
    cfg = synth.CONFIGS[name] if cfg is None else cfg
    share = None
    for other, (ocfg, ow, _) in _layers.items():
        if (ocfg.hidden, ocfg.oproj_in, ocfg.n_experts, ocfg.inter, ocfg.dtype, ocfg.layer_seed) == (
                cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.inter, cfg.dtype, cfg.layer_seed):
            share = ow
            break
    log(f"[gpu_layer] {name}: filling weights on device (shared={share is not None})")
    w = sd.device_weights(cfg, share_from=share)
    kcfg = kk.make_config(cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.top_k, cfg.inter,
                          cfg.shared_inter, cfg.dtype, norm_eps=synth.NORM_EPS)
    layer = kk.Layer(kcfg, w, cfg.max_batch)
    _layers[name] = (cfg, w, layer)
    return _layers[name]


@functools.lru_cache(maxsize=None)
def host_layer_weights(name: str) -> O.LayerWeights:
    cfg = synth.CONFIGS[name]
    return O.LayerWeights(synth.host_weight(cfg, "w_o"), synth.host_weight(cfg, "w_r"),
                          synth.host_bias(cfg), lambda e: synth.host_expert(cfg, e),
                          synth.host_weight(cfg, "ws13"), synth.host_weight(cfg, "ws2"),
                          norm_weight=synth.host_norm_weight(cfg))


@functools.lru_cache(maxsize=None)
def oracle_step(name: str, B: int, out_tokens: tuple | None = None) -> dict:
    cfg = synth.CONFIGS[name]
    x, r = synth.host_tokens(cfg, B)
    return O.layer_step(x, r, host_layer_weights(name), cfg.top_k,
                        out_tokens=None if out_tokens is None else list(out_tokens),
                        norm_eps=synth.NORM_EPS)


@functools.lru_cache(maxsize=None)
def golden_out(name: str, B: int) -> np.ndarray:
    """The oracle's output [B][H] for token seeds 0..B-1 of a workload whose oracle run is too
    long for a test, read from the file tests/golden/make_expected.py wrote for a batch of at
    least B tokens (a token's output does not depend on the rest of its batch); the file's
    input fingerprint must match the current inputs."""
    from tests.golden import make_expected as me
    for name_, Bg in me.CASES:
        if name_ == name and Bg >= B:
            z = np.load(me.path_for(name_, Bg), allow_pickle=False)
            want = me.fingerprint(synth.CONFIGS[name_], Bg)
            assert str(z["fingerprint"]) == want, (
                f"{me.path_for(name_, Bg)} was written for other inputs: rerun "
                "tests/golden/make_expected.py")
            return z["out"][:B]
    raise KeyError(f"no stored oracle output for {name} at batch {B}")


def has_golden(name: str, B: int) -> bool:
    from tests.golden import make_expected as me
    return any(n == name and Bg >= B for n, Bg in me.CASES)


def as_f64_out(t) -> np.ndarray:
    torch = torch_mod()
    t = t.detach().float().cpu() if t.dtype == torch.bfloat16 else t.detach().cpu()
    return t.numpy().astype(np.float64)


def tol_report(gpu: np.ndarray, ref: np.ndarray) -> dict:
    d = np.abs(gpu - ref)
    bad = d > TOL_ABS + TOL_REL * np.abs(ref)
    big = np.abs(ref) >= 0.5
    return {"violations": int(bad.sum()), "n": int(d.size), "max_abs": float(d.max()),
            "max_rel_big": float((d[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
            "normwise": float(d.max() / max(np.abs(ref).max(), 1e-30))}


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str) -> dict:
    rep = tol_report(gpu, ref)
    assert not np.isnan(gpu).any(), f"{what}: NaN in GPU output"
    assert rep["violations"] == 0, f"{what}: {rep}"
    return rep


def assert_routing_equal(got: dict, ref: dict, B: int, k: int, what: str) -> None:
    np.testing.assert_array_equal(got["topk_idx"], ref["topk_idx"], err_msg=f"{what}: topk_idx")
    np.testing.assert_allclose(got["topk_gate"], ref["topk_gate"], rtol=0, atol=GATE_TOL,
                               err_msg=f"{what}: topk_gate")
    if "offsets" in got:
        np.testing.assert_array_equal(got["offsets"], ref["offsets"], err_msg=f"{what}: offsets")
    if "perm" in got:
        np.testing.assert_array_equal(got["perm"], ref["perm"], err_msg=f"{what}: perm")


def gpu_chain(name: str):
    """(chain cfg, [kk.Layer per layer]) for a chain workload; layer l is registered as
    "<name>.<l>" (its own weights, layer seed + l)."""
    cfg = synth.CONFIGS[name]
    layers = []
    for l in range(cfg.layers):
        lc = synth.layer_of(cfg, l)
        lc = synth.replace(lc, batches=cfg.batches)
        layers.append(gpu_layer(lc.name, lc)[2])
    return cfg, layers


@functools.lru_cache(maxsize=None)
def oracle_chain(name: str, B: int) -> list:
    cfg = synth.CONFIGS[name]
    xs, r0 = synth.host_chain_tokens(cfg, B)
    ws = []
    for l in range(cfg.layers):
        lc = synth.layer_of(cfg, l)
        ws.append(O.LayerWeights(synth.host_weight(lc, "w_o"), synth.host_weight(lc, "w_r"),
                                 synth.host_bias(lc), lambda e, lc=lc: synth.host_expert(lc, e),
                                 synth.host_weight(lc, "ws13"), synth.host_weight(lc, "ws2"),
                                 norm_weight=synth.host_norm_weight(lc)))
    return O.chain_step(xs, r0, ws, cfg.top_k, cfg.dtype, norm_eps=synth.NORM_EPS)
