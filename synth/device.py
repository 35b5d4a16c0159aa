"""Device-resident synthetic layers and tokens (torch tensors filled by synth's generators).

Weights are filled in HBM by the device Philox fill (bit-identical to the host generator),
so a full-size layer (~34 GB of routed experts) never crosses PCIe.  Tokens and the router
bias are generated on the host and copied.  Holds no arithmetic of the layer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import (LayerConfig, device_stream, host_bias, host_norm_weight, host_tokens, weight_spec)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def device_weights(cfg: LayerConfig, device="cuda", share_from: dict | None = None) -> dict:
    """w_o, w_r, router_bias, w13, w2, ws13, ws2 (and norm_w with a norm) as device tensors.

    ``share_from``: reuse the weight tensors of another config with the same shapes and layer
    seed (only the router bias differs between such workloads).
    """
    out = {}
    dt = _TORCH_DTYPE[cfg.dtype]
    stream = torch.cuda.current_stream(device).cuda_stream
    for name, (shape, tid, sigma) in weight_spec(cfg).items():
        if share_from is not None:
            out[name] = share_from[name]
            continue
        t = torch.empty(shape, dtype=dt, device=device)
        device_stream(t.data_ptr(), t.numel(), cfg.layer_seed, tid, sigma, cfg.dtype, stream=stream)
        out[name] = t
    out["router_bias"] = torch.from_numpy(host_bias(cfg)).to(device)
    if cfg.norm:
        out["norm_w"] = host_to_device(host_norm_weight(cfg), cfg.dtype, device)
    torch.cuda.synchronize(device)
    return out


def host_to_device(a: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """uint16 bf16 bits or float32 host array -> device tensor of the config dtype."""
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def device_chain_tokens(cfg: LayerConfig, B: int, device="cuda"):
    """([x_l device tensors], r_0 device tensor) of a chain and their host copies."""
    from . import host_chain_tokens
    xs, r0 = host_chain_tokens(cfg, B)
    return ([host_to_device(x, cfg.dtype, device) for x in xs], host_to_device(r0, cfg.dtype, device),
            xs, r0)


def device_tokens(cfg: LayerConfig, B: int, attempts=None, device="cuda"):
    """(x [B][Ko], r [B][H]) device tensors and their host bits/values."""
    x, r = host_tokens(cfg, B, attempts)
    return host_to_device(x, cfg.dtype, device), host_to_device(r, cfg.dtype, device), x, r


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    """bf16 device tensor -> uint16 bit array; fp32 -> float32 array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()
