"""GPU parity of the layer with the RMSNorm before the router and the experts, against the fp64
oracle, on both paths: the GEMV launches normalise the rows they stage (batch 1-2), the split-K
path normalises in the o-proj's reduce launch, or in a launch of its own when the router or
the experts are called on their own (batch 3-64).
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_common import (as_f64_out, assert_close, assert_routing_equal, gpu_layer,
                              host_layer_weights, log, oracle_step)

pytestmark = pytest.mark.gpu

CASES = [("tiny_norm", 1), ("tiny_norm", 2), ("tp_norm", 1), ("tp_norm", 2), ("tp_norm", 8),
         ("tp_norm", 64), ("full_norm", 1), ("full_norm", 8)]


def _bufs(cfg, B):
    import torch
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    return {
        "h32": torch.empty(B, cfg.hidden, dtype=torch.float32, device="cuda"),
        "h_out": torch.empty(B, cfg.hidden, dtype=dt, device="cuda"),
        "out": torch.empty(B, cfg.hidden, dtype=dt, device="cuda"),
        "idx": torch.full((B, cfg.top_k), -1, dtype=torch.int32, device="cuda"),
        "gate": torch.zeros(B, cfg.top_k, dtype=torch.float32, device="cuda"),
        "offsets": torch.full((cfg.n_experts + 1,), -1, dtype=torch.int32, device="cuda"),
        "perm": torch.full((B * cfg.top_k,), -1, dtype=torch.int32, device="cuda"),
    }


@pytest.mark.parametrize("name,B", CASES)
def test_norm_layer_parity(name, B):
    log(f"[norm-layer] {name} B={B}")
    import torch
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    assert cfg.norm
    ref = oracle_step(name, B)
    x, r, _, _ = sd.device_tokens(cfg, B)
    b = _bufs(cfg, B)
    ws = L.new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"], stream=s)
    s.synchronize()
    eager = b["out"].clone()
    rep = assert_close(as_f64_out(eager), ref["out"], "layer out")
    assert_routing_equal({"topk_idx": b["idx"].cpu().numpy(), "topk_gate": b["gate"].cpu().numpy()},
                         ref, B, cfg.top_k, "layer routing")
    log(f"[norm-layer] {name} B={B}: {rep}")
    gemv = L.query_plan(B)["path_name"] == "gemv"
    runs = [(True, False), (True, False)] + ([(False, True), (True, True)] if gemv else [])
    for graph, two in runs:
        b["out"].zero_()
        with torch.cuda.stream(s):
            L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"], stream=s, graph=graph,
                           two_stream=two)
        s.synchronize()
        assert torch.equal(b["out"], eager), f"graph={graph} two_stream={two} differs (bitwise)"
    if cfg.hidden * cfg.inter <= 7168 * 128:
        # the norm really ran: the gates (scores of u, not of h) sit far from those of the same
        # layer without its norm, and an fp32 output far closer to the normalised reference
        hw = host_layer_weights(name)
        plain = O.LayerWeights(hw.w_o, hw.w_r, hw.bias, hw.expert, *hw.shared())
        xh, rh = synth.host_tokens(cfg, B)
        ref0 = O.layer_step(xh, rh, plain, cfg.top_k)
        gate = b["gate"].cpu().numpy()
        same_sets = np.array_equal(ref0["topk_idx"], b["idx"].cpu().numpy())
        assert not same_sets or np.abs(gate - ref0["topk_gate"]).max() > 1e-4
        if cfg.dtype == "f32":
            d_gpu = np.abs(as_f64_out(eager) - ref["out"]).max()
            assert d_gpu < 0.01 * np.abs(ref0["out"] - ref["out"]).max()


@pytest.mark.parametrize("name,B", CASES)
def test_norm_per_op_parity(name, B):
    """Router and experts called on their own from the caller's h32 normalise it themselves."""
    log(f"[norm-ops] {name} B={B}")
    import torch
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    ref = oracle_step(name, B)
    x, r, _, _ = sd.device_tokens(cfg, B)
    b = _bufs(cfg, B)
    ws = L.new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.oproj_residual(B, x, r, b["h32"], ws, h_out=b["h_out"], stream=s)
        L.router_topk(B, b["h32"], b["idx"], b["gate"], b["offsets"], b["perm"], ws, stream=s)
        L.moe_decode(B, b["h32"], b["idx"], b["gate"], b["offsets"], b["perm"], b["out"], ws,
                     stream=s)
    s.synchronize()
    assert_close(b["h32"].cpu().numpy().astype(np.float64), ref["h"], "h32 (residual stream)")
    assert_close(as_f64_out(b["h_out"]), ref["h"], "h_out")
    got = {"topk_idx": b["idx"].cpu().numpy(), "topk_gate": b["gate"].cpu().numpy(),
           "offsets": b["offsets"].cpu().numpy(), "perm": b["perm"].cpu().numpy()}
    assert_routing_equal(got, ref, B, cfg.top_k, "router")
    rep = assert_close(as_f64_out(b["out"]), ref["out"], "moe out")
    log(f"[norm-ops] {name} B={B}: {rep}")


def test_norm_plan_launch_counts_unchanged():
    """The norm adds no launch to a layer step on either path."""
    log("[norm-plan] tp_norm")
    _, _, L = gpu_layer("tp_norm")
    assert L.query_plan(1)["kernels_per_step"] == 4
    # K-split gate/up (its chunks summed by the down-projection up to 16 tokens)
    assert L.query_plan(8)["kernels_per_step"] == 7
    assert L.query_plan(64)["kernels_per_step"] == 9  # pieces over K chunks + SwiGLU
