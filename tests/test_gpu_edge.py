"""GPU edge cases of the method against the fp64 oracle: a router with every key equal (the
tie rule decides the whole selection) and a layer whose experts are all zero (the output is
the residual stream itself), on both paths.
"""
import numpy as np
import pytest

import oracle as O
import synth
from tests.gpu_common import (as_f64_out, assert_close, gpu_layer, host_layer_weights, log)

pytestmark = pytest.mark.gpu

CASES = [("tiny_fp32", 1), ("tp_rank", 1), ("tp_rank", 2), ("tp_rank", 8)]


def _layer_with(name, replace):
    """A kk.Layer over the workload's device weights with some tensors replaced."""
    from moe_layer_skinny_amd import kk
    cfg, w, _ = gpu_layer(name)
    w2 = dict(w)
    w2.update(replace)
    kcfg = kk.make_config(cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.top_k, cfg.inter,
                          cfg.shared_inter, cfg.dtype)
    return cfg, w2, kk.Layer(kcfg, w2, cfg.max_batch)


def _run(L, cfg, B):
    import torch
    import synth.device as sd
    x, r, _, _ = sd.device_tokens(cfg, B)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty(B, cfg.hidden, dtype=dt, device="cuda")
    idx = torch.full((B, cfg.top_k), -1, dtype=torch.int32, device="cuda")
    gate = torch.zeros(B, cfg.top_k, dtype=torch.float32, device="cuda")
    h32 = torch.empty(B, cfg.hidden, dtype=torch.float32, device="cuda")
    h_out = torch.empty(B, cfg.hidden, dtype=dt, device="cuda")
    ws = L.new_workspace()
    L.layer_decode(B, x, r, out, ws, idx, gate)
    L.oproj_residual(B, x, r, h32, ws, h_out=h_out)
    torch.cuda.synchronize()
    return out, idx, gate, h_out


@pytest.mark.parametrize("name,B", CASES)
def test_all_keys_equal_select_lowest_indices(name, B):
    """W_r = 0 and b = 0: every score is 1/2, every key equal; the lower expert index wins
    each tie, so experts 0..k-1 are selected with gates exactly 1/k."""
    log(f"[ties] {name} B={B}")
    import torch
    cfg, w, _ = gpu_layer(name)
    zr = torch.zeros_like(w["w_r"])
    zb = torch.zeros_like(w["router_bias"])
    cfg, _, L = _layer_with(name, {"w_r": zr, "router_bias": zb})
    try:
        out, idx, gate, _ = _run(L, cfg, B)
    finally:
        L.close()
    k = cfg.top_k
    np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(k, dtype=np.int32), (B, 1)))
    np.testing.assert_array_equal(gate.cpu().numpy(), np.full((B, k), 1.0 / k, dtype=np.float32))
    hw = host_layer_weights(name)
    zw = O.LayerWeights(hw.w_o, np.zeros_like(hw.w_r), np.zeros_like(hw.bias), hw.expert,
                        *hw.shared())
    x, r = synth.host_tokens(cfg, B)
    ref = O.layer_step(x, r, zw, k)
    np.testing.assert_array_equal(ref["topk_idx"], idx.cpu().numpy())
    rep = assert_close(as_f64_out(out), ref["out"], "out with tied keys")
    log(f"[ties] {name} B={B}: {rep}")


@pytest.mark.parametrize("name,B", CASES)
def test_zero_experts_leave_the_residual_stream(name, B):
    """All routed and shared expert weights 0: out = RNE(h32), bit for bit the o-proj output."""
    log(f"[zero-experts] {name} B={B}")
    import torch
    cfg, w, _ = gpu_layer(name)
    zeros = {n: torch.zeros_like(w[n]) for n in ("w13", "w2", "ws13", "ws2")}
    cfg, _, L = _layer_with(name, zeros)
    try:
        out, idx, _, h_out = _run(L, cfg, B)
    finally:
        L.close()
        del zeros
        torch.cuda.empty_cache()
    assert torch.equal(out, h_out)
    assert (idx.cpu().numpy() >= 0).all()


MAX_CASES = [("tp_max", 1), ("tp_max", 2), ("tp_max", 64)]


@pytest.mark.parametrize("name,B", MAX_CASES)
def test_largest_routing(name, B):
    """512 experts, top-16 and 64 tokens (1024 slots): the routing-table and on-chip limits of
    both paths, through the whole step and through the three ops on their own."""
    log(f"[max] {name} B={B}")
    import torch
    import synth.device as sd
    from tests.gpu_common import assert_routing_equal, oracle_step
    cfg, _, L = gpu_layer(name)
    assert (cfg.n_experts, cfg.top_k) == (512, 16)
    ref = oracle_step(name, B)
    out, idx, gate, _ = _run(L, cfg, B)
    rep = assert_close(as_f64_out(out), ref["out"], "layer out")
    assert_routing_equal({"topk_idx": idx.cpu().numpy(), "topk_gate": gate.cpu().numpy()}, ref, B,
                         cfg.top_k, "layer routing")
    log(f"[max] {name} B={B} layer: {rep}")
    x, r, _, _ = sd.device_tokens(cfg, B)
    h32 = torch.empty(B, cfg.hidden, dtype=torch.float32, device="cuda")
    offsets = torch.full((cfg.n_experts + 1,), -1, dtype=torch.int32, device="cuda")
    perm = torch.full((B * cfg.top_k,), -1, dtype=torch.int32, device="cuda")
    out2 = torch.empty_like(out)
    ws = L.new_workspace()
    L.oproj_residual(B, x, r, h32, ws)
    L.router_topk(B, h32, idx, gate, offsets, perm, ws)
    L.moe_decode(B, h32, idx, gate, offsets, perm, out2, ws)
    torch.cuda.synchronize()
    assert_routing_equal({"topk_idx": idx.cpu().numpy(), "topk_gate": gate.cpu().numpy(),
                          "offsets": offsets.cpu().numpy(), "perm": perm.cpu().numpy()}, ref, B,
                         cfg.top_k, "router tables")
    assert_close(as_f64_out(out2), ref["out"], "moe out")


@pytest.mark.parametrize("B", [1, 2])
def test_every_expert_selected(B):
    """k = E (the dense special case): every expert is selected for every token, in index
    order, with gates s / sum of all s; the layer output matches the oracle run with k = E."""
    log(f"[dense] tiny_fp32 k=E B={B}")
    import torch
    import synth.device as sd
    from moe_layer_skinny_amd import kk
    cfg, w, _ = gpu_layer("tiny_fp32")
    E = cfg.n_experts
    kcfg = kk.make_config(cfg.hidden, cfg.oproj_in, E, E, cfg.inter, cfg.shared_inter, cfg.dtype)
    L = kk.Layer(kcfg, w, 2)
    try:
        # with k = E no top-k boundary exists, so the first draw of every token serves
        x, r, xh, rh = sd.device_tokens(cfg, B, attempts=[0] * B)
        out = torch.empty(B, cfg.hidden, dtype=torch.float32, device="cuda")
        idx = torch.full((B, E), -1, dtype=torch.int32, device="cuda")
        gate = torch.zeros(B, E, dtype=torch.float32, device="cuda")
        ws = L.new_workspace()
        L.layer_decode(B, x, r, out, ws, idx, gate)
        torch.cuda.synchronize()
    finally:
        L.close()
    ref = O.layer_step(xh, rh, host_layer_weights("tiny_fp32"), E)
    np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(E, dtype=np.int32), (B, 1)))
    np.testing.assert_allclose(gate.cpu().numpy(), ref["topk_gate"], rtol=0, atol=1e-5)
    assert_close(as_f64_out(out), ref["out"], "dense-case out")
