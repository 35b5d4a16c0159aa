"""GPU parity of the split-K MFMA path (batch 3-64) against the fp64 oracle.

Routing tables and outputs are compared for every token.  At full size and batch 64 the
oracle's routing and h are computed in the test and its outputs are read from the file that
tests/golden/make_expected.py wrote (the ~285 experts that step touches take minutes to
regenerate on the host).
"""
import os

import numpy as np
import pytest

import synth

from tests.gpu_common import (as_f64_out, assert_close, assert_routing_equal, golden_out,
                              gpu_layer, has_golden, log, oracle_step)

pytestmark = pytest.mark.gpu

MFMA_CASES = [("tp_rank", 8), ("tp_rank", 64), ("full_b8", 8), ("verify_b8", 8), ("full_b64", 64)]


def _torch():
    import torch
    return torch


def _bufs(cfg, B):
    torch = _torch()
    return {
        "h32": torch.empty(B, cfg.hidden, dtype=torch.float32, device="cuda"),
        "h_out": torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda"),
        "out": torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda"),
        "idx": torch.full((B, cfg.top_k), -1, dtype=torch.int32, device="cuda"),
        "gate": torch.zeros(B, cfg.top_k, dtype=torch.float32, device="cuda"),
        "offsets": torch.full((cfg.n_experts + 1,), -1, dtype=torch.int32, device="cuda"),
        "perm": torch.full((B * cfg.top_k,), -1, dtype=torch.int32, device="cuda"),
    }


def _ref(name, B):
    """The oracle's step for every token (outputs from the stored file where one exists)."""
    if has_golden(name, B):
        ref = dict(oracle_step(name, B, ()))
        ref["out"] = golden_out(name, B)
    else:
        ref = oracle_step(name, B)
    return ref, list(range(B))


@pytest.mark.parametrize("name,B", MFMA_CASES)
def test_plan_is_mfma(name, B):
    log(f"[plan-mfma] {name} B={B}")
    _, _, L = gpu_layer(name)
    p = L.query_plan(B)
    assert p["path_name"] == "splitk_mfma" and p["forced"] == 0
    # a small intermediate (up to 16 tokens and over 32) splits the gate/up over K chunks, which
    # over 32 tokens adds the SwiGLU launch that sums them; over 32 tokens an unsplit gate/up
    # adds the shared expert's split-K launch and its SwiGLU
    cfg = synth.CONFIGS[name]
    split = (B <= 16 or B > 32) and cfg.inter <= 256
    # (up to 16 tokens the down-projection sums the K chunks of an intermediate of 128 itself)
    swiglu_launch = split and not (B <= 16 and cfg.inter == 128)
    want = (8 if B > 16 else 7) + swiglu_launch + (2 if B > 32 and not split else 0)
    # a 448-wide o-proj slice without a norm: the o-proj (with its residual) and the router
    # run as one launch (no reduce, no router launch), ten logit partials
    fused = cfg.oproj_in < cfg.hidden and not cfg.norm
    assert p["kernels_per_step"] == want - (2 if fused else 0)
    assert p["oproj_splitk"] == (7 if cfg.oproj_in == 7168 else 1)
    assert p["router_splitk"] == (10 if fused else 7)


@pytest.mark.parametrize("name,B", MFMA_CASES)
def test_per_op_parity_mfma(name, B):
    log(f"[ops-mfma] {name} B={B}")
    torch = _torch()
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    ref, toks = _ref(name, B)
    x, r, _, _ = sd.device_tokens(cfg, B)
    b = _bufs(cfg, B)
    ws = L.new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.oproj_residual(B, x, r, b["h32"], ws, h_out=b["h_out"], stream=s)
        L.router_topk(B, b["h32"], b["idx"], b["gate"], b["offsets"], b["perm"], ws, stream=s)
        L.moe_decode(B, b["h32"], b["idx"], b["gate"], b["offsets"], b["perm"], b["out"], ws, stream=s)
    s.synchronize()
    assert_close(b["h32"].cpu().numpy().astype(np.float64), ref["h"], "h32")
    assert_close(as_f64_out(b["h_out"]), ref["h"], "h_out")
    got = {"topk_idx": b["idx"].cpu().numpy(), "topk_gate": b["gate"].cpu().numpy(),
           "offsets": b["offsets"].cpu().numpy(), "perm": b["perm"].cpu().numpy()}
    assert_routing_equal(got, ref, B, cfg.top_k, "router")
    rep = assert_close(as_f64_out(b["out"])[toks], ref["out"][toks], "moe out")
    log(f"[ops-mfma] {name} B={B} out: {rep}")


@pytest.mark.parametrize("name,B", MFMA_CASES)
def test_layer_parity_mfma(name, B):
    log(f"[layer-mfma] {name} B={B}")
    torch = _torch()
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    ref, toks = _ref(name, B)
    x, r, _, _ = sd.device_tokens(cfg, B)
    b = _bufs(cfg, B)
    ws = L.new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"], stream=s)
    s.synchronize()
    eager = b["out"].clone()
    rep = assert_close(as_f64_out(eager)[toks], ref["out"][toks], "layer out")
    assert_routing_equal({"topk_idx": b["idx"].cpu().numpy(), "topk_gate": b["gate"].cpu().numpy()},
                         ref, B, cfg.top_k, "layer routing")
    log(f"[layer-mfma] {name} B={B} out: {rep}")
    for rep_i in range(3):
        b["out"].zero_()
        with torch.cuda.stream(s):
            L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"], stream=s, graph=rep_i > 0)
        s.synchronize()
        assert torch.equal(b["out"], eager), f"replay {rep_i} differs (bitwise)"


@pytest.mark.parametrize("B", [3, 5, 16, 17, 24, 32, 33])
def test_odd_batches_mfma(B):
    log(f"[odd-mfma] tp_rank B={B}")
    torch = _torch()
    import synth.device as sd
    cfg, _, L = gpu_layer("tp_rank")
    ref = oracle_step("tp_rank", B)
    x, r, _, _ = sd.device_tokens(cfg, B)
    b = _bufs(cfg, B)
    ws = L.new_workspace()
    assert L.query_plan(B)["path_name"] == "splitk_mfma"
    L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"])
    torch.cuda.synchronize()
    assert_close(as_f64_out(b["out"]), ref["out"], "layer out")
    np.testing.assert_array_equal(b["idx"].cpu().numpy(), ref["topk_idx"])


def test_forced_plans_are_visible_and_agree():
    log("[forced] tp_rank B=2 mfma, B=8 gemv")
    torch = _torch()
    import synth.device as sd
    from moe_layer_skinny_amd import kk
    cfg, _, L = gpu_layer("tp_rank")
    ref = oracle_step("tp_rank", 2)
    x, r, _, _ = sd.device_tokens(cfg, 2)
    b = _bufs(cfg, 2)
    ws = L.new_workspace()
    os.environ["KK_FORCE_PLAN"] = "mfma"
    try:
        p = L.query_plan(2)
        assert p["path_name"] == "splitk_mfma" and p["forced"] == 1
        L.layer_decode(2, x, r, b["out"], ws, b["idx"], b["gate"])
        torch.cuda.synchronize()
        assert_close(as_f64_out(b["out"]), ref["out"], "forced mfma out")
        np.testing.assert_array_equal(b["idx"].cpu().numpy(), ref["topk_idx"])
        os.environ["KK_FORCE_PLAN"] = "gemv"
        with pytest.raises(kk.KKError) as e:
            L.query_plan(8)
        assert e.value.status == kk.KK_ERR_UNSUPPORTED
        os.environ["KK_FORCE_PLAN"] = "bogus"
        with pytest.raises(kk.KKError) as e:
            L.query_plan(1)
        assert e.value.status == kk.KK_ERR_INVALID_ARG
    finally:
        del os.environ["KK_FORCE_PLAN"]
    assert L.query_plan(2)["forced"] == 0


# (TP share: K-chunk gate/up with the SwiGLU in the down-projection up to 16 tokens, pieces at 24,
# K chunks and a SwiGLU launch at 64, the fused o-proj + router; with a norm: the fork after the
# norm; full size: grouped launches at 8, pieces and the mixed down at 24, the shared expert's
# split-K gate/up at 64)
TWO_STREAM_CASES = [("tp_rank", 3), ("tp_rank", 8), ("tp_rank", 16), ("tp_rank", 24),
                    ("tp_rank", 64), ("tp_norm", 8), ("full_b8", 8), ("full_b64", 24),
                    ("full_b64", 64)]


@pytest.mark.parametrize("name,B", TWO_STREAM_CASES)
def test_two_stream_mfma_step_equals_one_stream(name, B):
    """The shared expert on the auxiliary stream runs the grouped launches' own kernels on its
    group alone, so the step's bits equal the one-stream step's."""
    log(f"[two-stream-mfma] {name} B={B}")
    torch = _torch()
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    assert L.query_plan(B)["path_name"] == "splitk_mfma"
    x, r, _, _ = sd.device_tokens(cfg, B)
    b = _bufs(cfg, B)
    ws = L.new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"], stream=s)
    s.synchronize()
    ref, ref_idx, ref_gate = b["out"].clone(), b["idx"].clone(), b["gate"].clone()
    for graph in (False, True, True):
        b["out"].zero_()
        with torch.cuda.stream(s):
            L.layer_decode(B, x, r, b["out"], ws, b["idx"], b["gate"], stream=s, two_stream=True,
                           graph=graph)
        s.synchronize()
        assert torch.equal(b["out"], ref), f"two-stream step differs (graph={graph})"
        assert torch.equal(b["idx"], ref_idx) and torch.equal(b["gate"], ref_gate)