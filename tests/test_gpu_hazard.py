"""Stream-hazard tests: the variants that use the context's second stream (the shared expert's
gate/up with KK_TWO_STREAM, the next-layer weight reads with KK_PREFETCH) must give the same
bits as the single-stream step however the two streams are timed against each other.

A bounded delay kernel (kk_set_stream_delay) is placed first on one stream, then on the other,
so that the undelayed stream runs ahead; before each delayed step the workspace is filled with
the intermediates of a step on other inputs, so a read that escaped its wait would find stale
values and change the output.  ("Hyper Optimizing Kimi K3 in vLLM: Moving Fast and
Responsibly", section "Faster code needs targeted validation": activation reads moved before
a synchronisation wait are timing errors that ordinary functional tests can miss.)
Every delay kernel ends after its fixed time; no test leaves a kernel waiting.
"""
import pytest

from tests.gpu_common import gpu_chain, gpu_layer, log

pytestmark = pytest.mark.gpu

DELAY_US = 300.0


def _torch():
    import torch
    return torch


# (the full-width layer at two tokens takes the 3-launch step, its shared gate/up on the
# auxiliary stream beside the top-k + routed gate/up launch; from three tokens the split-K path
# forks the shared expert's gate/up and down-projection after the o-proj and joins before the
# combine)
@pytest.mark.parametrize("name,B", [("tp_rank", 1), ("tp_rank", 2), ("full_b1", 1), ("full_b64", 2),
                                    ("tp_rank", 8), ("tp_rank", 64), ("full_b64", 24),
                                    ("full_b64", 64)])
def test_two_stream_step_is_timing_independent(name, B):
    log(f"[hazard-two-stream] {name} B={B}")
    torch = _torch()
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    x, r, _, _ = sd.device_tokens(cfg, B)
    out = torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    idx = torch.empty(B, cfg.top_k, dtype=torch.int32, device="cuda")
    gate = torch.empty(B, cfg.top_k, dtype=torch.float32, device="cuda")
    ws = L.new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        L.layer_decode(B, x, r, out, ws, idx, gate, stream=s)
    s.synchronize()
    ref, ref_idx, ref_gate = out.clone(), idx.clone(), gate.clone()
    xo, ro = -x.flip(0), -r.flip(0)  # other inputs: other intermediates in the workspace
    try:
        for which in (0, 1, 0, 1):
            with torch.cuda.stream(s):
                L.layer_decode(B, xo, ro, out, ws, idx, gate, stream=s)
            s.synchronize()
            assert not torch.equal(out, ref)
            L.set_stream_delay(which, DELAY_US)
            out.zero_()
            with torch.cuda.stream(s):
                L.layer_decode(B, x, r, out, ws, idx, gate, stream=s, two_stream=True)
            s.synchronize()
            L.set_stream_delay(which, 0.0)
            assert torch.equal(out, ref), f"two-stream step with stream {which} delayed differs"
            assert torch.equal(idx, ref_idx) and torch.equal(gate, ref_gate)
    finally:
        L.set_stream_delay(0, 0.0)
        L.set_stream_delay(1, 0.0)


@pytest.mark.parametrize("B", [1, 8])
def test_prefetch_chain_is_timing_independent(B):
    log(f"[hazard-prefetch] chain_tp B={B}")
    torch = _torch()
    import synth.device as sd
    from moe_layer_skinny_amd import kk
    cfg, layers = gpu_chain("chain_tp")
    xs, r0, _, _ = sd.device_chain_tokens(cfg, B)
    outs = [torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda") for _ in layers]
    ws = layers[0].new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kk.chain_decode(layers, B, xs, r0, outs, ws, stream=s)
    s.synchronize()
    ref = [o.clone() for o in outs]
    xo = [-x.flip(0) for x in xs]
    try:
        for which in (0, 1):
            with torch.cuda.stream(s):
                kk.chain_decode(layers, B, xo, -r0.flip(0), outs, ws, stream=s)
            s.synchronize()
            for layer in (layers if which == 0 else layers[:1]):
                layer.set_stream_delay(which, DELAY_US)
            for o in outs:
                o.zero_()
            with torch.cuda.stream(s):
                kk.chain_decode(layers, B, xs, r0, outs, ws, stream=s, prefetch=True)
            s.synchronize()
            for layer in layers:
                layer.set_stream_delay(which, 0.0)
            for l, (o, want) in enumerate(zip(outs, ref)):
                assert torch.equal(o, want), f"layer {l} differs with stream {which} delayed"
    finally:
        for layer in layers:
            layer.set_stream_delay(0, 0.0)
            layer.set_stream_delay(1, 0.0)


def test_delay_hook_arguments():
    log("[hazard-args]")
    from moe_layer_skinny_amd import kk
    _, _, L = gpu_layer("tp_rank")
    for which, us in ((2, 1.0), (0, -1.0), (1, 20000.0)):
        with pytest.raises(kk.KKError) as e:
            L.set_stream_delay(which, us)
        assert e.value.status == kk.KK_ERR_INVALID_ARG
