"""GPU parity of consecutive layers (kk_chain_decode) against the fp64 oracle's chain: each
layer's output is compared, the next layer reading the previous stored (bf16) output; graph
replay and the weight prefetch on the auxiliary stream give the same bits as the eager chain.
"""
import numpy as np
import pytest

from tests.gpu_common import as_f64_out, assert_close, gpu_chain, log, oracle_chain

pytestmark = pytest.mark.gpu

CASES = [("chain_tp", 1), ("chain_tp", 2), ("chain_tp", 8), ("chain_full", 1), ("chain_full", 8)]


def _run(name, B, **kw):
    import torch
    import synth.device as sd
    from moe_layer_skinny_amd import kk
    cfg, layers = gpu_chain(name)
    xs, r0, _, _ = sd.device_chain_tokens(cfg, B)
    outs = [torch.empty(B, cfg.hidden, dtype=torch.bfloat16, device="cuda") for _ in layers]
    ws = layers[0].new_workspace()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        kk.chain_decode(layers, B, xs, r0, outs, ws, stream=s, **kw)
    s.synchronize()
    return cfg, layers, xs, r0, outs, ws, s


@pytest.mark.parametrize("name,B", CASES)
def test_chain_parity(name, B):
    log(f"[chain] {name} B={B}")
    import torch
    from moe_layer_skinny_amd import kk
    cfg, layers, xs, r0, outs, ws, s = _run(name, B)
    ref = oracle_chain(name, B)
    eager = [o.clone() for o in outs]
    for l, (o, rl) in enumerate(zip(eager, ref)):
        rep = assert_close(as_f64_out(o), rl["out"], f"layer {l} out")
        log(f"[chain] {name} B={B} layer {l}: {rep}")
    for graph, prefetch in ((False, True), (True, False), (True, False), (True, True), (True, True)):
        for o in outs:
            o.zero_()
        with torch.cuda.stream(s):
            kk.chain_decode(layers, B, xs, r0, outs, ws, stream=s, graph=graph, prefetch=prefetch)
        s.synchronize()
        for l in range(cfg.layers):
            assert torch.equal(outs[l], eager[l]), f"graph={graph} prefetch={prefetch} layer {l}"


@pytest.mark.parametrize("name,B", [("chain_tp", 2)])
def test_chain_equals_layer_by_layer(name, B):
    """The chain is the layers' own steps in order: the same bits as kk_layer_decode per layer."""
    log(f"[chain-steps] {name} B={B}")
    import torch
    cfg, layers, xs, r0, outs, ws, s = _run(name, B)
    r = r0
    for l, layer in enumerate(layers):
        o = torch.empty_like(outs[l])
        layer.layer_decode(B, xs[l], r, o, ws)
        torch.cuda.synchronize()
        assert torch.equal(o, outs[l]), f"layer {l}"
        r = o


def test_chain_argument_errors():
    log("[chain-errors]")
    import torch
    from moe_layer_skinny_amd import kk
    from tests.gpu_common import gpu_layer
    cfg, layers = gpu_chain("chain_tp")
    _, _, tiny = gpu_layer("tiny_fp32")
    x = torch.zeros(1, cfg.oproj_in, dtype=torch.bfloat16, device="cuda")
    r = torch.zeros(1, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    o = [torch.empty(1, cfg.hidden, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ws = layers[0].new_workspace()
    for bad_layers, code in (([layers[0], tiny], kk.KK_ERR_INVALID_ARG),
                             ([layers[0], layers[0]], kk.KK_ERR_INVALID_ARG)):
        with pytest.raises(kk.KKError) as e:
            kk.chain_decode(bad_layers, 1, [x, x], r, o, ws)
        assert e.value.status == code
    with pytest.raises(kk.KKError) as e:
        kk.chain_decode(layers[:2], 9, [x, x], r, o, ws)
    assert e.value.status == kk.KK_ERR_INVALID_ARG
    with pytest.raises(kk.KKError) as e:
        kk.chain_decode(layers[:2], 1, [x, x], r, o, None)
    assert e.value.status == kk.KK_ERR_WORKSPACE
    with pytest.raises(kk.KKError) as e:
        kk.chain_decode(layers[:2], 1, [x, x], r, o, ws, stream=0, graph=True)
    assert e.value.status == kk.KK_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert np.isfinite(as_f64_out(r)).all()
