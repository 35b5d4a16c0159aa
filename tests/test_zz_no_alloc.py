"""The entry point that allocates nothing (kk_layer_decode_static) against kk_layer_decode with a
caller workspace: the same kernels, so the same bits, on two calls in a row, the second with a
smaller batch (the static scratch keeps the first call's contents, which the second must not
depend on)."""
import pytest

from tests.gpu_common import gpu_layer, log

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _run_pair(L, cfg, B, x, r, static, two_stream=False):
    torch = _torch()
    out = torch.empty(B, cfg.hidden, dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                      device="cuda")
    idx = torch.full((B, cfg.top_k), -1, dtype=torch.int32, device="cuda")
    gate = torch.zeros(B, cfg.top_k, dtype=torch.float32, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        if static:
            L.layer_decode_static(B, x, r, out, idx, gate, stream=s, two_stream=two_stream)
        else:
            L.layer_decode(B, x, r, out, L.new_workspace(), idx, gate, stream=s,
                           two_stream=two_stream)
    s.synchronize()
    return out, idx, gate


@pytest.mark.parametrize("name,batches", [("tp_rank", (8, 2)), ("tp_rank", (64, 1)),
                                          ("full_b64", (32, 8)), ("full_b64", (2, 1)),
                                          ("tiny_fp32", (1, 1)), ("tp_max", (64, 2))])
def test_static_entry_matches_workspace_entry(name, batches):
    log(f"[no-alloc] {name} batches {batches}")
    torch = _torch()
    import synth.device as sd
    cfg, _, L = gpu_layer(name)
    for B in batches:
        x, r, _, _ = sd.device_tokens(cfg, B)
        want = _run_pair(L, cfg, B, x, r, static=False)
        got = _run_pair(L, cfg, B, x, r, static=True)
        for w, g, what in zip(want, got, ("out", "topk_idx", "topk_gate")):
            assert torch.equal(w, g), f"{name} B={B}: {what} differs"
        log(f"[no-alloc] {name} B={B}: equal")


def test_static_entry_two_stream_and_errors():
    log("[no-alloc] tp_rank two-stream and errors")
    torch = _torch()
    import synth.device as sd
    from moe_layer_skinny_amd import kk
    cfg, _, L = gpu_layer("tp_rank")
    # (batch 8: the split-K path, its shared expert forked onto the auxiliary stream)
    for B in (8, 2):
        xb, rb, _, _ = sd.device_tokens(cfg, B)
        want = _run_pair(L, cfg, B, xb, rb, static=False)
        got = _run_pair(L, cfg, B, xb, rb, static=True, two_stream=True)
        assert all(torch.equal(w, g) for w, g in zip(want, got)), f"B={B}"
    x, r, _, _ = sd.device_tokens(cfg, 2)
    out = torch.empty(2, cfg.hidden, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kk.KKError) as e:  # no graph capture through this entry point
        kk.lib()
        _ = kk.lib().kk_layer_decode_static(L._h, 2, x.data_ptr(), r.data_ptr(), out.data_ptr(),
                                            None, None, None, kk.KK_GRAPH)
        kk._check(_)
    assert e.value.status == kk.KK_ERR_INVALID_ARG
    for bad_b in (0, cfg.max_batch + 1):
        with pytest.raises(kk.KKError) as e:
            L.layer_decode_static(bad_b, x, r, out)
        assert e.value.status == kk.KK_ERR_INVALID_ARG
