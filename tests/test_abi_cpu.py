"""C-ABI checks that need no GPU: the library loads, exports every declared symbol, and the
host-side validation returns the documented status codes before touching a device."""
import ctypes
import subprocess

import pytest

import synth
from moe_layer_skinny_amd import kk


def _cfg(name="full_b1", **over):
    c = synth.CONFIGS[name]
    d = dict(hidden=c.hidden, oproj_in=c.oproj_in, n_experts=c.n_experts, top_k=c.top_k,
             inter=c.inter, shared_inter=c.shared_inter, dtype=c.dtype)
    d.update(over)
    return kk.make_config(**d)


def test_library_exports_every_declared_function():
    names = kk.header_functions()
    assert len(names) >= 13
    L = kk.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", kk.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    assert set(names) <= exported


def test_header_names_the_four_layer_ops():
    for n in ("kk_oproj_residual", "kk_router_topk", "kk_moe_decode", "kk_layer_decode"):
        assert n in kk.header_functions()


@pytest.mark.parametrize("name", list(synth.CONFIGS))
def test_every_workload_validates(name):
    c = synth.CONFIGS[name]
    cfg = _cfg(name)
    assert kk.validate(cfg, c.max_batch) == kk.KK_OK, kk.last_error()
    assert kk.workspace_bytes(cfg, c.max_batch) > 0


@pytest.mark.parametrize("over,mb,code", [
    (dict(dtype=7), 1, kk.KK_ERR_INVALID_ARG),
    (dict(top_k=400), 1, kk.KK_ERR_INVALID_ARG),
    (dict(hidden=0), 1, kk.KK_ERR_INVALID_ARG),
    (dict(hidden=7170), 1, kk.KK_ERR_INVALID_ARG),  # rows not whole 16-byte chunks
    ({}, 0, kk.KK_ERR_INVALID_ARG),
    ({}, 65, kk.KK_ERR_INVALID_ARG),
    (dict(hidden=4096), 1, kk.KK_ERR_UNSUPPORTED),
    (dict(top_k=17, n_experts=384), 1, kk.KK_ERR_UNSUPPORTED),
    (dict(n_experts=1024), 1, kk.KK_ERR_UNSUPPORTED),
    (dict(inter=2048, shared_inter=128), 1, kk.KK_ERR_UNSUPPORTED),
])
def test_validate_error_codes(over, mb, code):
    assert kk.validate(_cfg(**over), mb) == code
    assert kk.last_error()
    if code != kk.KK_OK:
        assert kk.workspace_bytes(_cfg(**over), mb) == 0


def test_fp32_layer_limited_to_small_batch():
    assert kk.validate(_cfg("tiny_fp32"), 2) == kk.KK_OK
    assert kk.validate(_cfg("tiny_fp32"), 8) == kk.KK_ERR_UNSUPPORTED


def test_routed_scale_must_be_positive():
    cfg = _cfg()
    cfg.routed_scale = 0.0
    assert kk.validate(cfg, 1) == kk.KK_ERR_INVALID_ARG
    cfg.routed_scale = float("nan")
    assert kk.validate(cfg, 1) == kk.KK_ERR_INVALID_ARG


def test_null_arguments_rejected_without_device():
    L = kk.lib()
    assert L.kk_validate(None, 1) == kk.KK_ERR_INVALID_ARG
    assert L.kk_create(None, None, 1, None) == kk.KK_ERR_INVALID_ARG
    h = ctypes.c_void_p()
    cfg = _cfg()
    assert L.kk_create(ctypes.byref(cfg), None, 1, ctypes.byref(h)) == kk.KK_ERR_INVALID_ARG
    assert "weights" in kk.last_error()
    w = kk.KKWeights(16, 32, 48, 64, 80, 96, 113)  # ws2 misaligned: rejected on the host
    assert L.kk_create(ctypes.byref(cfg), ctypes.byref(w), 1, ctypes.byref(h)) == kk.KK_ERR_INVALID_ARG
    assert "ws2" in kk.last_error()
    assert L.kk_destroy(None) == kk.KK_OK
    assert L.kk_query_plan(None, 1, None) == kk.KK_ERR_INVALID_ARG
    for fn, nargs in (("kk_oproj_residual", 8), ("kk_router_topk", 9), ("kk_moe_decode", 10)):
        assert getattr(L, fn)(*([None, 1] + [None] * (nargs - 2))) == kk.KK_ERR_INVALID_ARG
    assert L.kk_layer_decode(None, 1, None, None, None, None, None, None, None, 0) == kk.KK_ERR_INVALID_ARG


def test_status_strings():
    assert kk.status_string(kk.KK_OK) == "KK_OK"
    assert kk.status_string(kk.KK_ERR_UNSUPPORTED) == "KK_ERR_UNSUPPORTED"
    assert kk.status_string(99) == "KK_ERR_UNKNOWN"


def test_workspace_grows_with_batch():
    cfg = _cfg("full_b64")
    assert kk.workspace_bytes(cfg, 64) > kk.workspace_bytes(cfg, 8) > kk.workspace_bytes(cfg, 1)


def test_norm_eps_must_be_finite_and_non_negative():
    for bad in (-1e-6, float("nan"), float("inf")):
        assert kk.validate(_cfg(norm_eps=bad), 1) == kk.KK_ERR_INVALID_ARG
    for ok in (0.0, 1e-6, 1.0):
        assert kk.validate(_cfg(norm_eps=ok), 1) == kk.KK_OK


def _header_struct_fields(name: str) -> list[str]:
    import re
    text = open(kk.HEADER).read()
    body = re.search(r"typedef struct \{([^{}]*)\}\s*" + name + r";", text).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    return [re.findall(r"(\w+)\s*;", d)[0] for d in body.split(";") if d.strip()
            for d in [d + ";"]]


@pytest.mark.parametrize("cname,pystruct", [("kk_config", kk.KKConfig), ("kk_weights", kk.KKWeights),
                                            ("kk_plan", kk.KKPlan)])
def test_binding_structs_match_header(cname, pystruct):
    """The ctypes structures list the header's fields in the header's order."""
    assert [f for f, _ in pystruct._fields_] == _header_struct_fields(cname)


def test_chain_rejects_null_arrays_without_device():
    L = kk.lib()
    assert L.kk_chain_decode(None, 1, 1, None, None, None, None, None, 0) == kk.KK_ERR_INVALID_ARG
    assert kk.last_error()
