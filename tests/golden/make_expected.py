"""Write tests/golden/<workload>_b<B>_out.npz: the fp64 oracle's layer output for every token of
workloads too large for the oracle to run inside a GPU test.

At full size and batch 64 the step touches ~285 routed experts; regenerating each on the host
and upcasting it to fp64 takes minutes, so the oracle's result is computed here once and
stored.  Each file holds the output `out` [B][H] (float64, as the oracle returns it), the
selected experts `topk_idx` [B][k] and a fingerprint of the inputs (the seeded tokens, the
router bias and the head of every weight stream), which the tests recompute: a change of the
generator, the workload or the resample table makes them fail instead of comparing against
stale values.

Calls only synth (inputs) and oracle (the layer); nothing from the HIP library.
Run:  python tests/golden/make_expected.py
"""
import hashlib
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
CASES = [("full_b64", 64)]


def path_for(name: str, B: int) -> str:
    return os.path.join(HERE, f"{name}_b{B}_out.npz")


def fingerprint(cfg, B: int) -> str:
    """sha256 over the seeded inputs of (cfg, B): tokens, bias, and the first 4096 elements of
    every weight stream (expert 0's for the routed experts)."""
    h = hashlib.sha256()
    h.update(f"{cfg.name}:{B}".encode())
    x, r = synth.host_tokens(cfg, B)
    for a in (x, r, synth.host_bias(cfg)):
        h.update(np.ascontiguousarray(a).tobytes())
    for name, (shape, tid, sigma) in synth.weight_spec(cfg).items():
        h.update(synth.host_stream(4096, cfg.layer_seed, tid, sigma, cfg.dtype).tobytes())
    return h.hexdigest()


def host_layer(cfg) -> O.LayerWeights:
    return O.LayerWeights(synth.host_weight(cfg, "w_o"), synth.host_weight(cfg, "w_r"),
                          synth.host_bias(cfg), lambda e: synth.host_expert(cfg, e),
                          synth.host_weight(cfg, "ws13"), synth.host_weight(cfg, "ws2"),
                          norm_weight=synth.host_norm_weight(cfg))


def main():
    for name, B in CASES:
        cfg = synth.CONFIGS[name]
        x, r = synth.host_tokens(cfg, B)
        res = O.layer_step(x, r, host_layer(cfg), cfg.top_k, norm_eps=synth.NORM_EPS)
        path = path_for(name, B)
        np.savez_compressed(path, out=res["out"], topk_idx=res["topk_idx"].astype(np.int32),
                            fingerprint=np.array(fingerprint(cfg, B)))
        print("wrote", path, "n_act", res["n_act"], flush=True)


if __name__ == "__main__":
    main()
