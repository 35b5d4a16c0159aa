"""Write tests/golden/attempts.json: per-token resample attempts that keep the top-k boundary gap.

For every workload and token seed t = 0..B_max-1, attempt j = 0, 1, ... draws (x_t, r_t)
from the seeded generator (synth) and the fp64 oracle computes the router's ranking values;
the first attempt whose gap between the k-th and (k+1)-th largest value is >= 1e-3 is kept.
For a chain of layers, each later layer's x_l is drawn again the same way, on the residual
stream that the oracle's chain gives that layer.
Layers with an RMSNorm rank on the router logits of the normalised h.  Gap space (a reading of "seeded so the top-k boundary gap is >= 1e-3"): the selection key
sigmoid(l) + b, except for the layer with a uniform (all-zero) bias, where the sigmoid is
saturated and the key order is the logit order, so the gap is taken on the logits l.

Calls only synth (inputs) and oracle (routing); nothing from the HIP library.
Run:  python tests/golden/make_attempts.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

GAP = 1e-3
MAX_ATTEMPTS = 64


def ranking_values(cfg, x, r, w_o, w_r, b):
    h = O.oproj_residual(x[None], r[None], w_o)
    g = synth.host_norm_weight(cfg)
    l = O.router_logits(h if g is None else O.rms_norm(h, g, synth.NORM_EPS), w_r)
    if cfg.gap_space == "logit":
        return l
    return O.selection_keys(O.sigmoid(l), b)


def first_reaching_gap(cfg, draw, r_of, w_o, w_r, b, what):
    """Per token t: the first attempt j whose draw(t, j) -> (x, r) reaches the gap."""
    attempts, gaps = [], []
    for t in range(cfg.max_batch):
        for j in range(MAX_ATTEMPTS):
            x, r = draw(t, j)
            g = O.topk_gap(ranking_values(cfg, O.as_f64(x), O.as_f64(r), w_o, w_r, b), cfg.top_k)[0]
            if g >= GAP:
                attempts.append(j)
                gaps.append(float(g))
                break
        else:
            raise RuntimeError(f"{what} token {t}: no attempt reached the gap")
    return attempts, gaps


def host_layer(cfg):
    return O.LayerWeights(synth.host_weight(cfg, "w_o"), synth.host_weight(cfg, "w_r"),
                          synth.host_bias(cfg), lambda e: synth.host_expert(cfg, e),
                          synth.host_weight(cfg, "ws13"), synth.host_weight(cfg, "ws2"),
                          norm_weight=synth.host_norm_weight(cfg))


def chain_attempts(cfg, attempts0):
    """Layers 1.. of a chain: the oracle runs the chain with the chosen draws so far, and each
    token's x_l is drawn again until layer l's gap holds on that residual stream."""
    B = cfg.max_batch
    x, r = synth.host_tokens(cfg, B, attempts0)
    per_layer, per_gaps = [], []
    for l in range(1, cfg.layers):
        prev = synth.layer_of(cfg, l - 1)
        step = O.chain_step([x], r, [host_layer(prev)], cfg.top_k, cfg.dtype)[0]
        r = step["out_stored"]
        lc = synth.layer_of(cfg, l)
        w_o, w_r = O.as_f64(synth.host_weight(lc, "w_o")), O.as_f64(synth.host_weight(lc, "w_r"))
        att, gaps = first_reaching_gap(lc, lambda t, j: (synth.host_chain_x(cfg, l, t, j), r[t]),
                                       None, w_o, w_r, synth.host_bias(lc), f"{cfg.name} layer {l}")
        per_layer.append(att)
        per_gaps.append(gaps)
        x = np.stack([synth.host_chain_x(cfg, l, t, att[t]) for t in range(B)])
        print(cfg.name, "layer", l, "attempts", att[:16], flush=True)
    return per_layer, per_gaps


def main():
    out = {"gap": GAP, "script": "tests/golden/make_attempts.py", "configs": {}}
    cache = {}
    for cfg in synth.CONFIGS.values():
        shape_key = (cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.dtype, cfg.layer_seed)
        if shape_key not in cache:
            cache[shape_key] = (O.as_f64(synth.host_weight(cfg, "w_o")),
                                O.as_f64(synth.host_weight(cfg, "w_r")))
        w_o, w_r = cache[shape_key]
        b = synth.host_bias(cfg)
        attempts, gaps = first_reaching_gap(cfg, lambda t, j: synth.host_token(cfg, t, j), None,
                                            w_o, w_r, b, cfg.name)
        out["configs"][cfg.name] = {"gap_space": cfg.gap_space, "attempts": attempts,
                                    "gaps": gaps}
        if cfg.layers > 1:
            la, lg = chain_attempts(cfg, attempts)
            out["configs"][cfg.name].update(layer_attempts=la, layer_gaps=lg)
        print(cfg.name, "attempts", attempts[:16], "max", max(attempts), flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attempts.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
