"""Write tests/golden/attempts.json: per-token resample attempts that keep the top-k boundary gap.

For every workload and token seed t = 0..B_max-1, attempt j = 0, 1, ... draws (x_t, r_t)
from the seeded generator (synth) and the fp64 oracle computes the router's ranking values;
the first attempt whose gap between the k-th and (k+1)-th largest value is >= 1e-3 is kept.
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


def main():
    out = {"gap": GAP, "script": "tests/golden/make_attempts.py", "configs": {}}
    cache = {}
    for cfg in synth.CONFIGS.values():
        shape_key = (cfg.hidden, cfg.oproj_in, cfg.n_experts, cfg.dtype)
        if shape_key not in cache:
            cache[shape_key] = (O.as_f64(synth.host_weight(cfg, "w_o")),
                                O.as_f64(synth.host_weight(cfg, "w_r")))
        w_o, w_r = cache[shape_key]
        b = synth.host_bias(cfg)
        attempts, gaps = [], []
        for t in range(cfg.max_batch):
            for j in range(MAX_ATTEMPTS):
                x, r = synth.host_token(cfg, t, j)
                g = O.topk_gap(ranking_values(cfg, O.as_f64(x), O.as_f64(r), w_o, w_r, b), cfg.top_k)[0]
                if g >= GAP:
                    attempts.append(j)
                    gaps.append(float(g))
                    break
            else:
                raise RuntimeError(f"{cfg.name} token {t}: no attempt reached the gap")
        out["configs"][cfg.name] = {"gap_space": cfg.gap_space, "attempts": attempts,
                                    "gaps": gaps}
        print(cfg.name, "attempts", attempts[:16], "max", max(attempts), flush=True)
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "attempts.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
