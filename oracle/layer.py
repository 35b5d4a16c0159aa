"""Plain fp64 definition of one MoE decode-layer step (the weight-bandwidth-bound part).

TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the benchmark's CPU-baseline
leg, never by the product path.  No blocking, fusion or reordering beyond what each
definition states; each function is a direct transcription of the math it names.

Sources (cited by page title and section):
  [P2] "vLLM Hyper-Optimizes Kimi K3 on NVIDIA GB300 for Blazing-FAST Inference",
       section "What's Optimized".
  [P3] "Hyper Optimizing Kimi K3 in vLLM: Moving Fast and Responsibly" (engineering
       summary), section "Recovering time between operators".
The pages name the operations (attention output projection fused with the residual,
router scores, selected experts, a shared expert on its own stream) but print no formula.
Where they are silent this module takes the plain reading of the layer being built, stated
in each docstring as READING:
  * router: sigmoid scores s = 1/(1+exp(-l)); selection key s + b with a per-expert bias b;
    the k largest keys are selected (lower expert index first on equal keys);
  * gates: the selected *unbiased* scores renormalised to sum to 1 (times routed_scale = 1);
    the bias steers selection only;
  * expert FFN: gated SwiGLU, W2 (silu(W1 u) * (W3 u)); in the stacked W13 the gate rows
    W1 come first, then the up rows W3;
  * no normalisation between the residual add and the experts (u = h), unless the layer
    carries an RMSNorm weight: then u = RMSNorm(h) feeds the router and every expert while
    the residual stream h goes on to the combine unnormalised (eps 1e-6);
  * the shared expert is added unweighted;
  * output order of the selected experts: ascending expert index.

Array conventions: ``uint16`` arrays are bf16 bit patterns; any other dtype is taken at its
value.  Every computation is done in float64.
"""
from __future__ import annotations

import numpy as np


def as_f64(a) -> np.ndarray:
    """Exact upcast to float64 (uint16 = bf16 bit pattern: the 16 high bits of an fp32)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Each value rounded to the nearest bf16 number (8 significant bits, fp32 exponent range),
    ties to the even significand; returned as float64.  Overflow past the largest bf16 gives
    +-inf.  (The layer's output in a bf16 layer; the residual stream of the next layer.)"""
    v = np.asarray(v, dtype=np.float64)
    out = v.copy()
    fin = np.isfinite(v) & (v != 0)
    _, e = np.frexp(v[fin])  # v = m * 2**e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)  # below the normal range the spacing stays 2**-133
    q = np.ldexp(v[fin], 8 - e)  # one unit of q = one bf16 step at this exponent
    out[fin] = np.ldexp(np.round(q), e - 8)  # numpy rounds halves to even
    big = np.abs(out) > 3.3895313892515355e38
    out[big] = np.sign(out[big]) * np.inf
    return out


def round_to_f32(v) -> np.ndarray:
    """Each value rounded to the nearest fp32 number (ties to even), as float64; past the
    largest fp32 the result is +-inf."""
    with np.errstate(over="ignore"):
        return np.asarray(v, dtype=np.float64).astype(np.float32).astype(np.float64)


def oproj_residual(x, r, w_o) -> np.ndarray:
    """h = r + x W_o^T: attention output projection plus the residual add.

    [P3 "Recovering time between operators"], [P2 "What's Optimized"]: the output projection
    of attention is fused with its all-reduce and the residual processing.  On one GPU the
    all-reduce is the identity.  x [B][Ko], r [B][H], W_o [H][Ko] (row n = output n).
    """
    return as_f64(r) + as_f64(x) @ as_f64(w_o).T


def rms_norm(h, weight, eps: float) -> np.ndarray:
    """u = weight * h / sqrt(mean(h^2) + eps), row by row (RMS normalisation, per-channel weight).

    READING of the "residual processing" that [P3 "Recovering time between operators"]
    fuses with the attention output projection: the residual add, then the normalisation
    whose output is the MoE block's input.  The pages give neither the norm nor eps; RMSNorm
    with eps = 1e-6 is the plain reading for this layer family.  h [B][H], weight [H].
    """
    h = np.asarray(h, dtype=np.float64)
    ms = np.mean(h * h, axis=1, keepdims=True)
    return as_f64(weight)[None, :] * h / np.sqrt(ms + eps)


def router_logits(h, w_r) -> np.ndarray:
    """l = h W_r^T, W_r [E][H]: per-token router scores before the activation.

    [P3 "Recovering time between operators"]: MoE preparation computes router scores.
    """
    return as_f64(h) @ as_f64(w_r).T


def sigmoid(z) -> np.ndarray:
    """1 / (1 + exp(-z)) -- READING: sigmoid router scores."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def selection_keys(s, b) -> np.ndarray:
    """key = s + b -- READING: a per-expert bias shifts selection only."""
    return np.asarray(s, dtype=np.float64) + as_f64(b)[None, :]


def topk_sets(key, k: int) -> np.ndarray:
    """Indices of the k largest keys per token, listed in ascending expert index.

    Ranking: key descending, then expert index ascending on equal keys (READING).
    Returns int64 [B][k].
    """
    key = np.asarray(key, dtype=np.float64)
    B, E = key.shape
    out = np.empty((B, k), dtype=np.int64)
    idx = np.arange(E)
    for t in range(B):
        order = np.lexsort((idx, -key[t]))  # primary: -key, secondary: index
        out[t] = np.sort(order[:k])
    return out


def topk_gap(values, k: int) -> np.ndarray:
    """Per token: (k-th largest value) - ((k+1)-th largest value); +inf when k == E."""
    v = -np.sort(-np.asarray(values, dtype=np.float64), axis=1)
    if k >= v.shape[1]:
        return np.full(v.shape[0], np.inf)
    return v[:, k - 1] - v[:, k]


def gates_for(s, idx, routed_scale: float = 1.0) -> np.ndarray:
    """g_{t,j} = routed_scale * s_{t,idx[t,j]} / sum_{j'} s_{t,idx[t,j']} (READING: unbiased s)."""
    s = np.asarray(s, dtype=np.float64)
    sel = np.take_along_axis(s, np.asarray(idx), axis=1)
    return routed_scale * sel / sel.sum(axis=1, keepdims=True)


def routing_tables(idx, n_experts: int) -> dict:
    """Token->expert permutation and expert offsets (prefix sum of per-expert counts).

    Slot id of (token t, position j) is t*k + j.  perm lists the slots ordered by
    (expert, token); offsets[e] .. offsets[e+1] is expert e's range of perm; act lists the
    experts with at least one slot, ascending; n_act = len(act).
    """
    idx = np.asarray(idx, dtype=np.int64)
    B, k = idx.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for t in range(B):
        for j in range(k):
            counts[idx[t, j]] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm = np.empty(B * k, dtype=np.int64)
    for t in range(B):  # tokens in ascending order -> stable within each expert
        for j in range(k):
            e = idx[t, j]
            perm[fill[e]] = t * k + j
            fill[e] += 1
    act = np.nonzero(counts)[0].astype(np.int64)
    return {"counts": counts, "offsets": offsets, "perm": perm, "act": act, "n_act": int(len(act))}


def silu(z) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(u, w13, w2) -> np.ndarray:
    """y = W2 (silu(W1 u) * (W3 u)) for each row of u.

    [P3 "Recovering time between operators"]: selected-expert computation (and the shared
    expert).  READING: gated SwiGLU; W13 [2I][H] stacks the gate rows W1 (0..I-1) over the up
    rows W3 (I..2I-1); W2 [H][I].  u [n][H] -> y [n][H].
    """
    w13 = as_f64(w13)
    inter = w13.shape[0] // 2
    u = np.asarray(u, dtype=np.float64)
    z1 = u @ w13[:inter].T
    z3 = u @ w13[inter:].T
    return (silu(z1) * z3) @ as_f64(w2).T


class LayerWeights:
    """Accessor for one layer's weights: dense tensors as attributes, experts on demand.

    w_o [H][Ko], w_r [E][H], bias [E]; expert(e) -> (w13_e [2I][H], w2_e [H][I]);
    shared() -> (ws13 [2Is][H], ws2 [H][Is]); norm_weight [H] or None (no normalisation).
    ``expert_fn`` lets callers regenerate one expert at a time instead of holding all of them.
    """

    def __init__(self, w_o, w_r, bias, expert_fn, ws13, ws2, norm_weight=None):
        self.w_o, self.w_r, self.bias = w_o, w_r, bias
        self._expert_fn = expert_fn
        self._ws13, self._ws2 = ws13, ws2
        self.norm_weight = norm_weight

    def expert(self, e: int):
        return self._expert_fn(int(e))

    def shared(self):
        return self._ws13, self._ws2


def layer_step(x, r, w: LayerWeights, top_k: int, routed_scale: float = 1.0,
               out_tokens=None, norm_eps: float = 1e-6) -> dict:
    """One decode-layer step for B tokens.

      h   = r + x W_o^T                                     (o-proj + residual)
      u   = h, or RMSNorm(h) with w.norm_weight             (READING)
      l   = u W_r^T ; s = sigmoid(l) ; key = s + b           (router scores, READING)
      S_t = top-k of key_t ; g_t = s_t[S_t] / sum s_t[S_t]   (READING: gates from unbiased s)
      out_t = h_t + sum_{e in S_t} g_{t,e} swiglu_e(u_t) + swiglu_shared(u_t)

    [P2 "What's Optimized"], [P3 "Recovering time between operators"]: the shared expert
    runs alongside the routed ones and the results are combined into the residual stream.
    Routed experts are evaluated one active expert at a time over its tokens (each upcast
    once).  ``out_tokens`` restricts the expert part to a subset of tokens (routing is
    still computed for all B); ``out`` rows of other tokens are NaN.
    """
    h = oproj_residual(x, r, w.w_o)
    B, H = h.shape
    u = h if w.norm_weight is None else rms_norm(h, w.norm_weight, norm_eps)
    logits = router_logits(u, w.w_r)
    s = sigmoid(logits)
    key = selection_keys(s, w.bias)
    idx = topk_sets(key, top_k)
    gates = gates_for(s, idx, routed_scale)
    tables = routing_tables(idx, as_f64(w.bias).shape[0])

    tokens = (np.arange(B) if out_tokens is None
              else np.asarray(sorted(set(out_tokens)), dtype=np.int64))
    want = np.zeros(B, dtype=bool)
    want[tokens] = True
    routed = np.zeros((B, H), dtype=np.float64)
    for e in tables["act"]:
        rows = [(t, j) for t in range(B) for j in range(top_k) if idx[t, j] == e and want[t]]
        if not rows:
            continue
        w13, w2 = w.expert(e)
        ts = np.array([t for t, _ in rows])
        y = swiglu_expert(u[ts], w13, w2)
        for n, (t, j) in enumerate(rows):
            routed[t] += gates[t, j] * y[n]
    ws13, ws2 = w.shared()
    ys = np.zeros((B, H), dtype=np.float64)
    ys[tokens] = swiglu_expert(u[tokens], ws13, ws2)
    out = np.full((B, H), np.nan)
    out[tokens] = h[tokens] + routed[tokens] + ys[tokens]
    return {"h": h, "u": u, "logits": logits, "scores": s, "key": key, "topk_idx": idx,
            "topk_gate": gates, **tables, "out": out, "tokens": tokens}


def chain_step(xs, r0, ws, top_k: int, out_dtype: str, routed_scale: float = 1.0,
               norm_eps: float = 1e-6) -> list:
    """Several layers in sequence, each with its own weights: layer l reads x_l and the
    residual stream r_l; r_0 is given and r_{l+1} is layer l's output as stored in the layer
    dtype (rounded to nearest-even bf16, or fp32), the next layer's input.

    READING of consecutive decode layers ([P2 "What's Optimized"] and [P3 "Recovering time
    between operators"] load the next operation's weights into cache from a side stream
    while the current one runs; prefetching changes timing only, never values): the layers
    here have no attention between them, so x_l is a given input per layer.  Returns
    layer_step's result per layer, each with "out_stored" (its output after rounding).
    """
    rnd = round_to_bf16 if out_dtype == "bf16" else round_to_f32
    r = as_f64(r0)
    res = []
    for x, w in zip(xs, ws):
        step = layer_step(x, r, w, top_k, routed_scale, norm_eps=norm_eps)
        step["out_stored"] = rnd(step["out"])
        res.append(step)
        r = step["out_stored"]
    return res
