"""Pins for the fp64 oracle: closed forms, exhaustive enumeration, invariants, special cases.

None of these re-types the oracle's formula: each checks it against something fixed by the
mathematics (a permutation matrix, a one-hot expert, an exhaustive subset search, a library
routine for the sigmoid, linearity, symmetry).  A dropped term, a wrong sign or index, a
transposed operand, a gate/up swap, bias leaking into the gates or a wrong normaliser each
fails at least one test here.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit

import oracle as O

RNG = np.random.default_rng(1234)


def _rand_weights(H, Ko, E, I, Is, rng, scale=0.3):
    w13 = rng.normal(0, scale, (E, 2 * I, H))
    w2 = rng.normal(0, scale, (E, H, I))
    return O.LayerWeights(
        rng.normal(0, scale, (H, Ko)), rng.normal(0, scale, (E, H)), rng.normal(0, 0.1, E),
        lambda e: (w13[e], w2[e]), rng.normal(0, scale, (2 * Is, H)), rng.normal(0, scale, (H, Is)),
    ), w13, w2


# ----------------------------------------------------------------------------- upcast
def test_bf16_upcast_exact_values():
    bits = np.array([0x3F80, 0xC000, 0x4049, 0x0000, 0x8000, 0x3C23], dtype=np.uint16)
    want = [1.0, -2.0, 3.140625, 0.0, -0.0, 0.0099487304687500]
    assert O.as_f64(bits).tolist() == want


# ----------------------------------------------------------------------------- o-proj
def test_oproj_permutation_matrix_orientation():
    rng = np.random.default_rng(1)
    B, H = 3, 9
    pi = rng.permutation(H)
    assert (pi != np.arange(H)).any() and (pi[pi] != np.arange(H)).any()
    w_o = np.zeros((H, H))
    w_o[np.arange(H), pi] = 1.0  # row n (output n) picks input pi[n]
    x, r = rng.normal(size=(B, H)), rng.normal(size=(B, H))
    h = O.oproj_residual(x, r, w_o)
    np.testing.assert_array_equal(h, r + x[:, pi])


def test_oproj_nonsquare_slice():
    rng = np.random.default_rng(2)
    B, H, Ko = 2, 10, 4
    c = rng.normal(size=H)
    w_o = np.zeros((H, Ko))
    w_o[np.arange(H), np.arange(H) % Ko] = c
    x, r = rng.normal(size=(B, Ko)), rng.normal(size=(B, H))
    h = O.oproj_residual(x, r, w_o)
    np.testing.assert_allclose(h, r + c[None, :] * x[:, np.arange(H) % Ko], rtol=0, atol=1e-15)


def test_oproj_zero_weight_is_residual_exactly():
    rng = np.random.default_rng(3)
    r = rng.normal(size=(4, 16)).astype(np.float32)
    h = O.oproj_residual(rng.normal(size=(4, 16)), r, np.zeros((16, 16)))
    assert np.array_equal(h, r.astype(np.float64))


# ----------------------------------------------------------------------------- router
def test_sigmoid_matches_library_and_symmetry():
    z = np.concatenate([np.linspace(-40, 40, 2001), [0.0, 1e-9, -745.0, 745.0]])
    np.testing.assert_allclose(O.sigmoid(z), expit(z), rtol=1e-15, atol=1e-300)
    assert O.sigmoid(np.array([0.0]))[0] == 0.5
    np.testing.assert_allclose(O.sigmoid(-z) + O.sigmoid(z), 1.0, rtol=0, atol=1e-15)


def test_router_logits_one_hot_rows():
    rng = np.random.default_rng(4)
    H, E = 12, 5
    cols = rng.choice(H, E, replace=False)
    w_r = np.zeros((E, H))
    w_r[np.arange(E), cols] = 2.0
    h = rng.normal(size=(3, H))
    np.testing.assert_array_equal(O.router_logits(h, w_r), 2.0 * h[:, cols])


@pytest.mark.parametrize("E,k", [(16, 2), (8, 3), (10, 4)])
def test_topk_exhaustive(E, k):
    rng = np.random.default_rng(E * 10 + k)
    key = rng.normal(size=(20, E))
    idx = O.topk_sets(key, k)
    for t in range(key.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda S: sum(key[t, list(S)]))
        assert tuple(idx[t]) == tuple(sorted(best))
        sel = set(idx[t].tolist())
        lo_sel = min(key[t, e] for e in sel)
        hi_uns = max(key[t, e] for e in range(E) if e not in sel)
        assert lo_sel > hi_uns
        assert list(idx[t]) == sorted(idx[t])


def test_topk_ties_prefer_lower_index():
    key = np.array([[0.5, 0.7, 0.7, 0.7, 0.1]])
    assert O.topk_sets(key, 2).tolist() == [[1, 2]]
    assert O.topk_sets(np.zeros((1, 6)), 3).tolist() == [[0, 1, 2]]


def test_topk_gap_hand_example():
    v = np.array([[0.1, 0.9, 0.5, 0.45]])
    assert O.topk_gap(v, 2)[0] == pytest.approx(0.05, abs=1e-15)
    assert O.topk_gap(v, 1)[0] == pytest.approx(0.4, abs=1e-15)


def test_zero_router_weights_select_by_bias_and_equal_gates():
    rng = np.random.default_rng(5)
    B, H, E, k = 4, 8, 16, 3
    b = rng.normal(0, 0.1, E)
    s = O.sigmoid(O.router_logits(rng.normal(size=(B, H)), np.zeros((E, H))))
    assert np.all(s == 0.5)
    idx = O.topk_sets(O.selection_keys(s, b), k)
    want = np.sort(np.argsort(-b)[:k])
    assert all(list(idx[t]) == list(want) for t in range(B))
    g = O.gates_for(s, idx)
    assert np.all(g == 1.0 / k)


def test_gates_are_convex_weights():
    rng = np.random.default_rng(6)
    s = O.sigmoid(rng.normal(0, 3, size=(50, 24)))
    idx = O.topk_sets(O.selection_keys(s, rng.normal(0, 0.1, 24)), 5)
    g = O.gates_for(s, idx)
    assert np.all(np.abs(g.sum(axis=1) - 1.0) <= 1e-12)
    assert np.all(g > 0) and np.all(g <= 1.0)
    # ratios between gates are the ratios between the selected (unbiased) scores
    sel = np.take_along_axis(s, idx, axis=1)
    np.testing.assert_allclose(g[:, 1:] / g[:, :1], sel[:, 1:] / sel[:, :1], rtol=1e-13)


# ----------------------------------------------------------------------------- routing tables
def test_routing_tables_against_sorted_tuples():
    rng = np.random.default_rng(7)
    for B, E, k in [(1, 16, 2), (5, 12, 3), (64, 40, 8)]:
        idx = np.stack([np.sort(rng.choice(E, k, replace=False)) for _ in range(B)])
        tab = O.routing_tables(idx, E)
        tuples = sorted((idx[t, j], t, j) for t in range(B) for j in range(k))
        assert tab["perm"].tolist() == [t * k + j for _, t, j in tuples]
        np.testing.assert_array_equal(tab["counts"], np.bincount(idx.ravel(), minlength=E))
        assert tab["offsets"][0] == 0 and tab["offsets"][-1] == B * k
        for e in range(E):
            seg = tab["perm"][tab["offsets"][e]:tab["offsets"][e + 1]]
            assert all(idx[p // k, p % k] == e for p in seg)
        assert tab["act"].tolist() == sorted(set(idx.ravel().tolist()))
        assert tab["n_act"] == len(set(idx.ravel().tolist()))


def test_routing_tables_hand_example():
    idx = np.array([[0, 2], [2, 3]])
    tab = O.routing_tables(idx, 4)
    assert tab["counts"].tolist() == [1, 0, 2, 1]
    assert tab["offsets"].tolist() == [0, 1, 1, 3, 4]
    assert tab["perm"].tolist() == [0, 1, 2, 3]
    idx = np.array([[1, 3], [0, 1]])
    tab = O.routing_tables(idx, 4)
    assert tab["perm"].tolist() == [2, 0, 3, 1]
    assert tab["act"].tolist() == [0, 1, 3] and tab["n_act"] == 3


# ----------------------------------------------------------------------------- SwiGLU
def test_silu_closed_form():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(O.silu(z), z * expit(z), rtol=1e-14, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    assert O.silu(np.array([-800.0]))[0] == 0.0


def test_swiglu_one_hot_closed_form_and_gate_up_order():
    H, I = 7, 5
    q, p, m = 3, 2, 6
    alpha, beta, gamma = 1.7, -0.6, 2.5
    w13 = np.zeros((2 * I, H))
    w13[p, q] = alpha  # gate row p reads input q
    w13[I + p, q] = beta  # up row p reads input q
    w2 = np.zeros((H, I))
    w2[m, p] = gamma
    u = np.random.default_rng(8).normal(size=(4, H))
    y = O.swiglu_expert(u, w13, w2)
    want = np.zeros_like(y)
    zq = u[:, q]
    want[:, m] = gamma * (alpha * zq) * expit(alpha * zq) * (beta * zq)
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-300)
    swapped = gamma * (beta * zq) * expit(beta * zq) * (alpha * zq)
    assert np.abs(swapped - want[:, m]).max() > 1e-3


# ----------------------------------------------------------------------------- whole step
def test_zero_expert_weights_give_residual_bitwise():
    rng = np.random.default_rng(9)
    H, Ko, E, k, I = 16, 12, 6, 2, 4
    w = O.LayerWeights(rng.normal(0, 0.3, (H, Ko)), rng.normal(0, 0.3, (E, H)), rng.normal(0, .1, E),
                       lambda e: (np.zeros((2 * I, H)), np.zeros((H, I))),
                       np.zeros((2 * I, H)), np.zeros((H, I)))
    res = O.layer_step(rng.normal(size=(3, Ko)), rng.normal(size=(3, H)), w, k)
    assert np.array_equal(res["out"], res["h"])


def test_shared_expert_only_one_hot():
    rng = np.random.default_rng(10)
    H, E, k, I = 8, 4, 2, 3
    ws13 = np.zeros((2 * I, H))
    ws13[1, 5] = 0.8
    ws13[I + 1, 5] = 1.3
    ws2 = np.zeros((H, I))
    ws2[2, 1] = -1.5
    w = O.LayerWeights(rng.normal(0, 0.3, (H, H)), rng.normal(0, 0.3, (E, H)), np.zeros(E),
                       lambda e: (np.zeros((2 * I, H)), np.zeros((H, I))), ws13, ws2)
    res = O.layer_step(rng.normal(size=(2, H)), rng.normal(size=(2, H)), w, k)
    d = res["out"] - res["h"]
    z = res["h"][:, 5]
    want = np.zeros_like(d)
    want[:, 2] = -1.5 * (0.8 * z) * expit(0.8 * z) * (1.3 * z)
    np.testing.assert_allclose(d, want, rtol=1e-13, atol=1e-300)


def test_zeroed_expert_forced_in_keeps_other_gates():
    rng = np.random.default_rng(11)
    H, Ko, E, k, I = 12, 12, 8, 3, 4
    w, w13, w2 = _rand_weights(H, Ko, E, I, I, rng)
    z = 5
    w.bias = np.zeros(E)
    w.bias[z] = 10.0  # always selected
    x, r = rng.normal(size=(4, Ko)), rng.normal(size=(4, H))
    full = O.layer_step(x, r, w, k)
    w13z, w2z = w13.copy(), w2.copy()
    w13z[z] = 0.0
    w2z[z] = 0.0
    wz = O.LayerWeights(w.w_o, w.w_r, w.bias, lambda e: (w13z[e], w2z[e]), *w.shared())
    zero = O.layer_step(x, r, wz, k)
    assert np.array_equal(full["topk_idx"], zero["topk_idx"])
    assert np.array_equal(full["topk_gate"], zero["topk_gate"])  # gates ignore expert weights
    jz = np.argmax(full["topk_idx"] == z, axis=1)
    gz = full["topk_gate"][np.arange(4), jz]
    yz = np.stack([O.swiglu_expert(full["h"][t:t + 1], w13[z], w2[z])[0] for t in range(4)])
    np.testing.assert_allclose(full["out"] - zero["out"], gz[:, None] * yz, rtol=1e-10, atol=1e-12)


def test_linear_in_down_projections():
    rng = np.random.default_rng(12)
    H, Ko, E, k, I = 10, 6, 6, 2, 3
    w, w13, w2 = _rand_weights(H, Ko, E, I, I, rng)
    x, r = rng.normal(size=(3, Ko)), rng.normal(size=(3, H))
    base = O.layer_step(x, r, w, k)
    c = -2.75
    ws13, ws2 = w.shared()
    w_c = O.LayerWeights(w.w_o, w.w_r, w.bias, lambda e: (w13[e], c * w2[e]), ws13, c * ws2)
    scaled = O.layer_step(x, r, w_c, k)
    np.testing.assert_allclose(scaled["out"] - scaled["h"], c * (base["out"] - base["h"]),
                               rtol=1e-12, atol=1e-12)


def test_expert_relabeling_invariance():
    rng = np.random.default_rng(13)
    H, Ko, E, k, I = 10, 10, 7, 3, 4
    w, w13, w2 = _rand_weights(H, Ko, E, I, I, rng)
    x, r = rng.normal(size=(5, Ko)), rng.normal(size=(5, H))
    base = O.layer_step(x, r, w, k)
    sig = rng.permutation(E)  # new id n holds old expert sig[n]
    inv = np.argsort(sig)
    wp = O.LayerWeights(w.w_o, w.w_r[sig], w.bias[sig], lambda e: (w13[sig[e]], w2[sig[e]]), *w.shared())
    perm = O.layer_step(x, r, wp, k)
    np.testing.assert_allclose(perm["out"], base["out"], rtol=1e-12, atol=1e-12)
    for t in range(5):
        assert sorted(sig[perm["topk_idx"][t]].tolist()) == base["topk_idx"][t].tolist()
    assert np.array_equal(np.sort(inv[base["topk_idx"]], axis=1), perm["topk_idx"])


def test_batch_equals_stacked_single_tokens():
    rng = np.random.default_rng(14)
    H, Ko, E, k, I = 12, 8, 9, 3, 5
    w, _, _ = _rand_weights(H, Ko, E, I, I, rng)
    x, r = rng.normal(size=(6, Ko)), rng.normal(size=(6, H))
    batch = O.layer_step(x, r, w, k)
    for t in range(6):
        one = O.layer_step(x[t:t + 1], r[t:t + 1], w, k)
        np.testing.assert_array_equal(one["topk_idx"][0], batch["topk_idx"][t])
        np.testing.assert_allclose(one["out"][0], batch["out"][t], rtol=1e-13, atol=1e-13)


def test_dense_case_all_experts_selected():
    rng = np.random.default_rng(15)
    H, Ko, E, I = 10, 10, 5, 4
    w, w13, w2 = _rand_weights(H, Ko, E, I, I, rng)
    x, r = rng.normal(size=(3, Ko)), rng.normal(size=(3, H))
    res = O.layer_step(x, r, w, E)
    h = res["h"]
    s = expit(h @ w.w_r.T)
    g = s / s.sum(axis=1, keepdims=True)
    # dense evaluation: every expert on every token via einsum, weighted by g
    z1 = np.einsum("eih,th->tei", w13[:, :I], h)
    z3 = np.einsum("eih,th->tei", w13[:, I:], h)
    a = z1 * expit(z1) * z3
    y = np.einsum("ehi,tei->teh", w2, a)
    ws13, ws2 = w.shared()
    zs1, zs3 = h @ ws13[:I].T, h @ ws13[I:].T
    ys = (zs1 * expit(zs1) * zs3) @ ws2.T
    want = h + np.einsum("te,teh->th", g, y) + ys
    np.testing.assert_allclose(res["out"], want, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(res["topk_gate"], g, rtol=1e-13)


def test_hand_worked_example():
    # H = Ko = 2, E = 3, k = 2, I = 1; numbers chosen so every step has a closed form
    w_o = np.eye(2)
    w_r = np.array([[0.0, 0.0], [2.0, 0.0], [-1.0, 0.0]])
    bias = np.zeros(3)
    a = [0.5, 1.0, 3.0]  # gate weights
    b_ = [2.0, -1.0, 1.0]  # up weights
    c = [1.0, 4.0, 9.0]  # down weights
    experts = {e: (np.array([[a[e], 0.0], [b_[e], 0.0]]), np.array([[c[e]], [0.0]])) for e in range(3)}
    w = O.LayerWeights(w_o, w_r, bias, lambda e: experts[e], np.zeros((2, 2)), np.zeros((2, 1)))
    res = O.layer_step(np.array([[1.0, 0.0]]), np.array([[0.25, -1.0]]), w, 2)
    # h = [1.25, -1]; logits = [0, 2.5, -1.25]; top-2 = {0, 1}
    assert res["topk_idx"].tolist() == [[0, 1]]
    s0, s1 = 0.5, 1.0 / (1.0 + np.exp(-2.5))
    g0, g1 = s0 / (s0 + s1), s1 / (s0 + s1)
    u = 1.25
    y0 = c[0] * (a[0] * u / (1 + np.exp(-a[0] * u))) * (b_[0] * u)
    y1 = c[1] * (a[1] * u / (1 + np.exp(-a[1] * u))) * (b_[1] * u)
    assert res["out"][0, 0] == pytest.approx(1.25 + g0 * y0 + g1 * y1, rel=1e-14)
    assert res["out"][0, 1] == -1.0
    assert res["n_act"] == 2 and res["perm"].tolist() == [0, 1]


def test_out_tokens_subset_matches_full():
    rng = np.random.default_rng(16)
    H, Ko, E, k, I = 10, 10, 8, 2, 3
    w, _, _ = _rand_weights(H, Ko, E, I, I, rng)
    x, r = rng.normal(size=(6, Ko)), rng.normal(size=(6, H))
    full = O.layer_step(x, r, w, k)
    sub = O.layer_step(x, r, w, k, out_tokens=[1, 4])
    np.testing.assert_allclose(sub["out"][[1, 4]], full["out"][[1, 4]], rtol=1e-13, atol=1e-13)
    assert np.isnan(sub["out"][0]).all()
    assert np.array_equal(sub["perm"], full["perm"])


# ----------------------------------------------------------------------------- RMSNorm (optional step)
def _with_norm(w: O.LayerWeights, gamma) -> O.LayerWeights:
    return O.LayerWeights(w.w_o, w.w_r, w.bias, w.expert, *w.shared(), norm_weight=gamma)


def test_rms_norm_unit_mean_square_and_row_scale():
    """weight 1, eps 0: every row has mean square 1 exactly (to rounding) and is a positive
    multiple of its input row."""
    rng = np.random.default_rng(40)
    h = rng.normal(0, 3.0, (5, 37))
    u = O.rms_norm(h, np.ones(37), 0.0)
    np.testing.assert_allclose(np.mean(u * u, axis=1), 1.0, rtol=0, atol=1e-13)
    ratio = u / h
    assert (ratio > 0).all()
    np.testing.assert_allclose(ratio, ratio[:, :1] * np.ones((1, 37)), rtol=1e-13, atol=0)


def test_rms_norm_constant_and_one_hot_rows_closed_form():
    """h = c (every entry): u = w c / sqrt(c^2 + eps).  h = a e_i: u_i = w_i a /
    sqrt(a^2 / H + eps), the other entries 0."""
    rng = np.random.default_rng(41)
    H = 24
    w = rng.normal(1.0, 0.3, H)
    c, eps = -3.0, 0.5
    u = O.rms_norm(np.full((1, H), c), w, eps)
    np.testing.assert_allclose(u[0], w * c / np.sqrt(9.0 + 0.5), rtol=1e-15, atol=0)
    a, i = 2.5, 7
    h = np.zeros((1, H))
    h[0, i] = a
    u = O.rms_norm(h, w, eps)
    want = np.zeros(H)
    want[i] = w[i] * a / np.sqrt(a * a / H + eps)
    np.testing.assert_allclose(u[0], want, rtol=1e-15, atol=0)


def test_rms_norm_scale_invariance_and_eps():
    """eps 0: u(c h) = u(h) for c > 0 and -u(h) for c < 0; eps > 0 shrinks every |u|."""
    rng = np.random.default_rng(42)
    h = rng.normal(size=(3, 16))
    w = rng.normal(1.0, 0.2, 16)
    np.testing.assert_allclose(O.rms_norm(7.0 * h, w, 0.0), O.rms_norm(h, w, 0.0), rtol=1e-13)
    np.testing.assert_allclose(O.rms_norm(-0.5 * h, w, 0.0), -O.rms_norm(h, w, 0.0), rtol=1e-13)
    assert (np.abs(O.rms_norm(h, w, 1e-2)) < np.abs(O.rms_norm(h, w, 0.0))).all()


def test_norm_layer_residual_keeps_h_experts_read_u():
    """W_o = 0 and a constant residual row c: h = c, u = w c / sqrt(c^2 + eps) in closed form.
    The normalised layer then routes like the plain layer fed u, and out - h equals that
    layer's out - u: router and experts read u, the combine adds h."""
    rng = np.random.default_rng(43)
    H, E, k, I = 16, 8, 2, 6
    w, _, _ = _rand_weights(H, H, E, I, I, rng)
    gamma = rng.normal(1.0, 0.3, H)
    B, c, eps = 3, np.array([2.0, -1.5, 0.25]), 1e-6
    wz = O.LayerWeights(np.zeros((H, H)), w.w_r, w.bias, w.expert, *w.shared())
    r = c[:, None] * np.ones((B, H))
    x = rng.normal(size=(B, H))
    got = O.layer_step(x, r, _with_norm(wz, gamma), k, norm_eps=eps)
    u = gamma[None, :] * c[:, None] / np.sqrt(c[:, None] ** 2 + eps)
    plain = O.layer_step(x, u, wz, k)
    np.testing.assert_array_equal(got["topk_idx"], plain["topk_idx"])
    np.testing.assert_allclose(got["topk_gate"], plain["topk_gate"], rtol=1e-13)
    np.testing.assert_allclose(got["out"] - r, plain["out"] - u, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(got["u"], u, rtol=1e-14)


def test_norm_layer_scale_invariance():
    """eps 0: scaling x and r by c > 0 scales h by c and leaves u, the routing and the expert
    part out - h unchanged."""
    rng = np.random.default_rng(44)
    H, Ko, E, k, I = 16, 12, 8, 3, 6
    w, _, _ = _rand_weights(H, Ko, E, I, I, rng)
    wn = _with_norm(w, rng.normal(1.0, 0.3, H))
    x, r = rng.normal(size=(2, Ko)), rng.normal(size=(2, H))
    a = O.layer_step(x, r, wn, k, norm_eps=0.0)
    b = O.layer_step(4.0 * x, 4.0 * r, wn, k, norm_eps=0.0)
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(b["h"], 4.0 * a["h"], rtol=1e-14)
    np.testing.assert_allclose(b["out"] - b["h"], a["out"] - a["h"], rtol=1e-11, atol=1e-12)


# ----------------------------------------------------------------------------- chained layers
def test_round_to_bf16_hand_values_and_bit_rounding():
    """Ties go to the even significand; values agree with an independent bit-level RNE of
    fp32 inputs (synth's converter); overflow past the largest bf16 gives inf."""
    import synth
    v = np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8 + 2.0**-30), 3.0, 0.0,
                  2.0**-133 * 0.5, 2.0**-133 * 1.5, 3.4e38])
    want = [1.0, 1.0 + 2.0**-6, -(1.0 + 2.0**-7), 3.0, 0.0, 0.0, 2.0**-132, np.inf]
    assert O.round_to_bf16(v).tolist() == want
    rng = np.random.default_rng(50)
    a = (rng.normal(size=20000) * np.exp(rng.uniform(-60, 60, 20000))).astype(np.float32)
    ref = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(a)).astype(np.float64)
    np.testing.assert_array_equal(O.round_to_bf16(a.astype(np.float64)), ref)


def _f64_to_f32_bits_rne(v: np.ndarray) -> np.ndarray:
    """Round float64 values in the fp32 normal range to fp32 by integer work on the float64
    bit pattern: keep 23 of the 52 fraction bits, round the dropped 29 to nearest, ties to an
    even kept part (a carry out of the fraction moves to the next binade by itself)."""
    u = v.view(np.uint64)
    sign = (u >> np.uint64(63)).astype(np.uint64)
    exp = ((u >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64) - 1023
    frac = u & np.uint64((1 << 52) - 1)
    kept = frac >> np.uint64(29)
    rest = frac & np.uint64((1 << 29) - 1)
    half = np.uint64(1 << 28)
    up = (rest > half) | ((rest == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    mag = ((exp + 127).astype(np.uint64) << np.uint64(23)) + kept + up.astype(np.uint64)
    return ((sign << np.uint64(31)) | mag).astype(np.uint32)


def test_round_to_f32_hand_values_and_bit_rounding():
    """Ties go to the even significand (fp32 has 24 significant bits); subnormals are spaced by
    2^-149; values past the largest fp32 overflow to inf; normal values agree with a bit-level
    rounding of the float64 pattern."""
    v = np.array([1.0 + 2.0**-24, 1.0 + 3 * 2.0**-24, -(1.0 + 2.0**-24 + 2.0**-50), 3.0, 0.0,
                  2.0**-149 * 0.5, 2.0**-149 * 1.5, 2.0**-149 * 2.5, 3.5e38,
                  3.4028234663852886e38])
    want = [1.0, 1.0 + 2.0**-22, -(1.0 + 2.0**-23), 3.0, 0.0, 0.0, 2.0**-148, 2.0**-148,
            np.inf, 3.4028234663852886e38]
    assert O.round_to_f32(v).tolist() == want
    rng = np.random.default_rng(49)
    a = rng.normal(size=20000) * np.exp(rng.uniform(-60, 60, 20000))
    ref = _f64_to_f32_bits_rne(a).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(O.round_to_f32(a), ref)
    # hand-made ties in the random set's binades: exactly half a step above an fp32 value
    t = np.float32(rng.normal(size=2000)).astype(np.float64)
    ties = t + np.spacing(t.astype(np.float32)).astype(np.float64) / 2
    np.testing.assert_array_equal(O.round_to_f32(ties),
                                  _f64_to_f32_bits_rne(ties).view(np.float32).astype(np.float64))


def test_chain_of_one_is_the_layer_and_rounds_its_output():
    rng = np.random.default_rng(51)
    H, E, k, I = 16, 8, 2, 6
    w, _, _ = _rand_weights(H, H, E, I, I, rng)
    x, r = rng.normal(size=(2, H)), rng.normal(size=(2, H))
    one = O.layer_step(x, r, w, k)
    ch = O.chain_step([x], r, [w], k, "bf16")
    np.testing.assert_array_equal(ch[0]["out"], one["out"])
    np.testing.assert_array_equal(ch[0]["out_stored"], O.round_to_bf16(one["out"]))
    assert not np.array_equal(ch[0]["out_stored"], one["out"])


def test_chain_without_experts_accumulates_projections():
    """All expert weights 0: each layer adds only its projection, so the stored stream after
    layer l is the rounded running sum r + x_0 W_0^T + ... in that order."""
    rng = np.random.default_rng(52)
    H, E, k, I, L = 12, 6, 2, 4, 3
    ws, xs = [], []
    for _ in range(L):
        w, _, _ = _rand_weights(H, H, E, I, I, rng)
        z13, z2 = np.zeros((2 * I, H)), np.zeros((H, I))
        ws.append(O.LayerWeights(w.w_o, w.w_r, w.bias, lambda e, a=z13, b=z2: (a, b),
                                 np.zeros((2 * I, H)), np.zeros((H, I))))
        xs.append(rng.normal(size=(3, H)))
    r0 = rng.normal(size=(3, H))
    res = O.chain_step(xs, r0, ws, k, "bf16")
    r = r0
    for l in range(L):
        r = O.round_to_bf16(r + xs[l] @ ws[l].w_o.T)
        np.testing.assert_allclose(res[l]["out_stored"], r, rtol=0, atol=0)


def test_chain_feeds_each_layer_the_previous_stored_output():
    rng = np.random.default_rng(53)
    H, E, k, I = 16, 8, 2, 6
    w0, _, _ = _rand_weights(H, H, E, I, I, rng)
    w1, _, _ = _rand_weights(H, H, E, I, I, rng)
    x0, x1, r0 = rng.normal(size=(2, H)), rng.normal(size=(2, H)), rng.normal(size=(2, H))
    ch = O.chain_step([x0, x1], r0, [w0, w1], k, "f32")
    second = O.layer_step(x1, O.round_to_f32(O.layer_step(x0, r0, w0, k)["out"]), w1, k)
    np.testing.assert_array_equal(ch[1]["out"], second["out"])
    np.testing.assert_array_equal(ch[1]["topk_idx"], second["topk_idx"])
