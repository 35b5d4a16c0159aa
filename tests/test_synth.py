"""Seeded input generator: Philox known answers, stream consistency, distributions, gap table."""
import math

import numpy as np
import pytest

import oracle as O
import synth


# Known-answer vectors of Philox4x32-10 published with the generator's definition
# (Salmon, Moraes, Dror, Shaw, SC'11; Random123 distribution, kat_vectors):
# (counter words, key words) -> output words.
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    assert tuple(int(v) for v in synth.philox4x32_10(ctr, key)) == want


def _box_muller_reference(n, key0, key1, sigma):
    """Element n by the Box-Muller transform with the math library's log, sqrt and cos: u1 in
    (0, 1] from the top 53 bits of Philox words 0-1, the angle 2 pi w2 / 2^32 from word 2."""
    w = synth.philox4x32_10((n & 0xFFFFFFFF, n >> 32, 0, 0), (key0, key1))
    m53 = ((int(w[0]) << 32) | int(w[1])) >> 11
    u1 = (m53 + 1) * 2.0 ** -53
    return math.sqrt(-2.0 * math.log(u1)) * math.cos(2.0 * math.pi * int(w[2]) / 2.0 ** 32) * sigma


def test_element_is_box_muller_of_the_philox_words():
    # the generator's own log / sqrt / cos agree with the math library's to far below one fp32
    # step, so the stored fp32 value is the reference rounded to fp32 (or, at a rounding
    # boundary, its neighbour)
    ns = [0, 1, 12345, 2**32 + 7] + list(range(10**9, 10**9 + 2000))
    exact = 0
    for n in ns:
        want = _box_muller_reference(n, 3, 77, 0.5)
        g = float(synth.host_stream(1, 3, 77, 0.5, "f32", first=n)[0])
        ulp = float(np.spacing(np.float32(abs(want))))
        assert abs(g - want) <= ulp, (n, g, want)
        exact += g == float(np.float32(want))
    assert exact >= len(ns) - 2


def test_stream_offsets_are_consistent():
    full = synth.host_stream(5000, 0, 4, 0.02, "bf16")
    part = synth.host_stream(1000, 0, 4, 0.02, "bf16", first=3000)
    assert np.array_equal(full[3000:4000], part)


def test_bf16_is_rne_of_fp32():
    f = synth.host_stream(100000, 1, 9, 1.0, "f32")
    b = synth.host_stream(100000, 1, 9, 1.0, "bf16")
    u = f.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(b, rne)


def test_distribution_is_normal():
    """N(0, sigma^2): mean, standard deviation, kurtosis 3, normal tail mass beyond 4 sigma (an
    Irwin-Hall sum of four uniforms would have none past 3.46 sigma and kurtosis 2.7), and a
    Kolmogorov-Smirnov test against the normal distribution."""
    from scipy import stats
    v = synth.host_stream(4_000_000, 0, 5, 0.02, "f32").astype(np.float64)
    assert abs(v.mean()) < 1e-4
    assert v.std() == pytest.approx(0.02, rel=2e-3)
    k = ((v - v.mean()) ** 4).mean() / v.var() ** 2
    assert k == pytest.approx(3.0, abs=0.02)
    tail = (np.abs(v) > 4 * 0.02).mean()
    assert tail == pytest.approx(2 * stats.norm.sf(4), rel=0.25)  # ~253 of 4M draws
    assert np.abs(v).max() > 4.5 * 0.02
    assert stats.kstest(v[:1_000_000] / 0.02, "norm").pvalue > 1e-3


def test_expert_slices_match_whole_tensor():
    cfg = synth.CONFIGS["tiny_fp32"]
    w13 = synth.host_weight(cfg, "w13")
    w2 = synth.host_weight(cfg, "w2")
    for e in [0, 5, 15]:
        a, b = synth.host_expert(cfg, e)
        assert np.array_equal(a, w13[e]) and np.array_equal(b, w2[e])


def test_bias_recipes():
    b = synth.host_bias(synth.CONFIGS["tp_rank"]).astype(np.float64)
    assert b.sum() == pytest.approx(1.0, abs=1e-6)
    ranks = np.arange(1, 385, dtype=np.float64)
    pmf = ranks ** -1.2 / (ranks ** -1.2).sum()
    np.testing.assert_allclose(np.sort(b)[::-1], pmf, rtol=1e-6)
    assert b.max() == pytest.approx(0.246, abs=1e-3)
    assert np.all(synth.host_bias(synth.CONFIGS["full_b64"]) == 0)
    n = synth.host_bias(synth.CONFIGS["full_b1"]).astype(np.float64)
    assert n.std() == pytest.approx(0.1, rel=0.15)


def test_config_shapes():
    c = synth.CONFIGS
    assert (c["full_b1"].hidden, c["full_b1"].n_experts, c["full_b1"].top_k, c["full_b1"].inter) == (7168, 384, 8, 2048)
    assert (c["tp_rank"].oproj_in, c["tp_rank"].inter, c["tp_rank"].batches) == (448, 128, (1, 2, 8, 64))
    assert (c["tiny_fp32"].hidden, c["tiny_fp32"].n_experts, c["tiny_fp32"].top_k) == (256, 16, 2)
    assert c["full_b64"].bias == "zero" and c["full_b64"].gap_space == "logit"


def test_attempt_table_gaps_hold():
    table = synth.load_attempts()
    for name, cfg in synth.CONFIGS.items():
        ent = table["configs"][name]
        assert len(ent["attempts"]) == cfg.max_batch
        assert min(ent["gaps"]) >= 1e-3


def test_attempt_table_tiny_recomputed():
    cfg = synth.CONFIGS["tiny_fp32"]
    (j,) = synth.attempts_for(cfg, 1)
    x, r = synth.host_token(cfg, 0, j)
    h = O.oproj_residual(x[None], r[None], synth.host_weight(cfg, "w_o"))
    key = O.selection_keys(O.sigmoid(O.router_logits(h, synth.host_weight(cfg, "w_r"))), synth.host_bias(cfg))
    assert O.topk_gap(key, cfg.top_k)[0] >= 1e-3
    for jj in range(j):  # earlier attempts were rejected
        x, r = synth.host_token(cfg, 0, jj)
        h = O.oproj_residual(x[None], r[None], synth.host_weight(cfg, "w_o"))
        key = O.selection_keys(O.sigmoid(O.router_logits(h, synth.host_weight(cfg, "w_r"))), synth.host_bias(cfg))
        assert O.topk_gap(key, cfg.top_k)[0] < 1e-3


def test_verify_tokens_share_a_component():
    """Speculative-verify tokens: sqrt(rho) * shared + sqrt(1 - rho) * own, so two tokens of
    the batch correlate by rho, each has unit variance, and a resample redraws only the own
    part (the shared part is the same stream for every token and attempt)."""
    cfg = synth.CONFIGS["verify_b8"]
    f = synth.bf16_bits_to_f32
    x0, r0 = synth.host_token(cfg, 0, 0)
    x1, r1 = synth.host_token(cfg, 1, 0)
    rho = synth.VERIFY_RHO
    assert abs(np.corrcoef(f(x0), f(x1))[0, 1] - rho) < 0.02
    assert abs(np.corrcoef(f(r0), f(r1))[0, 1] - rho) < 0.02
    assert abs(np.std(f(r0)) - 1.0) < 0.02
    # x_t(attempt 1) - x_t(attempt 0) = sqrt(1 - rho) * (own_1 - own_0), up to rounding
    x0b, _ = synth.host_token(cfg, 0, 1)
    d = f(x0b).astype(np.float64) - f(x0)
    own0 = synth.host_stream(cfg.oproj_in, 0, synth.token_key(0, synth.KIND_X), 1.0, "f32")
    own1 = synth.host_stream(cfg.oproj_in, 0, synth.token_key(1, synth.KIND_X), 1.0, "f32")
    want = np.sqrt(1 - rho) * (own1.astype(np.float64) - own0)
    assert np.max(np.abs(d - want)) < 0.05  # two bf16 roundings of values of size ~3


def test_bf16_rounding_helper_matches_generator():
    a = synth.host_stream(4096, 11, 7, 1.0, "f32")
    b = synth.host_stream(4096, 11, 7, 1.0, "bf16")
    assert np.array_equal(synth.f32_to_bf16_bits(a), b)


def test_norm_weight_recipe():
    """RMSNorm weight: 1 + N(0, 0.1) per channel, in the config dtype; none without a norm."""
    assert synth.host_norm_weight(synth.CONFIGS["full_b1"]) is None
    g = synth.host_norm_weight(synth.CONFIGS["full_norm"])
    assert g.dtype == np.uint16 and g.shape == (7168,)
    v = synth.bf16_bits_to_f32(g).astype(np.float64)
    assert abs(v.mean() - 1.0) < 0.01 and abs(v.std() - synth.NORM_SIGMA) < 0.01
    t = synth.host_norm_weight(synth.CONFIGS["tiny_norm"])
    assert t.dtype == np.float32 and t.shape == (256,)
    np.testing.assert_array_equal(synth.host_norm_weight(synth.CONFIGS["full_norm"]), g)
