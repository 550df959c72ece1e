"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU needed).

Each test checks the oracle against something other than itself: a library routine, a closed form
or identity, a brute-force evaluation on tiny inputs, or a number the pages print
(tests/golden/k3_constants.json).
"""
import json
import math
import os
from dataclasses import replace

import numpy as np
import pytest
import scipy.special
import torch

from oracle import lmoe_oracle as O
from workloads import CONFIGS
from workloads.inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = CONFIGS["tiny_f32"]


# ------------------------------------------------------------------------------------------------
# storage rounding
# ------------------------------------------------------------------------------------------------
def test_bf16_rounding_matches_torch_on_float32_values():
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.0e38, -3.0e38, 1e-40])])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_to_bf16(a.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_bf16_rounding_is_nearest_even_from_float64_brute_force():
    # Brute force: the result must be one of the two bf16 neighbours, the nearer one, and on an
    # exact tie the one with an even last significand bit.
    rng = np.random.default_rng(2)
    a = rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))
    got = O.round_to_bf16(a)
    for v, r in zip(a[:2000], got[:2000]):
        bits = np.float32(v).view(np.uint32) & np.uint32(0xFFFF0000)
        cand = []
        for d in (-1, 0, 1, 2):
            b = np.uint32(int(bits) + d * 0x10000)
            cand.append(float(np.uint32(b).view(np.float32)))
        best = min(cand, key=lambda c: (abs(c - v), (np.float32(c).view(np.uint32) >> 16) & 1))
        assert r == best, (v, r, best)
    # exact bf16 halfway case: 1 + 2^-8 lies between 1 and 1 + 2^-7 -> ties to even -> 1.0
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert O.round_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    # just above the halfway point rounds up (float32 first would lose the sticky bit)
    assert O.round_to_bf16(np.array([1.0 + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7


def _bf16_from_fields(bits: int) -> float:
    """The value of a bfloat16 bit pattern written out from its fields: sign bit 15, 8-bit exponent
    (bias 127), 7-bit fraction; exponent 0 is subnormal (2^-126 * f/128), 255 is inf/NaN."""
    sign = -1.0 if bits >> 15 else 1.0
    e, f = (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0xFF:
        return sign * math.inf if f == 0 else math.nan
    if e == 0:
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def test_bf16_bits_decode_from_fields():
    # every finite bit pattern, against the field formula
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):  # signalling-NaN patterns
        got = O.bf16_bits_to_f64(bits)
    want = np.array([_bf16_from_fields(int(b)) for b in bits])
    finite = np.isfinite(want)
    np.testing.assert_array_equal(got[finite], want[finite])
    assert np.array_equal(np.isinf(got), np.isinf(want)) and np.array_equal(np.isnan(got), np.isnan(want))
    # worked values
    assert O.bf16_bits_to_f64(np.uint16([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F]))[:5].tolist() == [
        1.0, -2.0, 1.0 + 2.0 ** -7, 2.0 ** -133, (2.0 - 2.0 ** -7) * 2.0 ** 127]


def _exact_round_bf16(v) -> float:
    """Round an exact rational to the nearest bfloat16 (ties to an even significand), in rational
    arithmetic: with 2^e <= |v| < 2^(e+1), the spacing of bfloat16 values there is 2^(e-7)."""
    from fractions import Fraction

    v = Fraction(v)
    if v == 0:
        return 0.0
    a = abs(v)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    n, r = divmod(a, q)
    if r * 2 > q or (r * 2 == q and n % 2 == 1):
        n += 1
    return math.copysign(float(n * q), v)


def _bf16_matrix(rng, shape, scale):
    from workloads.inputs import f32_to_bf16_bits

    return f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


def test_down_projection_against_exact_sums():
    # x_lat[t, l] = sum_d x[t, d] W_dn[l, d], each sum formed exactly (rationals), then rounded once
    # to bfloat16; the oracle must give the same bits
    from fractions import Fraction

    rng = np.random.default_rng(21)
    T, D, L = 6, 40, 5
    x, w = _bf16_matrix(rng, (T, D), 1.0), _bf16_matrix(rng, (L, D), 1.0 / np.sqrt(D))
    xf, wf = O.bf16_bits_to_f64(x), O.bf16_bits_to_f64(w)
    got = O.down_project(xf, wf, "bf16")
    for t in range(T):
        for l in range(L):
            exact = sum(Fraction(float(xf[t, d])) * Fraction(float(wf[l, d])) for d in range(D))
            assert got[t, l] == _exact_round_bf16(exact), (t, l)
    # f32 storage: the same sums rounded to float32
    got32 = O.down_project(xf, wf, "f32")
    want32 = np.array([[float(np.float32(math.fsum(xf[t] * wf[l]))) for l in range(L)] for t in range(T)])
    np.testing.assert_array_equal(got32, want32)


def test_up_projection_against_explicit_sums():
    # out = n . W_up^T + y_sh per element with math.fsum over the products and the shared term; the
    # stored value is that sum rounded once to the storage type
    rng = np.random.default_rng(22)
    T, L, D = 5, 32, 7
    n, w = _bf16_matrix(rng, (T, L), 1.0), _bf16_matrix(rng, (D, L), 1.0 / np.sqrt(L))
    nf, wf = O.bf16_bits_to_f64(n), O.bf16_bits_to_f64(w)
    ysh = rng.standard_normal((T, D)).astype(np.float32).astype(np.float64)
    pre, stored = O.up_project(nf, wf, ysh, "bf16")
    want = np.array([[math.fsum(list(nf[t] * wf[d]) + [ysh[t, d]]) for d in range(D)] for t in range(T)])
    np.testing.assert_allclose(pre, want, rtol=1e-14, atol=0)
    np.testing.assert_array_equal(stored, [[_exact_round_bf16(v) for v in row] for row in pre])
    # without a shared part the products alone; a transposed W_up would not even have this shape
    pre0, _ = O.up_project(nf, wf, None, "f32")
    np.testing.assert_allclose(pre0, want - ysh, rtol=1e-13, atol=1e-15)
    assert pre0.shape == (T, D)


# ------------------------------------------------------------------------------------------------
# elementwise functions
# ------------------------------------------------------------------------------------------------
def test_sigmoid_matches_scipy_expit():
    a = np.linspace(-800, 800, 10001)
    np.testing.assert_allclose(O.sigmoid(a), scipy.special.expit(a), rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("beta", [4.0, 1.5, 10.0])
def test_situ_identities(beta):
    g = np.linspace(-60, 60, 4801)
    act = O.situ(g, beta)
    # odd part: sigma(g) + sigma(-g) = 1  =>  act(g) - act(-g) = beta*tanh(g/beta)
    np.testing.assert_allclose(act - O.situ(-g, beta), beta * np.tanh(g / beta), atol=1e-12)
    # even part: sigma(g) - sigma(-g) = tanh(g/2)  =>  act(g) + act(-g) = beta*tanh(g/beta)*tanh(g/2)
    np.testing.assert_allclose(act + O.situ(-g, beta), beta * np.tanh(g / beta) * np.tanh(g / 2), atol=1e-12)
    assert O.situ(np.array([0.0]), beta)[0] == 0.0
    d0 = (O.situ(np.array([1e-6]), beta) - O.situ(np.array([-1e-6]), beta))[0] / 2e-6
    assert abs(d0 - 0.5) < 1e-9                       # slope 1/2 at the origin, like SiLU
    # bounded by beta above (the page's (-beta, beta) range) and saturating to it
    assert np.all(act <= beta) and abs(O.situ(np.array([12.0 * beta]), beta)[0] - beta) < 1e-6 * beta
    # below: SiTU lies above SiLU for g < 0, whose textbook minimum is -0.278464542761074
    assert act.min() > -0.278464542761074


def test_situ_tends_to_silu_for_large_beta():
    g = np.linspace(-8, 8, 161)
    silu = g * scipy.special.expit(g)
    np.testing.assert_allclose(O.situ(g, 1e7), silu, atol=1e-9)


def test_softcap_closed_forms():
    beta = 25.0
    assert abs(O.softcap(np.array([beta * math.atanh(0.5)]), beta)[0] - 12.5) < 1e-12
    assert abs(O.softcap(np.array([-beta * math.atanh(0.9)]), beta)[0] + 22.5) < 1e-12
    u = np.linspace(-1e4, 1e4, 20001)
    c = O.softcap(u, beta)
    assert np.all(np.abs(c) <= beta)
    np.testing.assert_allclose(O.softcap(u[:50] * 1e-9, beta), u[:50] * 1e-9, rtol=1e-12)  # slope 1 at 0
    np.testing.assert_allclose(O.softcap(np.linspace(-3, 3, 61), 1e8), np.linspace(-3, 3, 61), atol=1e-12)


# ------------------------------------------------------------------------------------------------
# routing
# ------------------------------------------------------------------------------------------------
def test_router_scores_against_explicit_sums():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 7))
    w = rng.standard_normal((4, 7)).astype(np.float32)
    o = rng.standard_normal(4).astype(np.float32)
    s = O.router_scores(x, w, o)
    for t in range(5):
        for e in range(4):
            l = math.fsum(float(x[t, d]) * float(w[e, d]) for d in range(7)) + float(o[e])
            assert s[t, e] == np.float32(1.0 / (1.0 + math.exp(-l)))
    assert s.dtype == np.float32


def _brute_topk(row_s, row_b, k):
    sh = [np.float32(np.float32(a) + np.float32(b)) for a, b in zip(row_s, row_b)]
    order = sorted(range(len(sh)), key=lambda e: (-float(sh[e]), e))
    return order, sh


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(4)
    T, E, k = 300, 12, 4
    s = (rng.integers(0, 16, (T, E)) / 16.0).astype(np.float32)       # many exact ties
    b = (rng.integers(-2, 3, E) / 16.0).astype(np.float32)
    idx, w, thr = O.select_topk(s, b, k)
    for t in range(T):
        order, sh = _brute_topk(s[t], b, k)
        assert list(idx[t]) == order[:k]
        assert thr[t, 0] == sh[order[k - 1]] and thr[t, 1] == sh[order[k]]
        sel = [float(s[t, e]) for e in order[:k]]
        np.testing.assert_allclose(w[t], np.float32([v / sum(sel) for v in sel]), rtol=1e-6)
    with pytest.raises(ValueError):
        O.select_topk(s, b, E)


# ------------------------------------------------------------------------------------------------
# quantile balancing
# ------------------------------------------------------------------------------------------------
def test_bin_map_fixed_points():
    m = np.float32([-1.0, -2.5, 0.0, 1.0, 3.0, -0.5, 0.5, 0.999])
    np.testing.assert_array_equal(O.qb_bins(m, 1000), [0, 0, 500, 999, 999, 250, 750, 999])
    np.testing.assert_array_equal(O.qb_bins(m, 100), [0, 0, 50, 99, 99, 25, 75, 99])


def test_margin_is_the_bias_shift_that_flips_selection():
    # Leave-one-out meaning of the margin: with the other biases fixed, expert e is chosen by
    # token t after b_e += delta exactly when m(t, e) + delta > 0 (checked by re-running top-k).
    rng = np.random.default_rng(5)
    T, E, k = 40, 10, 3
    s = O.sigmoid(rng.standard_normal((T, E))).astype(np.float32)
    b = (rng.standard_normal(E) * 0.05).astype(np.float32)
    idx, _, thr = O.select_topk(s, b, k)
    m = O.qb_margins(s, b, idx, thr)
    for t in range(0, T, 3):
        for e in range(E):
            for sign in (+1, -1):
                delta = -float(m[t, e]) + sign * 1e-4
                b2 = b.copy()
                b2[e] = np.float32(float(b[e]) + delta)
                idx2, _, _ = O.select_topk(s[t:t + 1], b2, k)
                assert (e in idx2[0]) == (sign > 0), (t, e, sign)


def test_histogram_invariants():
    cfg = replace(TINY, T=512)
    inp = make_inputs(cfg)
    s, idx, w, thr = O.route(inp, cfg)
    H = O.qb_histogram(s, inp["bias"], idx, thr, cfg.n_bins)
    assert H.dtype == np.uint32 and H.shape == (cfg.n_experts, cfg.n_bins)
    np.testing.assert_array_equal(H.sum(axis=1), np.full(cfg.n_experts, cfg.T))
    load = np.bincount(idx.reshape(-1), minlength=cfg.n_experts)
    np.testing.assert_array_equal(H[:, cfg.n_bins // 2:].sum(axis=1), load)
    # additivity across micro-batches
    H1 = O.qb_histogram(s[:200], inp["bias"], idx[:200], thr[:200], cfg.n_bins)
    H2 = O.qb_histogram(s[200:], inp["bias"], idx[200:], thr[200:], cfg.n_bins, hist=H1)
    np.testing.assert_array_equal(H2, H)


def _exact_u(m):
    return np.clip((m.astype(np.float64) + 1.0) / 2.0, 0.0, 1.0)


@pytest.mark.parametrize("n_bins", [100, 1000])
def test_quantile_within_one_bin_of_sorted_quantile(n_bins):
    cfg = replace(TINY, T=2048, n_bins=n_bins)
    inp = make_inputs(cfg)
    s, idx, w, thr = O.route(inp, cfg)
    m = O.qb_margins(s, inp["bias"], idx, thr)
    H = O.qb_histogram(s, inp["bias"], idx, thr, n_bins)
    m_hat = O.qb_quantile_margins(H, cfg.T, cfg.top_k)
    E, k, N = cfg.n_experts, cfg.top_k, cfg.T
    rank = math.ceil((E - k) * N / E)                     # 1-based order statistic
    for e in range(E):
        u_sorted = np.sort(_exact_u(m[:, e]))[rank - 1]
        u_hat = (m_hat[e] + 1.0) / 2.0
        assert abs(u_hat - u_sorted) <= 1.0 / n_bins + 1e-12


def test_bias_update_gives_target_load_brute_force():
    # Tiny case: after the update of expert e alone, the number of tokens choosing e lies in the
    # count range of the bin holding the quantile, and that range contains the target N*k/E.
    rng = np.random.default_rng(6)
    T, E, k, NB = 64, 8, 2, 1000
    s = O.sigmoid(rng.standard_normal((T, E)) * 1.5).astype(np.float32)
    b = np.zeros(E, dtype=np.float32)
    idx, _, thr = O.select_topk(s, b, k)
    H = O.qb_histogram(s, b, idx, thr, NB)
    new_b, H0 = O.qb_update(H, T, b, k)
    assert not H0.any()
    c_star = (E - k) * T / E
    target = T * k / E
    for e in range(E):
        cum = np.cumsum(H[e].astype(np.int64))
        j = int(np.argmax(cum >= c_star))
        lo_cnt = T - int(cum[j])
        hi_cnt = T - (int(cum[j - 1]) if j else 0)
        assert lo_cnt <= target <= hi_cnt
        b2 = b.copy()
        b2[e] = new_b[e]
        idx2, _, _ = O.select_topk(s, b2, k)
        load = int((idx2 == e).sum())
        assert lo_cnt <= load <= hi_cnt, (e, lo_cnt, load, hi_cnt)


def test_bias_update_without_tokens_is_identity():
    H = np.zeros((4, 10), dtype=np.uint32)
    b = np.float32([0.1, -0.2, 0.0, 3.0])
    nb, _ = O.qb_update(H, 0, b, 1)
    np.testing.assert_array_equal(nb, b)


def test_qb_loop_balances_skewed_router():
    # The update moves a strongly skewed router toward the uniform load N*k/E.
    rng = np.random.default_rng(7)
    T, E, k, NB = 4096, 16, 2, 1000
    pref = np.linspace(-2, 2, E)
    b = np.zeros(E, dtype=np.float32)
    ratios = []
    for step in range(4):
        s = O.sigmoid(rng.standard_normal((T, E)) + pref).astype(np.float32)
        idx, _, thr = O.select_topk(s, b, k)
        load = np.bincount(idx.reshape(-1), minlength=E)
        ratios.append(load.max() / load.mean())
        H = O.qb_histogram(s, b, idx, thr, NB)
        b, _ = O.qb_update(H, T, b, k)
    assert ratios[0] > 3.0 and ratios[-1] < 1.25


# ------------------------------------------------------------------------------------------------
# permutation, experts, combine, norm
# ------------------------------------------------------------------------------------------------
def test_permutation_brute_force():
    rng = np.random.default_rng(8)
    T, E, k = 100, 9, 3
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    off, st, sp = O.permute(idx, E)
    rows = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t, j] == e:
                    rows.append((t, j))
    assert off[0] == 0 and off[-1] == T * k
    for e in range(E):
        assert off[e + 1] - off[e] == int((idx == e).sum())
    for r, (t, j) in enumerate(rows):
        assert st[r] == t and sp[t * k + j] == r
    assert sorted(sp.tolist()) == list(range(T * k))


def test_glu_gate_is_first_half():
    # a = identity rows, so the projections are columns of W1 read directly.
    rng = np.random.default_rng(9)
    I, K = 3, 4
    w1 = rng.standard_normal((2 * I, K))
    w2 = np.eye(I)
    a = np.eye(K)
    h, y = O.situ_glu_ffn(a, w1, w2, 4.0, 25.0, "f32")
    g, u = w1[:I].T, w1[I:].T
    want = O.situ(g, 4.0) * O.softcap(u, 25.0)
    np.testing.assert_allclose(h, want, rtol=1e-7)
    np.testing.assert_allclose(y, want, rtol=1e-7)


def test_combine_with_one_hot_and_equal_rows():
    rng = np.random.default_rng(10)
    y = rng.standard_normal((5, 3, 7))
    w = np.zeros((5, 3), dtype=np.float32)
    w[:, 1] = 1
    np.testing.assert_array_equal(O.combine(y, w), y[:, 1])
    yy = np.repeat(y[:, :1], 3, axis=1)
    np.testing.assert_allclose(O.combine(yy, np.full((5, 3), 1 / 3, np.float32)), y[:, 0], rtol=1e-7)


def test_rms_norm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(11)
    z = rng.standard_normal((50, 64)) * rng.uniform(0.01, 100, (50, 1))
    eps = 1e-6
    n = O.rms_norm(z, np.ones(64, np.float32), eps)
    ms = np.mean(z * z, axis=1)
    np.testing.assert_allclose(np.sqrt(np.mean(n * n, axis=1)), np.sqrt(ms / (ms + eps)), rtol=1e-12)
    np.testing.assert_allclose(O.rms_norm(3.0 * z, np.ones(64, np.float32), 0.0),
                               O.rms_norm(z, np.ones(64, np.float32), 0.0), rtol=1e-12)
    g = rng.uniform(0.5, 2, 64).astype(np.float32)
    np.testing.assert_allclose(O.rms_norm(z, g, eps), n * g.astype(np.float64), rtol=1e-12)


def test_shared_experts_equal_one_concatenated_ffn():
    cfg = replace(TINY, n_shared=3)
    inp = make_inputs(cfg)
    x = O.to_f64(inp["x"], "f32")
    w1s, w2s = O.to_f64(inp["w1s"], "f32"), O.to_f64(inp["w2s"], "f32")
    h_s, y_sh = O.shared_experts(x, w1s, w2s, 4.0, 25.0, "f32")
    Is = w1s.shape[1] // 2
    w1_cat = np.concatenate([w1s[:, :Is].reshape(-1, w1s.shape[2]), w1s[:, Is:].reshape(-1, w1s.shape[2])])
    w2_cat = np.concatenate(list(w2s), axis=1)
    h, _ = O.situ_glu_ffn(x, w1_cat, w2_cat, 4.0, 25.0, "f32")
    np.testing.assert_array_equal(h, h_s)
    np.testing.assert_allclose(y_sh, h @ w2_cat.T, rtol=1e-6, atol=1e-7)


def test_routed_layer_equals_dense_masked_evaluation():
    for cfg in (TINY, replace(TINY, name="tiny_bf16", act_dtype="bf16")):
        inp = make_inputs(cfg)
        r = O.forward(inp, cfg)
        wd = np.zeros((cfg.T, cfg.n_experts), dtype=np.float32)
        np.put_along_axis(wd, r["idx"], r["w"], axis=1)
        dense = O.dense_masked_forward(inp, cfg, wd)
        rms = np.sqrt(np.mean(dense ** 2))
        assert np.max(np.abs(dense - r["out_pre"])) <= 1e-6 * rms


def test_forward_layouts_consistent():
    cfg = TINY
    inp = make_inputs(cfg)
    r = O.forward(inp, cfg)
    T, k = cfg.T, cfg.top_k
    np.testing.assert_array_equal(r["x_perm"], r["x_lat"][r["sorted_token"]])
    # the sorted y rows gathered back through slot_of_pair reproduce z
    y_pairs = r["y"][r["slot_of_pair"]].reshape(T, k, -1)
    np.testing.assert_allclose(O.combine(y_pairs, r["w"]), r["z"], rtol=1e-12)


# ------------------------------------------------------------------------------------------------
# numbers the pages print
# ------------------------------------------------------------------------------------------------
def test_k3_constants_from_pages():
    g = {k: v["value"] for k, v in json.load(open(os.path.join(GOLDEN, "k3_constants.json"))).items()
         if not k.startswith("_")}
    k3 = CONFIGS["k3_prefill"]
    assert (k3.d_model, k3.d_latent, k3.n_experts, k3.top_k, k3.n_shared) == \
        (g["d_model"], g["d_latent"], g["routed_experts"], g["active_routed"], g["shared_experts"])
    assert (k3.beta1, k3.beta2, k3.n_bins) == (g["beta1"], g["beta2"], g["n_bins"])
    assert g["routed_experts"] + g["shared_experts"] == g["total_experts"]
    assert g["active_routed"] + g["shared_experts"] == g["active_per_token"]
    # same sparsity for 448-choose-8 and 896-choose-16
    assert g["earlier_plan_active"] / g["earlier_plan_experts"] == g["active_routed"] / g["routed_experts"]
    assert round(100 * g["active_routed"] / g["total_experts"], 1) == g["activation_ratio_percent"]


def test_latent_experts_nearly_halve_expert_flops():
    # lukebest.github.io "Stable Latent MoE", Latent-Space MoE: expert FLOPs nearly halved when the
    # experts run at d_latent = d_model / 2.
    k3 = CONFIGS["k3_prefill"]
    lat = O.expert_flops_per_token(k3.d_latent, k3.inter, k3.top_k)
    full = O.expert_flops_per_token(k3.d_model, k3.inter, k3.top_k)
    assert lat / full == 0.5
