"""Pins of the backward oracle (CPU): its gradients against central finite differences of an
independent float64 forward written out here, plus closed forms and invariants of single steps.

The forward below is the layer of [vxz] 01-02 / [slm] "Latent-Space MoE" in plain float64, coded
apart from the oracle (its own sigmoid, SiTU and soft cap). The routing (top-k set) is held fixed,
as the backward assumes: the balancing bias only selects experts ([vxz] 02).
"""
import numpy as np
import pytest

from oracle import lmoe_oracle as O
from oracle import lmoe_oracle_bwd as B


class Cfg:
    top_k = 2
    n_experts = 6
    inter = 8
    beta1 = 4.0
    beta2 = 25.0
    rms_eps = 1e-6
    act_dtype = "f64"


T, D, L, E, K, I, S, IS = 10, 12, 8, 6, 2, 8, 2, 4


def _sig(a):
    return 1.0 / (1.0 + np.exp(-a))


def _glu(gu, b1, b2):
    g, u = gu[..., : gu.shape[-1] // 2], gu[..., gu.shape[-1] // 2:]
    return b1 * np.tanh(g / b1) * _sig(g) * (b2 * np.tanh(u / b2))


def params(seed=0):
    rng = np.random.default_rng(seed)
    p = {
        "x": rng.standard_normal((T, D)),
        "w_router": rng.standard_normal((E, D)) * 2.0 / np.sqrt(D),
        "w_down": rng.standard_normal((L, D)) / np.sqrt(D),
        "w1": rng.standard_normal((E, 2 * I, L)) * 2.0 / np.sqrt(L),
        "w2": rng.standard_normal((E, L, I)) / np.sqrt(I),
        "gamma": 1.0 + 0.2 * rng.standard_normal(L),
        "w_up": rng.standard_normal((D, L)) / np.sqrt(L),
        "w1s": rng.standard_normal((S, 2 * IS, D)) * 2.0 / np.sqrt(D),
        "w2s": rng.standard_normal((S, D, IS)) / np.sqrt(IS),
    }
    s = _sig(p["x"] @ p["w_router"].T)
    idx = np.argsort(-s, axis=1, kind="stable")[:, :K]
    srt = -np.sort(-s, axis=1)
    assert np.min(srt[:, K - 1] - srt[:, K]) > 1e-4      # no near-tie: the selection is stable
    return p, idx


def forward64(p, idx):
    """Plain float64 layer forward with the top-k set idx; returns out and the stored tensors."""
    x = p["x"]
    s = _sig(x @ p["w_router"].T)
    sel = np.take_along_axis(s, idx, axis=1)
    w = sel / sel.sum(axis=1, keepdims=True)
    x_lat = x @ p["w_down"].T
    y_pair = np.zeros((T, K, L))
    h_pair = np.zeros((T, K, I))
    for t in range(T):
        for j in range(K):
            e = idx[t, j]
            h_pair[t, j] = _glu(x_lat[t] @ p["w1"][e].T, 4.0, 25.0)
            y_pair[t, j] = h_pair[t, j] @ p["w2"][e].T
    z = np.einsum("tk,tkl->tl", w, y_pair)
    n = p["gamma"] * z / np.sqrt(np.mean(z * z, axis=1, keepdims=True) + 1e-6)
    hs = [_glu(x @ p["w1s"][j].T, 4.0, 25.0) for j in range(S)]
    out = n @ p["w_up"].T + sum(hs[j] @ p["w2s"][j].T for j in range(S))
    offsets, sorted_token, slot_of_pair = O.permute(idx, E)
    order = np.empty(T * K, dtype=np.int64)
    order[slot_of_pair] = np.arange(T * K)
    fwd = {"s": s, "idx": idx.astype(np.int32), "w": w, "offsets": offsets, "sorted_token": sorted_token,
           "slot_of_pair": slot_of_pair, "x_lat": x_lat, "h": h_pair.reshape(T * K, I)[order],
           "y": y_pair.reshape(T * K, L)[order], "n": n, "h_s": np.concatenate(hs, axis=1)}
    return out, fwd


def _grad_of(g, name, ix):
    """The oracle gradient entry matching parameter entry ix (packed layouts for the shared experts)."""
    if name == "w1s":
        j, r, d = ix
        row = (j * IS + r) if r < IS else (S * IS + j * IS + r - IS)
        return g["dW1s_packed"][row, d]
    if name == "w2s":
        j, d, c = ix
        return g["dW2s_packed"][d, j * IS + c]
    key = {"x": "dx", "w_router": "dW_r", "w_down": "dW_dn", "w1": "dW1", "w2": "dW2", "gamma": "dgamma",
           "w_up": "dW_up"}[name]
    return g[key][ix]


@pytest.mark.parametrize("name", ["x", "w_router", "w_down", "w1", "w2", "gamma", "w_up", "w1s", "w2s"])
def test_gradients_match_finite_differences(name):
    p, idx = params(0)
    rng = np.random.default_rng(1)
    dout = rng.standard_normal((T, D))
    out, fwd = forward64(p, idx)
    g = B.backward(p, Cfg, fwd, dout, dtype="f64")
    shape = p[name].shape
    picks = [tuple(int(rng.integers(0, n)) for n in shape) for _ in range(8)]
    if name in ("w1", "w2"):      # entries of experts that received tokens
        used = np.unique(idx)
        picks = [(int(rng.choice(used)),) + pk[1:] for pk in picks]
    h = 1e-5
    for ix in picks:
        q = {kk: v.copy() for kk, v in p.items()}
        q[name][ix] += h
        op, _ = forward64(q, idx)
        q[name][ix] -= 2 * h
        om, _ = forward64(q, idx)
        fd = float(np.sum(dout * (op - om)) / (2 * h))
        an = float(_grad_of(g, name, ix))
        assert abs(fd - an) <= 1e-7 * (1.0 + abs(fd)), (name, ix, fd, an)


def test_unused_expert_gradients_are_zero():
    p, idx = params(0)
    _, fwd = forward64(p, idx)
    g = B.backward(p, Cfg, fwd, np.ones((T, D)), dtype="f64")
    for e in set(range(E)) - set(np.unique(idx).tolist()):
        assert not g["dW1"][e].any() and not g["dW2"][e].any() and not g["dW_r"][e].any()


def test_situ_derivative_closed_forms():
    # SiTU'(0) = 1/2 (tanh'(0) sigmoid(0)); large |g|: derivative of a saturated gate tends to 0
    assert B.situ_grad(np.array([0.0]), 4.0)[0] == pytest.approx(0.5, abs=1e-15)
    assert abs(B.situ_grad(np.array([60.0]), 4.0)[0]) < 1e-9
    assert abs(B.situ_grad(np.array([-60.0]), 4.0)[0]) < 1e-9
    g = np.linspace(-12, 12, 97)
    fd = (O.situ(g + 1e-6, 4.0) - O.situ(g - 1e-6, 4.0)) / 2e-6
    np.testing.assert_allclose(B.situ_grad(g, 4.0), fd, atol=1e-8)
    # beta -> infinity: SiLU' = sigmoid(g) (1 + g (1 - sigmoid(g)))
    s = 1.0 / (1.0 + np.exp(-g))
    np.testing.assert_allclose(B.situ_grad(g, 1e9), s * (1 + g * (1 - s)), atol=1e-7)
    u = np.linspace(-300, 300, 61)
    np.testing.assert_allclose(B.softcap_grad(u, 25.0), 1.0 / np.cosh(u / 25.0) ** 2, rtol=1e-12, atol=1e-15)


def test_routing_weight_gradient_is_scale_invariant():
    # w = s / sum(s) does not change when every selected s is scaled: sum_j ds_j s_j = 0, i.e.
    # sum_j dl_j / (1 - s_j) = 0 for dl = ds * s * (1 - s)
    rng = np.random.default_rng(3)
    s = rng.uniform(0.05, 0.95, (20, 5))
    dl = B.weights_backward(rng.standard_normal((20, 5)), s)
    np.testing.assert_allclose(np.sum(dl / (1.0 - s), axis=1), 0.0, atol=1e-12)


def test_rms_norm_backward_identity():
    # with gamma = 1: sum_l z_l dz_l = r * sum(dn z) * (1 - r^2 ms) = r * sum(dn z) * eps / (ms + eps)
    rng = np.random.default_rng(4)
    z = rng.standard_normal((6, 16))
    dn = rng.standard_normal((6, 16))
    eps = 0.3
    dz, _ = B.rms_norm_backward(z, np.ones(16), dn, eps)
    ms = np.mean(z * z, axis=1)
    r = 1.0 / np.sqrt(ms + eps)
    np.testing.assert_allclose(np.sum(z * dz, axis=1), r * np.sum(dn * z, axis=1) * eps / (ms + eps), rtol=1e-12)


def test_storage_rounding_stays_close_to_exact_gradients():
    """With bf16 storage points (RB1) the gradients stay within a few bf16 roundings of the exact
    ones; float32 storage points stay within float32 error."""
    p, idx = params(0)
    p = {kk: (O.round_to_bf16(v) if kk not in ("w_router", "gamma") else v) for kk, v in p.items()}
    rng = np.random.default_rng(5)
    dout = O.round_to_bf16(rng.standard_normal((T, D)))
    _, fwd = forward64(p, idx)
    exact = B.backward(p, Cfg, fwd, dout, dtype="f64")
    for dt, tol in (("bf16", 0.05), ("f32", 1e-5)):
        approx = B.backward(p, Cfg, fwd, dout, dtype=dt)
        for key in ("dx", "dW_r", "dW_up", "dW1", "dW2", "dW_dn", "dW1s_packed", "dgamma"):
            a, b = exact[key], approx[key]
            assert np.max(np.abs(a - b)) <= tol * np.sqrt(np.mean(a * a)), (dt, key)
