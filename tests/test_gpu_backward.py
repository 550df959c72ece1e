"""GPU parity of the backward calls against the backward oracle.

Each call is checked against the oracle fed the GPU's own inputs to that call (one rounding of the
storage type for activation gradients; float32 accumulation error, relative to the tensor's RMS,
for the float32 gradients), then the whole chain against the oracle's end-to-end gradients from
the GPU's forward tensors. Cases: the f32 layer; the f32 layer at T = 1024, whose 4096 expert rows
take the 256-row tiles for the recomputed GEMM1 and the 128-row register tiles for the [K, N]
products, each with its own m-tile numbering; a bf16 layer with a token count that is not a
multiple of 64; and a bf16 layer whose biases leave most experts without tokens. Every case draws
a non-unit RMSNorm gain and a non-zero starting bias.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_space_routed_amd import _lib as C
from oracle import lmoe_oracle as O
from oracle import lmoe_oracle_bwd as B
from workloads import CONFIGS
from workloads.inputs import make_inputs

from .gpu_helpers import assert_close_rows, device_layer, host, say

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_f32": (CONFIGS["tiny_f32"], 0),
    "tiny_f32_T1024": (replace(CONFIGS["tiny_f32"], T=1024), 0),
    "mid_bf16_T1000": (replace(CONFIGS["mid_bf16"], T=1000), 0),
    "mid_bf16_few_experts": (replace(CONFIGS["mid_bf16"], T=512), 8),
}


def assert_f32(got, ref, what, rel=2e-5):
    """float32 results of long f32 accumulations: |err| <= rel * RMS(ref) + 2^-20 |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    err = np.abs(got - ref)
    bad = err > rel * rms + 2.0 ** -20 * np.abs(ref)
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} off; worst {err.max():.3g} (rms {rms:.3g})"
    return float(err.max() / rms)


def run_case(name):
    cfg, n_live = CASES[name]
    dt = cfg.act_dtype
    inp = make_inputs(cfg, seed=3, gain_bias=True)
    if n_live:  # every expert but the first n_live is pushed out of every top-k
        inp["bias"] = np.where(np.arange(cfg.n_experts) < n_live, 0.0, -10.0).astype(np.float32)
    layer, x = device_layer(cfg, inp)
    b = layer.forward(x, accumulate_hist=False)
    rng = np.random.default_rng(11)
    dout_f = rng.standard_normal((cfg.T, cfg.d_model)).astype(np.float32)
    dout_h = O.store(dout_f, dt)
    dout = torch.as_tensor(dout_h, device="cuda").to(layer.dt)
    torch.cuda.synchronize()
    return cfg, inp, layer, x, b, dout, dout_h


@pytest.mark.parametrize("name", list(CASES))
def test_backward_stages(name):
    cfg, inp, layer, x, b, dout, dout_h = run_case(name)
    dt = cfg.act_dtype
    T, k, L, D, E, I = cfg.T, cfg.top_k, cfg.d_latent, cfg.d_model, cfg.n_experts, cfg.inter
    S, Is = cfg.n_shared, cfg.inter_shared
    Ss = S * Is
    shape = C.make_shape(cfg, T)
    w = layer.w
    dev, tdt, f32 = "cuda", layer.dt, torch.float32
    f64 = lambda name: O.to_f64(inp[name], dt)  # noqa: E731
    W_up, W_dn, W1, W2 = f64("w_up"), f64("w_down"), f64("w1"), f64("w2")
    W1s, W2s = f64("w1s"), f64("w2s")
    W1s_p = np.concatenate([W1s[:, :Is].reshape(Ss, -1), W1s[:, Is:].reshape(Ss, -1)], axis=0)
    W2s_p = np.concatenate(list(W2s), axis=1)
    xh = O.to_f64(inp["x"], dt)

    wt = {"w_up_t": torch.empty(L, D, dtype=tdt, device=dev), "w_down_t": torch.empty(D, L, dtype=tdt, device=dev),
          "w2s_t": torch.empty(Ss, D, dtype=tdt, device=dev), "w1s_t": torch.empty(D, 2 * Ss, dtype=tdt, device=dev)}
    C.lmoe_bwd_transpose_weights(shape, w["w_up"], layer.w2s_packed, layer.w1s_packed, w["w_down"], wt["w_up_t"],
                                 wt["w2s_t"], wt["w1s_t"], wt["w_down_t"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(wt["w_up_t"]), host(w["w_up"]).T)
    np.testing.assert_array_equal(host(wt["w2s_t"]), host(layer.w2s_packed).T)
    np.testing.assert_array_equal(host(wt["w1s_t"]), host(layer.w1s_packed).T)
    ws = lambda which: torch.empty(max(C.workspace_bytes(shape, which), 256), dtype=torch.uint8, device=dev)  # noqa

    # B1: up-projection
    dn = torch.empty(T, L, dtype=tdt, device=dev)
    dh_s = torch.empty(T, Ss, dtype=tdt, device=dev)
    dW_up = torch.empty(D, L, dtype=f32, device=dev)
    dW2s = torch.empty(D, Ss, dtype=f32, device=dev)
    C.lmoe_bwd_up(shape, dout, b["n"], b["h_s"], wt["w_up_t"], wt["w2s_t"], dn, dh_s, dW_up, dW2s, ws(C.LMOE_CALL_BWD_UP))
    torch.cuda.synchronize()
    n_h, hs_h = host(b["n"]), host(b["h_s"])[:, :Ss]
    assert_close_rows(host(dn), O.store(dout_h @ W_up, dt), dt, f"{name} dn")
    assert_close_rows(host(dh_s), O.store(dout_h @ W2s_p, dt), dt, f"{name} dh_s")
    assert_f32(host(dW_up), dout_h.T @ n_h, f"{name} dW_up")
    assert_f32(host(dW2s), dout_h.T @ hs_h, f"{name} dW2s")
    say(f"[{name}] up-projection backward ok")

    # B2: combine + norm + routing weights
    dy = torch.empty(T * k, L, dtype=tdt, device=dev)
    dl = torch.empty(T, k, dtype=f32, device=dev)
    dl_sorted = torch.empty(T * k, dtype=f32, device=dev)
    dgamma = torch.empty(L, dtype=f32, device=dev)
    C.lmoe_bwd_combine_norm(shape, dn, b["y"], b["slot_of_pair"], b["idx"], b["scores"], b["w"], w.get("gamma"), dy, dl,
                            dl_sorted, dgamma, ws(C.LMOE_CALL_BWD_COMBINE_NORM))
    torch.cuda.synchronize()
    idx = host(b["idx"]).astype(np.int64)
    slot = host(b["slot_of_pair"]).astype(np.int64).reshape(T, k)
    y_h = host(b["y"])
    w_h = host(b["w"])
    s_sel = np.take_along_axis(host(b["scores"]), idx, axis=1)
    y_pair = y_h[slot.reshape(-1)].reshape(T, k, L)
    z = np.einsum("tk,tkl->tl", w_h, y_pair)
    dz, dgamma_ref = B.rms_norm_backward(z, inp["gamma"], host(dn), cfg.rms_eps)
    dw_ref, dy_pair = B.combine_backward(dz, y_pair, w_h)
    dy_ref = np.empty_like(y_h)
    dy_ref[slot.reshape(-1)] = O.store(dy_pair.reshape(T * k, L), dt)
    assert_close_rows(host(dy), dy_ref, dt, f"{name} dy")
    assert_f32(host(dgamma), dgamma_ref, f"{name} dgamma", rel=1e-4)
    dl_ref = B.weights_backward(dw_ref, s_sel)
    assert_f32(host(dl), dl_ref, f"{name} dlogit", rel=1e-4)
    got_sorted = host(dl_sorted)
    np.testing.assert_array_equal(got_sorted[slot.reshape(-1)], host(dl).reshape(-1))
    say(f"[{name}] combine/norm/routing-weight backward ok")

    # B3: router
    dW_r = torch.empty(E, D, dtype=f32, device=dev)
    dx = torch.empty(T, D, dtype=f32, device=dev)
    C.lmoe_bwd_router(shape, x, w["w_router"], dl, dl_sorted, b["idx"], b["offsets"], b["sorted_token"], dW_r, dx)
    torch.cuda.synchronize()
    dW_r_ref, dx_r_ref = B.router_backward(host(dl), idx, xh, inp["w_router"])
    assert_f32(host(dW_r), dW_r_ref, f"{name} dW_r")
    assert_f32(host(dx), dx_r_ref, f"{name} dx (router part)")
    dx_r = host(dx).copy()
    say(f"[{name}] router backward ok")

    # B4: routed experts
    rows = T * k
    dh = torch.empty(rows, I, dtype=tdt, device=dev)
    dgu = torch.empty(rows, 2 * I, dtype=tdt, device=dev)
    dx_perm = torch.empty(rows, L, dtype=tdt, device=dev)
    dW1 = torch.empty(E, 2 * I, L, dtype=f32, device=dev)
    dW2 = torch.empty(E, L, I, dtype=f32, device=dev)
    C.lmoe_bwd_experts(shape, b["x_lat"], b["sorted_token"], b["offsets"], w["w1"], w["w2"], b["h"], dy, dh, dgu,
                       dx_perm, dW1, dW2, ws(C.LMOE_CALL_BWD_EXPERTS))
    torch.cuda.synchronize()
    off = host(b["offsets"]).astype(np.int64)
    st = host(b["sorted_token"]).astype(np.int64)
    x_lat = host(b["x_lat"])
    dy_g, dh_g, dgu_g, h_g = host(dy), host(dh), host(dgu), host(b["h"])
    dh_ref = np.zeros_like(dh_g)
    dgu_ref = np.zeros_like(dgu_g)
    dxp_ref = np.zeros((rows, L))
    dW1_ref = np.zeros((E, 2 * I, L))
    dW2_ref = np.zeros((E, L, I))
    for e in range(E):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        a_e = x_lat[st[r0:r1]]
        dh_ref[r0:r1] = O.store(dy_g[r0:r1] @ W2[e], dt)
        dW2_ref[e] = dy_g[r0:r1].T @ h_g[r0:r1]
        dgu_ref[r0:r1] = O.store(B.glu_backward(a_e @ W1[e].T, dh_g[r0:r1], cfg.beta1, cfg.beta2), dt)
        dxp_ref[r0:r1] = O.store(dgu_g[r0:r1] @ W1[e], dt)
        dW1_ref[e] = dgu_g[r0:r1].T @ a_e
    assert_close_rows(dh_g, dh_ref, dt, f"{name} dh")
    assert_close_rows(dgu_g, dgu_ref, dt, f"{name} dgu")
    assert_close_rows(host(dx_perm), dxp_ref, dt, f"{name} dx_perm")
    assert_f32(host(dW2), dW2_ref, f"{name} dW2")
    assert_f32(host(dW1), dW1_ref, f"{name} dW1")
    empty = np.nonzero(np.diff(off) == 0)[0]
    assert not host(dW1)[empty].any() and not host(dW2)[empty].any()
    say(f"[{name}] routed experts backward ok ({len(empty)} experts without tokens)")

    # B5: un-permutation and down-projection
    dx_lat = torch.empty(T, L, dtype=tdt, device=dev)
    dW_dn = torch.empty(L, D, dtype=f32, device=dev)
    C.lmoe_bwd_down(shape, x, dx_perm, b["slot_of_pair"], wt["w_down_t"], dx_lat, dW_dn, dx, ws(C.LMOE_CALL_BWD_DOWN))
    torch.cuda.synchronize()
    dxp_g = host(dx_perm)
    dxl_ref = O.store(dxp_g[slot.reshape(-1)].reshape(T, k, L).sum(axis=1), dt)
    assert_close_rows(host(dx_lat), dxl_ref, dt, f"{name} dx_lat")
    dxl_g = host(dx_lat)
    assert_f32(host(dW_dn), dxl_g.T @ xh, f"{name} dW_dn")
    assert_f32(host(dx), dx_r + dxl_g @ W_dn, f"{name} dx (router + down)")
    dx_rd = host(dx).copy()
    say(f"[{name}] down-projection backward ok")

    # B6: shared experts
    dgu_s = torch.empty(T, 2 * Ss, dtype=tdt, device=dev)
    dW1s = torch.empty(2 * Ss, D, dtype=f32, device=dev)
    C.lmoe_bwd_shared(shape, x, layer.w1s_packed, wt["w1s_t"], dh_s, dgu_s, dW1s, dx, ws(C.LMOE_CALL_BWD_SHARED))
    torch.cuda.synchronize()
    dgus_ref = O.store(B.glu_backward(xh @ W1s_p.T, host(dh_s), cfg.beta1, cfg.beta2), dt)
    assert_close_rows(host(dgu_s), dgus_ref, dt, f"{name} dgu_s")
    dgus_g = host(dgu_s)
    assert_f32(host(dW1s), dgus_g.T @ xh, f"{name} dW1s")
    assert_f32(host(dx), dx_rd + dgus_g @ W1s_p, f"{name} dx (all parts)")
    say(f"[{name}] shared experts backward ok")


# Activation-gradient storage points (each rounded to the activation type) on the path from dout
# to each gradient: dn, dy, dh, d[g|u], dx_perm, dx_lat for the routed experts' inputs; dh_s for
# the shared experts.
ROUNDINGS = {"dx": 6, "dW_r": 1, "dW_up": 0, "dW2s_packed": 0, "dW1": 4, "dW2": 2, "dW_dn": 6,
             "dW1s_packed": 1, "dgamma": 1}


@pytest.mark.parametrize("name", ["tiny_f32", "tiny_f32_T1024", "mid_bf16_T1000"])
def test_backward_end_to_end(name):
    """LatentMoE.backward against the oracle's whole chain from the GPU's forward tensors. Each
    storage point upstream of a gradient can differ by one unit u in the last place between the two
    sides (the rounding of a value that differs in its f32 accumulation order), so with n storage
    points on a gradient's path its error is (n + 1) such flips propagated through sums: the RMS of
    the error is bounded by (n + 1) u RMS(ref) (u = 2^-7 bf16, 2^-20 f32, plus the f32
    accumulation of the weight-gradient sums), and its maximum over N elements by the
    extreme-value factor sqrt(2 ln N) on top (a non-unit RMSNorm gain makes some rows of a gradient
    several times the tensor's RMS, and their flips with them)."""
    cfg, inp, layer, x, b, dout, dout_h = run_case(name)
    dt = cfg.act_dtype
    g = layer.backward(x, b, dout)
    g2 = layer.backward(x, b, dout)
    torch.cuda.synchronize()
    for key in ("dx", "dW1", "dW_r", "dgamma"):
        assert torch.equal(g[key], g2[key]), f"{key} not deterministic"
    T, k = cfg.T, cfg.top_k
    fwd = {"s": host(b["scores"]), "idx": host(b["idx"]), "w": host(b["w"]), "offsets": host(b["offsets"]),
           "sorted_token": host(b["sorted_token"]), "slot_of_pair": host(b["slot_of_pair"]), "x_lat": host(b["x_lat"]),
           "h": host(b["h"]), "y": host(b["y"]), "n": host(b["n"]),
           "h_s": host(b["h_s"])[:, : cfg.n_shared * cfg.inter_shared]}
    ref = B.backward(inp, cfg, fwd, dout_h)
    ulp = 2.0 ** -7 if dt == "bf16" else 2.0 ** -20
    for key in ("dx", "dW_r", "dW_up", "dW2s_packed", "dW1", "dW2", "dW_dn", "dW1s_packed", "dgamma"):
        tol = (ROUNDINGS[key] + 1) * ulp + 2e-5
        got = host(g[key])
        want = ref[key]
        if key == "dW2s_packed":
            got = got[:, : want.shape[1]]
        rms = float(np.sqrt(np.mean(want * want)))
        diff = got - want
        err_rms = float(np.sqrt(np.mean(diff * diff)))
        err = float(np.max(np.abs(diff)))
        ev = float(np.sqrt(2.0 * np.log(max(diff.size, 2))))
        say(f"[{name}] {key}: RMS err/RMS = {err_rms / rms:.2e} (bound {tol:.2e}), max|err|/RMS = {err / rms:.2e} "
            f"(bound {ev * tol:.2e})")
        assert err_rms <= tol * rms, (key, err_rms, rms)
        assert err <= ev * tol * rms, (key, err, rms)


def test_backward_k3_prefill_sampled():
    """K3 prefill (T=8192) backward through LatentMoE.backward, with a random RMSNorm gain and bias;
    every stage checked on 1024 sampled tokens, two experts in full and sampled weight rows, against
    the oracle fed the GPU's own inputs to that stage (so its routing: near-ties do not matter)."""
    cfg = CONFIGS["k3_prefill"]
    dt = cfg.act_dtype
    T, k, L, D, E, I = cfg.T, cfg.top_k, cfg.d_latent, cfg.d_model, cfg.n_experts, cfg.inter
    S, Is = cfg.n_shared, cfg.inter_shared
    Ss = S * Is
    say("[k3 bwd] inputs")
    inp = make_inputs(cfg, seed=0, gain_bias=True)
    layer, x = device_layer(cfg, inp)
    b = layer.forward(x, accumulate_hist=False)
    rng = np.random.default_rng(12)
    dout_h = O.store(rng.standard_normal((T, D)).astype(np.float32), dt)
    dout = torch.as_tensor(dout_h, device="cuda").to(layer.dt)
    say("[k3 bwd] GPU backward")
    g = layer.backward(x, b, dout)
    torch.cuda.synchronize()
    toks = np.sort(rng.choice(T, 1024, replace=False))
    say(f"[k3 bwd] checking {len(toks)} tokens")
    tt = torch.as_tensor(toks, device="cuda")
    xh = O.to_f64(inp["x"][toks], dt)
    f64 = lambda a: O.to_f64(a, dt)  # noqa: E731
    W_up = f64(inp["w_up"])
    n_h = host(b["n"][tt])
    # up-projection: dn rows, dW_up rows
    assert_close_rows(host(g["dn"][tt]), O.store(dout_h[toks] @ W_up, dt), dt, "k3 dn")
    drows = rng.choice(D, 4, replace=False)
    n_all = host(b["n"])
    assert_f32(host(g["dW_up"][torch.as_tensor(drows, device="cuda")]), dout_h[:, drows].T @ n_all, "k3 dW_up rows")
    say("[k3 bwd] up-projection ok")
    # combine / norm / routing weights on the sampled tokens
    idx = host(b["idx"]).astype(np.int64)
    slot = host(b["slot_of_pair"]).astype(np.int64).reshape(T, k)
    y_pair = host(b["y"][torch.as_tensor(slot[toks].reshape(-1), device="cuda")]).reshape(len(toks), k, L)
    w_h = host(b["w"])[toks]
    z = np.einsum("tk,tkl->tl", w_h, y_pair)
    dz, _ = B.rms_norm_backward(z, inp["gamma"], host(g["dn"][tt]), cfg.rms_eps)
    dw_ref, dy_pair = B.combine_backward(dz, y_pair, w_h)
    dy_g = host(g["dy"][torch.as_tensor(slot[toks].reshape(-1), device="cuda")]).reshape(len(toks), k, L)
    assert_close_rows(dy_g, O.store(dy_pair, dt), dt, "k3 dy")
    s_sel = np.take_along_axis(host(b["scores"])[toks], idx[toks], axis=1)
    assert_f32(host(g["dl"])[toks], B.weights_backward(dw_ref, s_sel), "k3 dlogit", rel=1e-4)
    say("[k3 bwd] combine/norm/routing weights ok")
    # routed experts: two sampled experts in full (their rows, dh, dgu, dx_perm, dW1, dW2, dW_r)
    off = host(b["offsets"]).astype(np.int64)
    st = host(b["sorted_token"]).astype(np.int64)
    dl_sorted = host(g["dl_sorted"])
    x_lat = host(b["x_lat"])
    for e in rng.choice(E, 2, replace=False):
        r0, r1 = off[e], off[e + 1]
        rr = torch.arange(int(r0), int(r1), device="cuda")
        W1e, W2e = f64(inp["w1"][e]), f64(inp["w2"][e])
        a_e = x_lat[st[r0:r1]]
        dy_e, dh_e, dgu_e, h_e = host(g["dy"][rr]), host(g["dh"][rr]), host(g["dgu"][rr]), host(b["h"][rr])
        assert_close_rows(dh_e, O.store(dy_e @ W2e, dt), dt, f"k3 dh e{e}")
        assert_close_rows(dgu_e, O.store(B.glu_backward(a_e @ W1e.T, dh_e, cfg.beta1, cfg.beta2), dt), dt, f"k3 dgu e{e}")
        assert_close_rows(host(g["dx_perm"][rr]), O.store(dgu_e @ W1e, dt), dt, f"k3 dx_perm e{e}")
        assert_f32(host(g["dW2"][int(e)]), dy_e.T @ h_e, f"k3 dW2 e{e}")
        assert_f32(host(g["dW1"][int(e)]), dgu_e.T @ a_e, f"k3 dW1 e{e}")
        xe = O.to_f64(inp["x"][st[r0:r1]], dt)
        assert_f32(host(g["dW_r"][int(e)]), dl_sorted[r0:r1] @ xe, f"k3 dW_r e{e}")
        say(f"[k3 bwd] expert {e} ({r1 - r0} rows) ok")
    # un-permutation, down-projection, shared experts and dx on the sampled tokens
    dxp = host(g["dx_perm"][torch.as_tensor(slot[toks].reshape(-1), device="cuda")]).reshape(len(toks), k, L)
    assert_close_rows(host(g["dx_lat"][tt]), O.store(dxp.sum(axis=1), dt), dt, "k3 dx_lat")
    W1s = f64(inp["w1s"])
    W1s_p = np.concatenate([W1s[:, :Is].reshape(Ss, -1), W1s[:, Is:].reshape(Ss, -1)], axis=0)
    dhs = host(g["dh_s"][tt])[:, :Ss]
    assert_close_rows(host(g["dgu_s"][tt])[:, : 2 * Ss],
                      O.store(B.glu_backward(xh @ W1s_p.T, dhs, cfg.beta1, cfg.beta2), dt), dt, "k3 dgu_s")
    _, dx_r = B.router_backward(host(g["dl"])[toks], idx[toks], xh, inp["w_router"])
    dx_ref = dx_r + host(g["dx_lat"][tt]) @ f64(inp["w_down"]) + host(g["dgu_s"][tt])[:, : 2 * Ss] @ W1s_p
    assert_f32(host(g["dx"][tt]), dx_ref, "k3 dx")
    lrows = rng.choice(L, 3, replace=False)
    x_all = O.to_f64(inp["x"], dt)
    assert_f32(host(g["dW_dn"][torch.as_tensor(lrows, device="cuda")]), host(g["dx_lat"])[:, lrows].T @ x_all,
               "k3 dW_dn rows")
    say("[k3 bwd] down-projection, shared experts and dx ok")
