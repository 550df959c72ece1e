"""CPU oracle for the backward pass of the Stable LatentMoE layer.

TEST INFRASTRUCTURE ONLY, like lmoe_oracle (whose forward it differentiates): only the test suite,
the package's smoke check and the benchmark's CPU-baseline leg may import it. NumPy only; it shares
no code with the GPU kernels.

What is differentiated is the forward of lmoe_oracle: the layer of [vxz] 01-02 and [slm]
"Latent-Space MoE" (down-projection to d_latent, routed SiTU-GLU experts in the latent space,
router-weighted combine, RMSNorm, up-projection, always-on shared experts). The pages train this
layer but print no backward pass; the gradients below are the chain rule applied to that forward,
written out step by step in float64, with rounding to the storage type at the points where the
GPU stores a tensor:

  RB1 the output gradient dout [T, D] arrives in the activation type; the gradients of every
      stored activation (dn, dh_s, dy, dh, d[g|u], dx_perm, dx_lat, d[g_s|u_s]) are stored in the
      activation type; weight gradients, dgamma, the router-logit gradient and dx are float32.
  RB2 the quantile-balancing bias only selects experts ([vxz] 02): it has no gradient, and the
      selection (top-k indices) is held fixed. The combine weights w = s / sum(s over the selected
      experts) are differentiated through the unbiased sigmoid scores s; unselected scores get no
      gradient.
  RB3 the SiTU-GLU of an expert is recomputed from its stored input rows (the projections g and u
      are not kept by the forward pass); the derivatives are
        d/dg [b1 tanh(g/b1) sigmoid(g)] = (1 - tanh^2(g/b1)) sigmoid(g) + b1 tanh(g/b1) sigmoid(g) (1 - sigmoid(g))
        d/du [b2 tanh(u/b2)]            = 1 - tanh^2(u/b2)
  RB4 RMSNorm n = gamma * z * r, r = (mean(z^2) + eps)^(-1/2):
        dz = r * (gamma dn) - (r^3 / L) * sum(gamma dn z) * z,   dgamma = sum_t dn z r
      with z recomputed from the stored expert outputs and combine weights (float64 here).
  RB5 the shared experts are differentiated in their packed form (one FFN of inner size S*I_s:
      all gate rows, then all up rows; the down block [D, S*I_s]); the weight gradients are
      returned in that packed layout.
  RB6 dx sums the router, down-projection and shared-expert contributions.
"""
from __future__ import annotations

import numpy as np

from .lmoe_oracle import F32, F64, sigmoid, situ, softcap, store, to_f64


def keep(a: np.ndarray, dtype: str) -> np.ndarray:
    """Value after storing in ``dtype``; "f64" keeps every bit (for finite-difference checks)."""
    if dtype == "f64":
        return np.asarray(a, dtype=F64)
    return store(a, dtype)


def inputs_f64(a, dtype: str) -> np.ndarray:
    if dtype == "f64":
        return np.asarray(a, dtype=F64)
    return to_f64(a, dtype)


# ----------------------------------------------------------------------------------------------
# elementwise derivatives (RB3)
# ----------------------------------------------------------------------------------------------
def situ_grad(g: np.ndarray, beta: float) -> np.ndarray:
    """Derivative of the SiTU gate beta * tanh(g / beta) * sigmoid(g) ([tahou] "SiTU激活优化")."""
    g = np.asarray(g, F64)
    t = np.tanh(g / beta)
    s = sigmoid(g)
    return (1.0 - t * t) * s + beta * t * s * (1.0 - s)


def softcap_grad(u: np.ndarray, beta: float) -> np.ndarray:
    """Derivative of the soft cap beta * tanh(u / beta)."""
    t = np.tanh(np.asarray(u, F64) / beta)
    return 1.0 - t * t


def glu_backward(gu: np.ndarray, dh: np.ndarray, beta1: float, beta2: float) -> np.ndarray:
    """d[g | u] of h = SiTU(g) * cap(u), given the unrounded projections gu = [g | u]."""
    gu = np.asarray(gu, F64)
    inter = gu.shape[1] // 2
    g, u = gu[:, :inter], gu[:, inter:]
    dh = np.asarray(dh, F64)
    dg = dh * softcap(u, beta2) * situ_grad(g, beta1)
    du = dh * situ(g, beta1) * softcap_grad(u, beta2)
    return np.concatenate([dg, du], axis=1)


# ----------------------------------------------------------------------------------------------
# combine, norm and routing weights (RB2, RB4)
# ----------------------------------------------------------------------------------------------
def rms_norm_backward(z: np.ndarray, gamma: np.ndarray, dn: np.ndarray, eps: float):
    """Returns (dz [T, L], dgamma [L]) of n = gamma * z / sqrt(mean(z^2) + eps)."""
    z = np.asarray(z, F64)
    L = z.shape[1]
    r = 1.0 / np.sqrt(np.mean(z * z, axis=1, keepdims=True) + eps)
    a = np.asarray(gamma, F64)[None, :] * np.asarray(dn, F64)
    dz = r * a - (r ** 3 / L) * np.sum(a * z, axis=1, keepdims=True) * z
    dgamma = np.sum(np.asarray(dn, F64) * z * r, axis=0)
    return dz, dgamma


def combine_backward(dz: np.ndarray, y_pair: np.ndarray, w: np.ndarray):
    """z_t = sum_j w_tj y_tj: returns (dw [T, k], dy_pair [T, k, L])."""
    dz = np.asarray(dz, F64)
    y_pair = np.asarray(y_pair, F64)
    w = np.asarray(w, F64)
    dw = np.einsum("tl,tkl->tk", dz, y_pair)
    dy_pair = w[:, :, None] * dz[:, None, :]
    return dw, dy_pair


def weights_backward(dw: np.ndarray, s_sel: np.ndarray) -> np.ndarray:
    """w_j = s_j / S over the selected scores, s = sigmoid(l): returns dl [T, k] for the selected
    experts' logits (w recomputed here in float64 from the selected scores)."""
    s_sel = np.asarray(s_sel, F64)
    S = s_sel.sum(axis=1, keepdims=True)
    w = s_sel / S
    ds = (np.asarray(dw, F64) - np.sum(w * dw, axis=1, keepdims=True)) / S
    return ds * s_sel * (1.0 - s_sel)


def router_backward(dl: np.ndarray, idx: np.ndarray, x: np.ndarray, w_router: np.ndarray):
    """l = x . W_r^T (+ offset): returns (dW_r [E, D], dx_r [T, D]) with dl nonzero only at the
    selected experts."""
    dl = np.asarray(dl, F64)
    x = np.asarray(x, F64)
    w_router = np.asarray(w_router, F64)
    idx = np.asarray(idx)
    E = w_router.shape[0]
    dW = np.zeros((E, x.shape[1]), F64)
    for e in np.unique(idx):
        tt, jj = np.nonzero(idx == e)
        dW[e] = dl[tt, jj] @ x[tt]
    dx = np.einsum("tk,tkd->td", dl, w_router[idx])
    return dW, dx


# ----------------------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------------------
def backward(inp: dict, cfg, fwd: dict, dout, dtype: str | None = None) -> dict:
    """Gradients of <dout, out> with respect to x and every weight, given the forward tensors.

    ``fwd`` holds the forward's stored tensors in the GPU's layouts (as returned by
    lmoe_oracle.forward: s, idx, w, offsets, sorted_token, slot_of_pair, x_lat, h, y, n, h_s).
    ``dtype`` overrides cfg.act_dtype for the storage points ("f64": no rounding anywhere); the
    inputs are read in cfg.act_dtype ("f64": plain float values).
    """
    dt = cfg.act_dtype if dtype is None else dtype
    din = cfg.act_dtype                                   # how the inputs are given ("f64": as values)
    b1, b2 = cfg.beta1, cfg.beta2
    x = inputs_f64(inp["x"], din)
    w_router = np.asarray(inp["w_router"], F64)
    w_down = inputs_f64(inp["w_down"], din)
    w_up = inputs_f64(inp["w_up"], din)
    w1 = inputs_f64(inp["w1"], din)
    w2 = inputs_f64(inp["w2"], din)
    w1s = inputs_f64(inp["w1s"], din)
    w2s = inputs_f64(inp["w2s"], din)
    gamma = np.asarray(inp["gamma"], F64)
    S, Is = w1s.shape[0], w1s.shape[1] // 2
    w1s_p = np.concatenate([w1s[:, :Is].reshape(S * Is, -1), w1s[:, Is:].reshape(S * Is, -1)], axis=0)
    w2s_p = np.concatenate(list(w2s), axis=1)                       # [D, S*Is]
    dout = keep(np.asarray(dout, F64), dt)

    idx = np.asarray(fwd["idx"])
    T, k = idx.shape
    slot = np.asarray(fwd["slot_of_pair"]).reshape(T, k)
    offsets = np.asarray(fwd["offsets"])
    sorted_token = np.asarray(fwd["sorted_token"])
    x_lat = np.asarray(fwd["x_lat"], F64)
    h = np.asarray(fwd["h"], F64)
    y = np.asarray(fwd["y"], F64)
    n = np.asarray(fwd["n"], F64)
    h_s = np.asarray(fwd["h_s"], F64)
    w = np.asarray(fwd["w"], F64)
    s_sel = np.take_along_axis(np.asarray(fwd["s"], F64), idx.astype(np.int64), axis=1)
    L = x_lat.shape[1]

    # A11 + shared down-projection: out = [n | h_s] . [W_up | W2s]^T
    dn = keep(dout @ w_up, dt)
    dh_s = keep(dout @ w2s_p, dt)
    dW_up = keep(dout.T @ n, "f32" if dt != "f64" else "f64")
    dW2s_p = keep(dout.T @ h_s, "f32" if dt != "f64" else "f64")

    # A9: combine and RMSNorm (z recomputed from the stored expert outputs)
    y_pair = y[slot.reshape(-1)].reshape(T, k, L)
    z = np.einsum("tk,tkl->tl", w, y_pair)
    dz, dgamma = rms_norm_backward(z, gamma, dn, cfg.rms_eps)
    dw, dy_pair = combine_backward(dz, y_pair, w)
    dy = np.empty_like(y)
    dy[slot.reshape(-1)] = keep(dy_pair.reshape(T * k, L), dt)

    # A1/A2: routing weights and router
    dl = weights_backward(dw, s_sel)
    dW_r, dx_r = router_backward(dl, idx, x, w_router)

    # A7/A8: routed experts, rows in expert-sorted order
    I = w1.shape[1] // 2
    dh = np.zeros((T * k, I), F64)
    dgu = np.zeros((T * k, 2 * I), F64)
    dx_perm = np.zeros((T * k, L), F64)
    dW1 = np.zeros_like(w1)
    dW2 = np.zeros_like(w2)
    wgt = "f32" if dt != "f64" else "f64"
    for e in range(w1.shape[0]):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        a_e = x_lat[sorted_token[r0:r1]]
        dy_e = dy[r0:r1]
        dh_e = keep(dy_e @ w2[e], dt)
        dW2[e] = dy_e.T @ h[r0:r1]
        gu = a_e @ w1[e].T
        dgu_e = keep(glu_backward(gu, dh_e, b1, b2), dt)
        dx_perm[r0:r1] = keep(dgu_e @ w1[e], dt)
        dW1[e] = dgu_e.T @ a_e
        dh[r0:r1] = dh_e
        dgu[r0:r1] = dgu_e
    dW1 = keep(dW1, wgt)
    dW2 = keep(dW2, wgt)

    # A6/A5: un-permute (sum of a token's k rows) and down-projection
    dx_lat = keep(dx_perm[slot.reshape(-1)].reshape(T, k, L).sum(axis=1), dt)
    dW_dn = keep(dx_lat.T @ x, wgt)
    dx_down = dx_lat @ w_down

    # A10: shared experts (packed)
    gu_s = x @ w1s_p.T
    dgu_s = keep(glu_backward(gu_s, dh_s, b1, b2), dt)
    dW1s_p = keep(dgu_s.T @ x, wgt)
    dx_s = dgu_s @ w1s_p

    dx = keep(dx_r + dx_down + dx_s, wgt)
    return {"dn": dn, "dh_s": dh_s, "dW_up": dW_up, "dW2s_packed": dW2s_p, "z": z, "dz": dz,
            "dgamma": keep(dgamma, wgt), "dw": dw, "dl": keep(dl, wgt), "dy": dy, "dW_r": keep(dW_r, wgt),
            "dx_r": dx_r, "dh": dh, "dgu": dgu, "dx_perm": dx_perm, "dW1": dW1, "dW2": dW2,
            "dx_lat": dx_lat, "dW_dn": dW_dn, "dgu_s": dgu_s, "dW1s_packed": dW1s_p, "dx": dx}
