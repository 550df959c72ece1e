"""CPU oracle for the Stable LatentMoE layer forward pass.

TEST INFRASTRUCTURE ONLY. This module exists to check the GPU library. Only the test suite, the
package's smoke check and the benchmark's CPU-baseline leg may import it; the product path never
does, and it shares no code with the GPU kernels (it imports NumPy and nothing else).

It is deliberately plain: float64 matrix products through NumPy, explicit loops over experts, and
rounding to the storage type (bfloat16 or float32) only at the points where the layer stores a
tensor. Pages cited (by site and section):

  [vxz]   vxz.us, "苏神复盘 Kimi K3：896 个专家背后，藏着哪些关键技术取舍？"
          sections "01 LatentMoE 如何重新分配专家预算" and "02 Stable LatentMoE 如何处理数值与负载风险".
  [tahou] tahou.com K3 architecture write-up, sections "SiTU激活优化", "归一化策略调整",
          "负载均衡优化".
  [slm]   lukebest.github.io "Stable Latent MoE", sections "K3 专家配置", "路由机制",
          "Quantile Balancing", "Latent-Space MoE", "SiTU 激活".

Readings taken where the pages are silent (each also listed in the design notes):
  R1 router: sigmoid of x . W_r^T on d_model, fp32 scores (the scores must lie in 0..1 for the
     binning of [tahou] "负载均衡优化"); the logits are formed in float64 and sigma rounded once.
  R2 the balancing bias is added to the scores for selection only; combine weights use the
     unbiased scores normalised over the selected k ([vxz] 02: traffic is steered by a per-expert
     selection bias). No extra routed scaling factor ([tahou] "归一化策略调整").
  R3 top-k order: descending biased score, ties to the lower expert index.
  R4 the quantity that is binned is the leave-one-out margin m = s_hat(t,e) - theta(t,-e), with
     theta the k-th largest biased score when e is not selected and the (k+1)-th when it is.
  R5 "compress to 0..1": u = clamp((m + 1) / 2, 0, 1), bin = min(NB - 1, floor(u * NB)), each
     step one float32 operation in that order (m = s_hat - theta; m + 1; times 0.5; times NB).
  R6 target load per expert is N*k/E tokens, so the quantile level is 1 - k/E; the quantile is
     read from the cumulative histogram with linear interpolation inside the bin, in float64; the
     bias then jumps by minus that margin quantile (no step size). Histograms add across
     micro-batches ([tahou] "负载均衡优化") until an update resets them.
  R7 expert FFN in latent space: W1_e [2I, L] with gate rows first then up rows, W2_e [L, I];
     one layer-level W_up [D, L] after combine and RMSNorm.
  R8 SiTU-GLU in float64 on unrounded projections; h rounded to the storage type.
  R9 RMSNorm over d_latent with eps = 1e-6 and gain gamma, after the weighted combine and before
     the up-projection ([vxz] 02, [tahou] "归一化策略调整").
  R10 shared experts are SiTU-GLU FFNs on d_model, added to the up-projected output unscaled; their
     summed output is kept in float32.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64


# ----------------------------------------------------------------------------------------------
# storage types
# ----------------------------------------------------------------------------------------------
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) to their exact float64 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32).astype(F64)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), returned as float64.

    Done in one step from float64 (no intermediate float32 rounding): with a = m * 2**e and
    0.5 <= |m| < 1, bfloat16 keeps 8 significant bits, so the value is rint(m * 2**8) * 2**(e - 8),
    with rint rounding half to even. Subnormal bfloat16 values have the fixed spacing 2**-133.
    """
    a = np.asarray(a, dtype=F64)
    m, e = np.frexp(a)
    e = np.maximum(e, -125)                      # below the normal range the spacing stays 2**-133
    q = np.ldexp(1.0, e - 8)
    r = np.rint(a / q) * q
    big = np.abs(r) >= 2.0 ** 128
    return np.where(big, np.copysign(np.inf, a), r)


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """An input tensor in its storage format (uint16 bits for bf16, float32) as float64 values."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=F32).astype(F64)


def store(a: np.ndarray, dtype: str) -> np.ndarray:
    """The value a tensor holds once stored in ``dtype`` ("bf16" or "f32"), as float64."""
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return np.asarray(a, dtype=F64).astype(F32).astype(F64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------------------------
# elementwise functions
# ----------------------------------------------------------------------------------------------
def sigmoid(a: np.ndarray) -> np.ndarray:
    """Logistic function in float64, written through exp(-|a|) so it never overflows."""
    a = np.asarray(a, dtype=F64)
    z = np.exp(-np.abs(a))
    return np.where(a >= 0, 1.0 / (1.0 + z), z / (1.0 + z))


def situ(g: np.ndarray, beta: float) -> np.ndarray:
    """SiTU gate activation beta * tanh(g / beta) * sigmoid(g) ([tahou] "SiTU激活优化"; [slm]
    "SiTU 激活" and its SiLU/SiTU table). Bounded by beta; tends to SiLU as beta grows."""
    g = np.asarray(g, dtype=F64)
    return beta * np.tanh(g / beta) * sigmoid(g)


def softcap(u: np.ndarray, beta: float) -> np.ndarray:
    """Soft cap of the linear (up) branch, beta * tanh(u / beta) ([tahou] "SiTU激活优化")."""
    u = np.asarray(u, dtype=F64)
    return beta * np.tanh(u / beta)


# ----------------------------------------------------------------------------------------------
# routing (R1-R3)
# ----------------------------------------------------------------------------------------------
def router_scores(x: np.ndarray, w_router: np.ndarray, logit_offset: np.ndarray | None = None) -> np.ndarray:
    """s = sigmoid(x . W_r^T (+ o)) as float32 [T, E]; x given as float64 values, W_r float32.

    [slm] "路由机制" describes a router over x followed by top-K; R1 fixes sigmoid and fp32.
    """
    logits = np.asarray(x, dtype=F64) @ np.asarray(w_router, dtype=F32).astype(F64).T
    if logit_offset is not None:
        logits = logits + np.asarray(logit_offset, dtype=F32).astype(F64)[None, :]
    return sigmoid(logits).astype(F32)


def biased_scores(s: np.ndarray, bias: np.ndarray) -> np.ndarray:
    """s_hat = s + b, one float32 addition per element ([vxz] 02: per-expert selection bias)."""
    return (np.asarray(s, dtype=F32) + np.asarray(bias, dtype=F32)[None, :]).astype(F32)


def select_topk(s: np.ndarray, bias: np.ndarray, k: int):
    """Top-k by biased score (R3), plus the normalised unbiased combine weights (R2).

    Returns idx [T, k] int32 in rank order, w [T, k] float32, thresh [T, 2] float32 holding the
    k-th and (k+1)-th largest biased scores of each row.
    """
    s = np.asarray(s, dtype=F32)
    E = s.shape[1]
    if not 0 < k < E:
        raise ValueError("need 0 < k < E")
    sh = biased_scores(s, bias)
    order = np.argsort(-sh, axis=1, kind="stable")        # descending; equal values keep index order
    idx = order[:, :k].astype(np.int32)
    rows = np.arange(s.shape[0])
    thresh = np.stack([sh[rows, order[:, k - 1]], sh[rows, order[:, k]]], axis=1).astype(F32)
    sel = np.take_along_axis(s, idx, axis=1).astype(F64)
    w = (sel / sel.sum(axis=1, keepdims=True)).astype(F32)
    return idx, w, thresh


# ----------------------------------------------------------------------------------------------
# quantile balancing (R4-R6)
# ----------------------------------------------------------------------------------------------
def qb_margins(s: np.ndarray, bias: np.ndarray, idx: np.ndarray, thresh: np.ndarray) -> np.ndarray:
    """Leave-one-out margin of every (token, expert) pair against the top-k threshold (R4), fp32.

    [vxz] 02 and [slm] "Quantile Balancing": the balancer looks at where router scores fall
    relative to the top-k threshold, per expert.
    """
    sh = biased_scores(s, bias)
    T, E = sh.shape
    selected = np.zeros((T, E), dtype=bool)
    selected[np.arange(T)[:, None], np.asarray(idx)] = True
    theta = np.where(selected, thresh[:, 1:2], thresh[:, 0:1]).astype(F32)
    return (sh - theta).astype(F32)


def qb_bins(m: np.ndarray, n_bins: int) -> np.ndarray:
    """Bin of each margin after mapping it to 0..1 (R5; [tahou] "负载均衡优化"), float32 steps."""
    m = np.asarray(m, dtype=F32)
    u = ((m + F32(1.0)).astype(F32) * F32(0.5)).astype(F32)
    u = np.clip(u, F32(0.0), F32(1.0))
    b = np.floor((u * F32(n_bins)).astype(F32)).astype(np.int64)
    return np.minimum(b, n_bins - 1).astype(np.int32)


def qb_histogram(s, bias, idx, thresh, n_bins: int, hist: np.ndarray | None = None) -> np.ndarray:
    """Per-expert histogram of margin bins [E, NB] uint32, added into ``hist`` when given."""
    bins = qb_bins(qb_margins(s, bias, idx, thresh), n_bins)
    T, E = bins.shape
    h = np.zeros((E, n_bins), dtype=np.uint64)
    for e in range(E):
        h[e] = np.bincount(bins[:, e], minlength=n_bins)
    if hist is not None:
        h += np.asarray(hist, dtype=np.uint64)
    return h.astype(np.uint32)


def qb_quantile_margins(hist: np.ndarray, n_acc: int, k: int) -> np.ndarray:
    """Margin quantile of every expert at level 1 - k/E, read from its histogram (R6), float64.

    c* = (E - k) * N / E tokens must fall below the quantile; j* is the first bin whose cumulative
    count reaches c*; inside j* the count is interpolated linearly. The bin coordinate u is mapped
    back to a margin by m = 2u - 1 (inverse of R5).
    """
    hist = np.asarray(hist, dtype=np.int64)
    E, NB = hist.shape
    c_star = float((E - k) * int(n_acc)) / float(E)
    out = np.empty(E, dtype=F64)
    for e in range(E):
        cum = np.cumsum(hist[e])
        j = int(np.argmax(cum >= c_star))
        prev = float(cum[j - 1]) if j > 0 else 0.0
        frac = (c_star - prev) / float(hist[e, j])
        u_hat = (float(j) + frac) / float(NB)
        out[e] = 2.0 * u_hat - 1.0
    return out


def qb_update(hist: np.ndarray, n_acc: int, bias: np.ndarray, k: int):
    """Bias update at a step boundary: b_e <- b_e - m_hat_e, in float64 then rounded to float32.

    [vxz] 02: the balancer solves for where each expert's threshold must move to receive its
    target token count instead of stepping by a fixed amount. Returns (new bias, zeroed histogram).
    With no accumulated tokens the bias is left as it is.
    """
    hist = np.asarray(hist)
    bias = np.asarray(bias, dtype=F32)
    if n_acc <= 0:
        return bias.copy(), np.zeros_like(hist, dtype=np.uint32)
    m_hat = qb_quantile_margins(hist, n_acc, k)
    new_bias = (bias.astype(F64) - m_hat).astype(F32)
    return new_bias, np.zeros_like(hist, dtype=np.uint32)


# ----------------------------------------------------------------------------------------------
# latent projection, permutation, experts, combine (R7-R10)
# ----------------------------------------------------------------------------------------------
def down_project(x: np.ndarray, w_down: np.ndarray, dtype: str) -> np.ndarray:
    """x_lat = x . W_dn^T, stored ([vxz] 01: tokens are compressed to d_latent before routing to
    experts; [slm] "Latent-Space MoE")."""
    return store(np.asarray(x, F64) @ np.asarray(w_down, F64).T, dtype)


def permute(idx: np.ndarray, n_experts: int):
    """Counting sort of (token, slot) pairs by expert, tokens ascending inside each expert.

    Returns offsets [E+1], sorted_token [T*k] (token of each sorted row), slot_of_pair [T*k]
    (sorted row of pair t*k + j).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=n_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    order = np.argsort(flat, kind="stable")               # pairs are in (t, j) order already
    slot_of_pair = np.empty(T * k, dtype=np.int32)
    slot_of_pair[order] = np.arange(T * k, dtype=np.int32)
    sorted_token = (order // k).astype(np.int32)
    return offsets, sorted_token, slot_of_pair


def situ_glu_ffn(a: np.ndarray, w1: np.ndarray, w2: np.ndarray, beta1: float, beta2: float, dtype: str):
    """One SiTU-GLU expert on rows a (float64 values of stored inputs).

    [g | u] = a . W1^T (gate = first half of the projection, up = second half, [slm] "SiTU 激活");
    h = SiTU_beta1(g) * softcap_beta2(u), stored; y = h . W2^T, stored.
    """
    a = np.asarray(a, F64)
    w1 = np.asarray(w1, F64)
    inter = w1.shape[0] // 2
    gu = a @ w1.T
    h = store(situ(gu[:, :inter], beta1) * softcap(gu[:, inter:], beta2), dtype)
    y = store(h @ np.asarray(w2, F64).T, dtype)
    return h, y


def combine(y_rows_per_pair: np.ndarray, w: np.ndarray) -> np.ndarray:
    """z_t = sum_j w[t, j] * y(t, j) in float64; y_rows_per_pair is [T, k, L]."""
    return np.einsum("tk,tkl->tl", np.asarray(w, F32).astype(F64), np.asarray(y_rows_per_pair, F64))


def rms_norm(z: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """gamma * z / sqrt(mean(z^2) + eps) over the last axis, float64 (R9)."""
    z = np.asarray(z, F64)
    ms = np.mean(z * z, axis=-1, keepdims=True)
    return np.asarray(gamma, F32).astype(F64)[None, :] * z / np.sqrt(ms + eps)


def shared_experts(x: np.ndarray, w1s: np.ndarray, w2s: np.ndarray, beta1: float, beta2: float, dtype: str):
    """Sum of the always-on shared SiTU-GLU experts on d_model (R10; [vxz] 01, [slm] expert table).

    Returns (h_s [T, S*I_s] stored, y_sh [T, D] float32-stored).
    """
    hs, acc = [], None
    for j in range(np.asarray(w1s).shape[0]):
        w1 = np.asarray(w1s[j], F64)
        inter = w1.shape[0] // 2
        gu = np.asarray(x, F64) @ w1.T
        h = store(situ(gu[:, :inter], beta1) * softcap(gu[:, inter:], beta2), dtype)
        y = h @ np.asarray(w2s[j], F64).T
        hs.append(h)
        acc = y if acc is None else acc + y
    return np.concatenate(hs, axis=1), store(acc, "f32")


def up_project(n: np.ndarray, w_up: np.ndarray, y_shared: np.ndarray | None, dtype: str):
    """out = n . W_up^T + y_sh; returns (value before the final rounding, stored value)."""
    pre = np.asarray(n, F64) @ np.asarray(w_up, F64).T
    if y_shared is not None:
        pre = pre + np.asarray(y_shared, F64)
    return pre, store(pre, dtype)


# ----------------------------------------------------------------------------------------------
# whole layer
# ----------------------------------------------------------------------------------------------
def _f64_inputs(inp: dict, dt: str) -> dict:
    return {
        "x": to_f64(inp["x"], dt),
        "w_down": to_f64(inp["w_down"], dt),
        "w_up": to_f64(inp["w_up"], dt),
        "w1s": to_f64(inp["w1s"], dt),
        "w2s": to_f64(inp["w2s"], dt),
    }


def route(inp: dict, cfg, bias: np.ndarray | None = None):
    """Routing of all tokens: scores, top-k, weights, thresholds."""
    x = to_f64(inp["x"], cfg.act_dtype)
    b = inp["bias"] if bias is None else bias
    s = router_scores(x, inp["w_router"], inp.get("logit_offset"))
    idx, w, thresh = select_topk(s, b, cfg.top_k)
    return s, idx, w, thresh


def expert_path(inp: dict, cfg, idx: np.ndarray, w: np.ndarray, tokens: np.ndarray | None = None) -> dict:
    """Everything after routing for the given tokens (all when None), with the routing given.

    The layer is independent per token once the routing is fixed, so a token subset is evaluated
    exactly as in the full pass: x_lat rows, each selected expert's FFN on the row, the weighted
    combine, RMSNorm, the up-projection and the shared experts.
    """
    dt = cfg.act_dtype
    T = np.asarray(inp["x"]).shape[0]
    tok = np.arange(T) if tokens is None else np.asarray(tokens)
    x = to_f64(np.asarray(inp["x"])[tok], dt)
    x_lat = down_project(x, to_f64(inp["w_down"], dt), dt)
    sel = np.asarray(idx)[tok]
    n, k = sel.shape
    L = x_lat.shape[1]
    y_pair = np.zeros((n, k, L), dtype=F64)
    h_pair = np.zeros((n, k, cfg.inter), dtype=F64)
    for e in np.unique(sel):
        rr, jj = np.nonzero(sel == e)
        h, y = situ_glu_ffn(x_lat[rr], to_f64(inp["w1"][e], dt), to_f64(inp["w2"][e], dt),
                            cfg.beta1, cfg.beta2, dt)
        y_pair[rr, jj] = y
        h_pair[rr, jj] = h
    z = combine(y_pair, np.asarray(w)[tok])
    nrm = store(rms_norm(z, inp["gamma"], cfg.rms_eps), dt)
    h_s, y_sh = shared_experts(x, to_f64(inp["w1s"], dt), to_f64(inp["w2s"], dt), cfg.beta1, cfg.beta2, dt)
    out_pre, out = up_project(nrm, to_f64(inp["w_up"], dt), y_sh, dt)
    return {"tokens": tok, "x_lat": x_lat, "h_pair": h_pair, "y_pair": y_pair, "z": z, "n": nrm,
            "h_s": h_s, "y_sh": y_sh, "out_pre": out_pre, "out": out}


def forward(inp: dict, cfg, bias: np.ndarray | None = None, hist: np.ndarray | None = None) -> dict:
    """The full layer forward on every token, with the intermediate tensors in the GPU's layouts.

    ``cfg`` needs the attributes top_k, n_experts, n_bins, inter, beta1, beta2, rms_eps, act_dtype.
    """
    b = inp["bias"] if bias is None else bias
    s, idx, w, thresh = route(inp, cfg, b)
    H = qb_histogram(s, b, idx, thresh, cfg.n_bins, hist)
    offsets, sorted_token, slot_of_pair = permute(idx, cfg.n_experts)
    ex = expert_path(inp, cfg, idx, w)
    T, k = idx.shape
    flat_y = ex["y_pair"].reshape(T * k, -1)
    flat_h = ex["h_pair"].reshape(T * k, -1)
    order = np.empty(T * k, dtype=np.int64)
    order[slot_of_pair] = np.arange(T * k)
    return {"s": s, "idx": idx, "w": w, "thresh": thresh, "hist": H, "offsets": offsets,
            "sorted_token": sorted_token, "slot_of_pair": slot_of_pair,
            "x_lat": ex["x_lat"], "x_perm": ex["x_lat"][sorted_token],
            "h": flat_h[order], "y": flat_y[order], "z": ex["z"], "n": ex["n"], "h_s": ex["h_s"],
            "y_sh": ex["y_sh"], "out_pre": ex["out_pre"], "out": ex["out"]}


def dense_masked_forward(inp: dict, cfg, w_dense: np.ndarray) -> np.ndarray:
    """Reference evaluation without routing: every expert on every token, weighted by w_dense
    [T, E] (zero for unselected experts), then RMSNorm, up-projection and shared experts.
    Returns the value before the final rounding."""
    dt = cfg.act_dtype
    x = to_f64(inp["x"], dt)
    x_lat = down_project(x, to_f64(inp["w_down"], dt), dt)
    z = np.zeros_like(x_lat)
    for e in range(np.asarray(inp["w1"]).shape[0]):
        _, y = situ_glu_ffn(x_lat, to_f64(inp["w1"][e], dt), to_f64(inp["w2"][e], dt), cfg.beta1, cfg.beta2, dt)
        z += np.asarray(w_dense[:, e], F32).astype(F64)[:, None] * y
    nrm = store(rms_norm(z, inp["gamma"], cfg.rms_eps), dt)
    _, y_sh = shared_experts(x, to_f64(inp["w1s"], dt), to_f64(inp["w2s"], dt), cfg.beta1, cfg.beta2, dt)
    pre, _ = up_project(nrm, to_f64(inp["w_up"], dt), y_sh, dt)
    return pre


def expert_flops_per_token(d_in: int, inter: int, k: int) -> int:
    """Multiply-add FLOPs of k SiTU-GLU experts of inner size ``inter`` acting on a d_in vector."""
    return k * (2 * d_in * 2 * inter + 2 * inter * d_in)
