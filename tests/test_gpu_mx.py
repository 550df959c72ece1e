"""GPU parity of the MX-format calls against the MX oracle (OCP MXFP4 / MXFP8).

Quantisation is integer output (element codes and E8M0 scale bytes), so it is compared bit for
bit with the oracle's codes on the same inputs: random rows mixed with blocks built to hit every
rounding decision (exact ties between neighbouring codes, saturation, subnormal elements, all-zero
and signed-zero blocks, float32 extremes).

The routed experts on MX operands are compared stage by stage: the layer's weight and x_lat codes
bit for bit, h against the oracle's first projection fed the GPU's x_lat, y against the second
fed the GPU's h (one bf16 rounding plus f32 accumulation noise). Cases: a ragged token count, a
batch where most experts get no tokens, and sampled experts and rows at the K3 prefill shape.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_space_routed_amd import LatentMoE, to_device, upload_weights
from latent_space_routed_amd import _lib as C
from oracle import lmoe_oracle as O
from oracle import lmoe_oracle_mx as M
from workloads import CONFIGS
from workloads.inputs import make_inputs

from .gpu_helpers import assert_close_rows, host, say

pytestmark = pytest.mark.gpu


def special_rows(fmt: str, K: int, dtype: str, rng) -> np.ndarray:
    """Rows whose blocks exercise the rounding rules after the shared scale is applied."""
    mags = M.FORMATS[fmt][0]
    emax = M.FORMATS[fmt][2]
    rows = []
    nb = K // 32
    for scale_exp in (-20, 0, 7):
        r = np.zeros(K)
        for b in range(nb):
            X = 2.0 ** (scale_exp + b % 5 - 2)
            blk = np.zeros(32)
            blk[0] = 1.5 * 2.0 ** emax * X            # sets the shared exponent to scale_exp + ...
            kind = b % 4
            if kind == 0:    # midpoints between neighbouring magnitudes: ties to the even code
                mids = (mags[:-1] + mags[1:]) / 2
                blk[1:] = np.resize(mids, 31) * X * np.where(np.arange(31) % 2, -1, 1)
            elif kind == 1:  # just above / below the midpoints
                mids = (mags[:-1] + mags[1:]) / 2
                eps = np.resize([1 + 2 ** -6, 1 - 2 ** -6], 31)
                blk[1:] = np.resize(mids, 31) * eps * X
            elif kind == 2:  # saturation: magnitudes in [max normal, 2^(emax+1))
                blk[1:] = rng.uniform(mags[-1], 2.0 ** (emax + 1) * 0.999, 31) * X * rng.choice([-1, 1], 31)
            else:            # small elements, down into the format's subnormals and to zero
                blk[1:] = rng.standard_normal(31) * 2.0 ** rng.integers(-12, 0, 31) * X
                blk[5] = 0.0
                blk[6] = -0.0
            r[32 * b:32 * b + 32] = blk
        rows.append(r)
    zero = np.zeros(K)
    zero[::7] = -0.0
    rows.append(zero)
    if dtype == "f32":  # extremes of float32: largest finite amax, subnormal blocks
        big = rng.uniform(-3e38, 3e38, K)
        big[0] = 3.4e38
        tiny = rng.standard_normal(K) * 2.0 ** -140
        rows += [big, tiny]
    return np.stack(rows)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("fmt", ["fp4", "fp8"])
def test_mx_quantize_bit_exact(fmt, dtype):
    cfg = CONFIGS["tiny_f32"] if dtype == "f32" else CONFIGS["mid_bf16"]
    rng = np.random.default_rng(5)
    K = 1024
    rand = rng.standard_normal((300, K)) * np.exp(rng.uniform(-4, 4, (300, 1)))
    x = np.concatenate([rand, special_rows(fmt, K, dtype, rng)])
    rows = x.shape[0]
    xs = O.store(x, dtype)                            # the values the GPU holds
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xd = torch.as_tensor(xs, dtype=torch.float64).to(tdt).cuda()
    assert np.array_equal(xd.double().cpu().numpy(), xs)
    per = K // 2 if fmt == "fp4" else K
    codes = torch.empty(rows, per, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, K // 32, dtype=torch.uint8, device="cuda")
    shape = C.make_shape(cfg, rows)
    say(f"mx_quantize fmt={fmt} dtype={dtype} rows={rows} K={K}")
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP4 if fmt == "fp4" else C.LMOE_MX_FP8, rows, K, xd, codes, scales)
    torch.cuda.synchronize()
    ref_codes, ref_scales = M.quantize(xs, fmt)
    if fmt == "fp4":
        ref_codes = M.pack_fp4(ref_codes)
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad_s = got_s != ref_scales
    assert not bad_s.any(), f"scales: {int(bad_s.sum())} differ, first at {np.argwhere(bad_s)[0]}"
    bad_c = got_c != ref_codes
    assert not bad_c.any(), (f"codes: {int(bad_c.sum())} differ, first at {np.argwhere(bad_c)[0]}: "
                             f"{got_c[bad_c][:8]} vs {ref_codes[bad_c][:8]}")


def test_mx_quantize_ragged_and_empty():
    """rows = 0 is a no-op; a row count that is not a multiple of the launch block is covered."""
    cfg = CONFIGS["mid_bf16"]
    shape = C.make_shape(cfg, 1)
    rng = np.random.default_rng(9)
    K = 96
    x = O.store(rng.standard_normal((37, K)), "bf16")
    xd = torch.as_tensor(x).to(torch.bfloat16).cuda()
    codes = torch.full((38, K), 0xAB, dtype=torch.uint8, device="cuda")
    scales = torch.full((38, K // 32), 0xCD, dtype=torch.uint8, device="cuda")
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP8, 0, K, xd, codes, scales)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP8, 37, K, xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = M.quantize(x, "fp8")
    assert np.array_equal(codes[:37].cpu().numpy(), rc)
    assert np.array_equal(scales[:37].cpu().numpy(), rs)
    assert (codes[37] == 0xAB).all() and (scales[37] == 0xCD).all()   # nothing written past the rows


# ------------------------------------------------------------------------------------------------
# routed experts on MX operands (lmoe_grouped_situ_glu_mx)
# ------------------------------------------------------------------------------------------------
MX_CASES = {
    "mid_bf16_T1000": (replace(CONFIGS["mid_bf16"], T=1000), 0),
    "mid_bf16_few_experts": (replace(CONFIGS["mid_bf16"], T=512), 8),
}


def run_mx_layer(cfg, n_live, seed=4):
    inp = make_inputs(cfg, seed=seed)
    if n_live:  # every expert but the first n_live is pushed out of every top-k
        inp["bias"] = np.where(np.arange(cfg.n_experts) < n_live, 0.0, -10.0).astype(np.float32)
    w = upload_weights(inp, cfg.act_dtype)
    layer = LatentMoE(cfg, w, mx=True)
    x = to_device(inp["x"], cfg.act_dtype)
    b = layer.forward(x, accumulate_hist=False)
    torch.cuda.synchronize()
    return inp, layer, b


def check_mx_weights(layer, inp, experts):
    """The layer's FP4 weights are the oracle's quantisation of the bf16 weights (bit for bit)."""
    out = {}
    for name in ("w1", "w2"):
        codes, scales = layer.mx_w[name]
        for e in experts:
            ref_c, ref_s = M.quantize(O.to_f64(inp[name][e], "bf16"), "fp4")
            assert np.array_equal(codes[e].cpu().numpy(), M.pack_fp4(ref_c)), (name, e)
            assert np.array_equal(scales[e].cpu().numpy(), ref_s), (name, e)
            out[(name, e)] = (ref_c, ref_s)
    return out


def check_mx_experts(cfg, inp, layer, b, experts, rows_per_expert=None):
    """Per expert: h against the oracle's first stage on the GPU's x_lat rows, y against the
    oracle's second stage on the GPU's h (each compared to one bf16 rounding plus f32 accumulation
    noise), and the layer's x_lat codes against the oracle's quantisation."""
    offs = b["offsets"].cpu().numpy()
    st = b["sorted_token"].cpu().numpy()
    x_lat = host(b["x_lat"])
    xc, xs = b["x_lat_codes"].cpu().numpy(), b["x_lat_scales"].cpu().numpy()
    rows_of = lambda name, rr: host(b[name][torch.as_tensor(rr, device=b[name].device)])  # noqa: E731
    wq = check_mx_weights(layer, inp, experts)
    worst = {"h": 0.0, "y": 0.0}
    for e in experts:
        lo, hi = int(offs[e]), int(offs[e + 1])
        if hi == lo:
            continue
        rr = np.arange(lo, hi)
        if rows_per_expert and hi - lo > rows_per_expert:
            rr = np.sort(np.random.default_rng(e).choice(rr, rows_per_expert, replace=False))
        tok = st[rr]
        h_ref, aq, asc = M.mx_glu_stage(x_lat[tok], *wq[("w1", e)], cfg.beta1, cfg.beta2)
        assert np.array_equal(xc[tok], aq) and np.array_equal(xs[tok], asc), f"x_lat codes, expert {e}"
        h = rows_of("h", rr)
        worst["h"] = max(worst["h"], assert_close_rows(h, h_ref, "bf16", f"h expert {e}"))
        y_ref = M.mx_down_stage(h, *wq[("w2", e)])
        worst["y"] = max(worst["y"], assert_close_rows(rows_of("y", rr), y_ref, "bf16", f"y expert {e}"))
    say(f"MX experts {len(experts)}: max err/RMS h {worst['h']:.3e}, y {worst['y']:.3e}")


@pytest.mark.parametrize("name", list(MX_CASES))
def test_grouped_mx_parity(name):
    cfg, n_live = MX_CASES[name]
    say(f"grouped MX parity {name}: T={cfg.T} L={cfg.d_latent} I={cfg.inter} E={cfg.n_experts}")
    inp, layer, b = run_mx_layer(cfg, n_live)
    offs = b["offsets"].cpu().numpy()
    counts = np.diff(offs)
    assert counts.sum() == cfg.T * cfg.top_k
    experts = list(range(cfg.n_experts)) if n_live else [int(e) for e in np.argsort(counts)[[0, 1, -1, -2]]] + \
        [e for e in range(0, cfg.n_experts, 9)]
    check_mx_experts(cfg, inp, layer, b, sorted(set(experts)))
    # whole layer output close to the bf16 layer's (MX quantisation noise only)
    w = upload_weights(inp, cfg.act_dtype)
    ref = LatentMoE(cfg, w).forward(to_device(inp["x"], cfg.act_dtype), accumulate_hist=False)
    out, out_ref = host(b["out"]), host(ref["out"])
    rel = float(np.sqrt(np.mean((out - out_ref) ** 2)) / np.sqrt(np.mean(out_ref ** 2)))
    say(f"MX layer vs bf16 layer: RMS diff / RMS = {rel:.3e}")
    assert rel < 0.3   # FP4 weights alone carry ~12 % RMS error on Gaussian rows: a sanity bound


def test_grouped_mx_k3_sampled():
    """K3 prefill shape (T=8192, L=3584, I=512, 896 experts), in the benchmark's launch
    configuration: sampled experts (largest, smallest, spread) and sampled rows of each."""
    cfg = CONFIGS["k3_prefill"]
    say(f"grouped MX K3 sampled: T={cfg.T}")
    inp, layer, b = run_mx_layer(cfg, 0, seed=0)
    counts = np.diff(b["offsets"].cpu().numpy())
    order = np.argsort(counts, kind="stable")
    experts = sorted(set([int(order[0]), int(order[-1]), int(order[len(order) // 2])] + list(range(3, 896, 149))))
    check_mx_experts(cfg, inp, layer, b, experts, rows_per_expert=48)


def test_grouped_mx_one_group_no_gather():
    """One group (group_offsets NULL) read without a row gather, a row count that is not a multiple
    of the 256-row tile, against the oracle's two stages."""
    cfg = CONFIGS["mid_bf16"]
    rng = np.random.default_rng(13)
    rows, K, inter, n_out = 300, 1024, 256, 1024
    a = O.store(rng.standard_normal((rows, K)), "bf16")
    w1 = O.store(rng.standard_normal((2 * inter, K)) * K ** -0.5, "bf16")
    w2 = O.store(rng.standard_normal((n_out, inter)) * inter ** -0.5, "bf16")
    dev = lambda v: torch.as_tensor(v).to(torch.bfloat16).cuda()  # noqa: E731
    shape = C.make_shape(cfg, rows)
    u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")  # noqa: E731
    ac, asc = u8(rows, K), u8(rows, K // 32)
    w1c, w1s, w2c, w2s = u8(2 * inter, K // 2), u8(2 * inter, K // 32), u8(n_out, inter // 2), u8(n_out, inter // 32)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP8, rows, K, dev(a), ac, asc)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP4, 2 * inter, K, dev(w1), w1c, w1s)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP4, n_out, inter, dev(w2), w2c, w2s)
    h = torch.empty(rows, inter, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(rows, n_out, dtype=torch.bfloat16, device="cuda")
    ws = u8(1 << 20)
    say(f"grouped MX one group: rows={rows} K={K} inter={inter} n_out={n_out}")
    C.lmoe_grouped_situ_glu_mx(shape, 1, rows, K, inter, n_out, ac, asc, rows, None, None, w1c, w1s, w2c, w2s, h, y,
                               ws)
    torch.cuda.synchronize()
    q1c, q1s = M.quantize(w1, "fp4")
    q2c, q2s = M.quantize(w2, "fp4")
    h_ref, _, _ = M.mx_glu_stage(a, q1c, q1s, cfg.beta1, cfg.beta2)
    e_h = assert_close_rows(host(h), h_ref, "bf16", "h")
    e_y = assert_close_rows(host(y), M.mx_down_stage(host(h), q2c, q2s), "bf16", "y")
    say(f"max err/RMS h {e_h:.3e}, y {e_y:.3e}")


def test_grouped_mx_k3_decode():
    """K3 decode (T = 64, 1024 pairs over 896 experts: most groups hold one or two rows)."""
    cfg = CONFIGS["k3_decode"]
    say(f"grouped MX K3 decode: T={cfg.T}")
    inp, layer, b = run_mx_layer(cfg, 0, seed=2)
    counts = np.diff(b["offsets"].cpu().numpy())
    live = np.nonzero(counts)[0]
    experts = sorted(set([int(live[0]), int(live[-1]), int(np.argmax(counts))] + [int(e) for e in live[::60]]))
    check_mx_experts(cfg, inp, layer, b, experts)


def test_grouped_mx_small_dims_and_empty_groups():
    """The smallest dimensions the call takes (K = inter = 128: one K-tile each), an output width
    that is not a multiple of the 256-column tile (n_out = 136), and groups that are empty at the
    start, in the middle and at the end, with rows gathered out of order."""
    cfg = CONFIGS["mid_bf16"]
    rng = np.random.default_rng(17)
    K, inter, n_out, G = 128, 128, 136, 6
    sizes = np.array([0, 5, 0, 300, 33, 0])
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    rows = int(offs[-1])
    a_rows = 100
    idx = rng.integers(0, a_rows, rows).astype(np.int32)
    a = O.store(rng.standard_normal((a_rows, K)), "bf16")
    w1 = O.store(rng.standard_normal((G, 2 * inter, K)) * K ** -0.5, "bf16")
    w2 = O.store(rng.standard_normal((G, n_out, inter)) * inter ** -0.5, "bf16")
    dev = lambda v: torch.as_tensor(v).to(torch.bfloat16).cuda()  # noqa: E731
    u8 = lambda *s: torch.empty(*s, dtype=torch.uint8, device="cuda")  # noqa: E731
    shape = C.make_shape(cfg, rows)
    ac, asc = u8(a_rows, K), u8(a_rows, K // 32)
    w1c, w1s = u8(G, 2 * inter, K // 2), u8(G, 2 * inter, K // 32)
    w2c, w2s = u8(G, n_out, inter // 2), u8(G, n_out, inter // 32)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP8, a_rows, K, dev(a), ac, asc)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP4, G * 2 * inter, K, dev(w1), w1c, w1s)
    C.lmoe_mx_quantize(shape, C.LMOE_MX_FP4, G * n_out, inter, dev(w2), w2c, w2s)
    h = torch.empty(rows, inter, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(rows, n_out, dtype=torch.bfloat16, device="cuda")
    ws = u8(1 << 20)
    say(f"grouped MX small dims: groups {sizes.tolist()}, K={K} inter={inter} n_out={n_out}")
    C.lmoe_grouped_situ_glu_mx(shape, G, rows, K, inter, n_out, ac, asc, a_rows, torch.as_tensor(idx).cuda(),
                               torch.as_tensor(offs).cuda(), w1c, w1s, w2c, w2s, h, y, ws)
    torch.cuda.synchronize()
    hg, yg = host(h), host(y)
    for g in range(G):
        lo, hi = int(offs[g]), int(offs[g + 1])
        if hi == lo:
            continue
        q1c, q1s = M.quantize(w1[g], "fp4")
        q2c, q2s = M.quantize(w2[g], "fp4")
        h_ref, _, _ = M.mx_glu_stage(a[idx[lo:hi]], q1c, q1s, cfg.beta1, cfg.beta2)
        assert_close_rows(hg[lo:hi], h_ref, "bf16", f"h group {g}")
        assert_close_rows(yg[lo:hi], M.mx_down_stage(hg[lo:hi], q2c, q2s), "bf16", f"y group {g}")
