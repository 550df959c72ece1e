"""GPU parity of every C-ABI call and of the whole layer against the CPU oracle (small workloads).

Sizes span several tiles plus ragged tails: tiny_f32 (T=64), mid_bf16 (T=4096), ragged token
counts, and tiny_f32 at T=1024 (4096 expert rows: the routed GEMMs take the 256-row DMA pipeline in
f32). The "_gb" cases draw a non-unit RMSNorm gain and a non-zero starting bias. Integer results
(top-k given the scores, histograms, bias updates, permutation) must be
bit-exact; stored floating tensors match to one rounding step of their storage type; the layer
output matches within 2e-2 x RMS (bf16) or 1e-4 x RMS (f32), excluding only near-tie tokens whose
top-k set legitimately differs (counted), and within the same bound on every token when the GPU's
routing is fed to the oracle.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_space_routed_amd import _lib as C
from oracle import lmoe_oracle as O
from workloads import CONFIGS
from workloads.inputs import make_inputs

from .gpu_helpers import (assert_close_rows, assert_out_parity, cached_inputs, device_layer, host, near_ties, say)

pytestmark = pytest.mark.gpu

TINY = CONFIGS["tiny_f32"]
MID = CONFIGS["mid_bf16"]
# (config, gain_bias): gain_bias draws gamma = 1 + 0.5 N(0,1) and b = 0.05 N(0,1)
SMALL_CASES = [(TINY, False), (replace(TINY, name="tiny_gb"), True), (replace(TINY, name="tiny_ragged_gb", T=77), True),
               (replace(TINY, name="tiny_big_gb", T=1024), True), (MID, False),
               (replace(MID, name="mid_ragged_gb", T=1000), True),
               # narrow bf16 experts with few rows each: the routed GEMMs on 128-row tiles (the
               # register pipeline), which wider bf16 experts no longer take
               (replace(MID, name="mid_narrow_gb", T=300, d_latent=512, inter=128), True)]
# fused: routed GEMM gathers x_lat rows, shared down-projection folded into the up-projection;
# unfused: x_perm and y_sh materialised
RUNS = [(c, gb, f) for c, gb in SMALL_CASES for f in (True, False)]
IDS = [f"{c.name}-{'fused' if f else 'unfused'}" for c, gb, f in RUNS]
_ORACLE = {}


def oracle_forward(cfg, inp):
    if cfg.name not in _ORACLE:
        _ORACLE[cfg.name] = O.forward(inp, cfg)
    return _ORACLE[cfg.name]


@pytest.fixture(scope="module", params=RUNS, ids=IDS)
def run(request):
    cfg, gain_bias, fused = request.param
    say(f"[case] {cfg.name} T={cfg.T} fused={fused} gain_bias={gain_bias}")
    inp = cached_inputs(cfg, gain_bias=gain_bias)
    layer, x = device_layer(cfg, inp, fused=fused)
    b = layer.forward(x)
    torch.cuda.synchronize()
    g = {k: host(v) for k, v in b.items() if not k.startswith("ws_") and v is not None}
    g["hist"] = layer.hist.cpu().numpy().view(np.uint32).copy()
    g["fused"] = fused
    ref = oracle_forward(cfg, inp)
    return cfg, inp, layer, x, g, ref


def test_route_scores_and_topk(run):
    cfg, inp, layer, x, g, ref = run
    ds = np.abs(g["scores"] - ref["s"]).max()
    say(f"{cfg.name}: max |s_gpu - s_oracle| = {ds:.3e}")
    assert ds <= 2e-6
    # given the GPU's scores, top-k, weights and thresholds are those of the oracle exactly
    s32 = g["scores"].astype(np.float32)
    idx, w, thr = O.select_topk(s32, inp["bias"], cfg.top_k)
    np.testing.assert_array_equal(g["idx"], idx)
    np.testing.assert_array_equal(g["thresh"].astype(np.float32), thr)
    np.testing.assert_allclose(g["w"], w, rtol=2e-7, atol=0)
    # against the oracle's own routing: same sets except near-ties
    tie = near_ties(ref["thresh"])
    same = np.array([set(a) == set(b) for a, b in zip(g["idx"], ref["idx"])])
    say(f"{cfg.name}: near-tie tokens {int(tie.sum())}, differing top-k sets {int((~same).sum())}")
    assert np.all(same | tie)


def test_qb_histogram_bit_exact(run):
    cfg, inp, layer, x, g, ref = run
    H = O.qb_histogram(g["scores"].astype(np.float32), inp["bias"], g["idx"], g["thresh"].astype(np.float32),
                       cfg.n_bins)
    np.testing.assert_array_equal(g["hist"], H)
    flips = int(np.abs(g["hist"].astype(np.int64) - ref["hist"].astype(np.int64)).sum() // 2)
    say(f"{cfg.name}: histogram bin moves vs oracle's own scores: {flips}")


def test_qb_histogram_with_bias_and_accumulation(run):
    cfg, inp, layer, x, g, ref = run
    rng = np.random.default_rng(3)
    bias = (rng.standard_normal(cfg.n_experts) * 0.05).astype(np.float32)
    shape = C.make_shape(cfg)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    s, tb = dev(g["scores"].astype(np.float32)), dev(bias)
    idx = torch.empty(cfg.T, cfg.top_k, dtype=torch.int32, device="cuda")
    w = torch.empty(cfg.T, cfg.top_k, dtype=torch.float32, device="cuda")
    thr = torch.empty(cfg.T, 2, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(C.workspace_bytes(shape, C.LMOE_CALL_ROUTE), 256), dtype=torch.uint8, device="cuda")
    C.lmoe_route(shape, x, layer.w["w_router"], tb, layer.w.get("logit_offset"), s, idx, w, thr, ws)
    hist = torch.zeros(cfg.n_experts, cfg.n_bins, dtype=torch.int32, device="cuda")
    C.lmoe_qb_histogram(shape, s, tb, idx, thr, hist)
    C.lmoe_qb_histogram(shape, s, tb, idx, thr, hist)
    sh, ih, th = host(s).astype(np.float32), host(idx), host(thr).astype(np.float32)
    H1 = O.qb_histogram(sh, bias, ih, th, cfg.n_bins)
    np.testing.assert_array_equal(ih, O.select_topk(sh, bias, cfg.top_k)[0])
    np.testing.assert_array_equal(hist.cpu().numpy().view(np.uint32), O.qb_histogram(sh, bias, ih, th, cfg.n_bins, H1))


def test_qb_update_bit_exact(run):
    cfg, inp, layer, x, g, ref = run
    hist = torch.from_numpy(g["hist"].view(np.int32).copy()).cuda()
    rng = np.random.default_rng(4)
    bias0 = (rng.standard_normal(cfg.n_experts) * 0.01).astype(np.float32)
    bias = torch.from_numpy(bias0.copy()).cuda()
    C.lmoe_qb_update(C.make_shape(cfg), hist, cfg.T, bias)
    want, _ = O.qb_update(g["hist"], cfg.T, bias0, cfg.top_k)
    np.testing.assert_array_equal(bias.cpu().numpy(), want)
    assert not hist.cpu().numpy().any()


def test_permute_bit_exact(run):
    cfg, inp, layer, x, g, ref = run
    off, st, sp = O.permute(g["idx"], cfg.n_experts)
    np.testing.assert_array_equal(g["offsets"], off)
    np.testing.assert_array_equal(g["sorted_token"], st)
    np.testing.assert_array_equal(g["slot_of_pair"], sp)
    if not g["fused"]:
        np.testing.assert_array_equal(g["x_perm"], g["x_lat"][g["sorted_token"]])
    e = assert_close_rows(g["x_lat"], ref["x_lat"], cfg.act_dtype, "x_lat")
    say(f"{cfg.name}: x_lat max err/RMS {e:.2e}")


def test_grouped_glu_parity(run):
    cfg, inp, layer, x, g, ref = run
    dt = cfg.act_dtype
    h_ref = np.zeros_like(g["h"])
    y_ref = np.zeros_like(g["y"])
    off = g["offsets"]
    rows_in = g["x_lat"][g["sorted_token"]]  # the GEMM's A rows, gathered or materialised
    for e in range(cfg.n_experts):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            h_ref[r0:r1], y_ref[r0:r1] = O.situ_glu_ffn(rows_in[r0:r1], O.to_f64(inp["w1"][e], dt),
                                                        O.to_f64(inp["w2"][e], dt), cfg.beta1, cfg.beta2, dt)
    assert_close_rows(g["h"], h_ref, dt, "h")
    # y from the GPU's own h isolates GEMM2 from the h rounding of GEMM1
    y_from_gpu_h = np.zeros_like(y_ref)
    for e in range(cfg.n_experts):
        r0, r1 = off[e], off[e + 1]
        if r1 > r0:
            y_from_gpu_h[r0:r1] = O.store(g["h"][r0:r1] @ O.to_f64(inp["w2"][e], dt).T, dt)
    assert_close_rows(g["y"], y_from_gpu_h, dt, "y")


def test_shared_experts_parity(run):
    cfg, inp, layer, x, g, ref = run
    dt = cfg.act_dtype
    S, Is = cfg.n_shared, cfg.inter_shared
    assert_close_rows(g["h_s"][:, : S * Is], ref["h_s"], dt, "h_s")
    if not g["fused"]:
        ysh = O.store(g["h_s"][:, : S * Is] @ np.concatenate(list(O.to_f64(inp["w2s"], dt)), axis=1).T, "f32")
        assert_close_rows(g["y_sh"], ysh, "f32" if dt == "f32" else "bf16", "y_sh")


def test_combine_norm_up_parity(run):
    cfg, inp, layer, x, g, ref = run
    dt = cfg.act_dtype
    T, k = cfg.T, cfg.top_k
    y_pairs = g["y"][g["slot_of_pair"]].reshape(T, k, -1)
    z = O.combine(y_pairs, g["w"].astype(np.float32))
    n_ref = O.store(O.rms_norm(z, inp["gamma"], cfg.rms_eps), dt)
    assert_close_rows(g["n"], n_ref, dt, "n")
    if g["fused"]:
        S, Is = cfg.n_shared, cfg.inter_shared
        w2s_cat = np.concatenate(list(O.to_f64(inp["w2s"], dt)), axis=1)
        pre, _ = O.up_project(g["n"], O.to_f64(inp["w_up"], dt), g["h_s"][:, : S * Is] @ w2s_cat.T, dt)
    else:
        pre, _ = O.up_project(g["n"], O.to_f64(inp["w_up"], dt), g["y_sh"], dt)
    assert_close_rows(g["out"], pre, "f32", "out (from the GPU's n)")


def test_layer_output_parity(run):
    cfg, inp, layer, x, g, ref = run
    tie = near_ties(ref["thresh"])
    same = np.array([set(a) == set(b) for a, b in zip(g["idx"], ref["idx"])])
    assert_out_parity(g["out"], ref["out_pre"], cfg.act_dtype, f"{cfg.name} end to end", mask=same)
    say(f"{cfg.name}: tokens excluded (differing near-tie routing): {int((~same).sum())} of {cfg.T}; "
        f"near-tie tokens {int(tie.sum())}")
    # every token, with the GPU's routing fed to the oracle
    forced = O.expert_path(inp, cfg, g["idx"], g["w"].astype(np.float32))
    assert_out_parity(g["out"], forced["out_pre"], cfg.act_dtype, f"{cfg.name} forced routing")


def test_deterministic(run):
    cfg, inp, layer, x, g, ref = run
    b = layer.forward(x, accumulate_hist=False)
    torch.cuda.synchronize()
    for name in ("scores", "idx", "w", "thresh", "x_lat", "offsets", "slot_of_pair", "x_perm", "h", "y", "n", "out"):
        if b[name] is not None:
            np.testing.assert_array_equal(host(b[name]), g[name], err_msg=name)


def test_side_stream_and_split_calls_bit_identical(run):
    """With the side stream on, the fused layer runs the shared GEMM1 on a stream forked at the start
    of the step, beside the routing, down-projection and permutation, and joins before the routed
    experts; off, every call runs on one stream. Both give the same n, h_s and out bit for bit (same
    kernels, same per-stream order)."""
    cfg, inp, layer, x, g, ref = run
    if not g["fused"] or cfg.n_shared == 0:
        pytest.skip("the side stream is used on the fused path with shared experts")
    side, _ = device_layer(cfg, inp)
    side.overlap_shared = True
    side.bias.copy_(layer.bias)
    layer.overlap_shared = False
    b1 = layer.forward(x, accumulate_hist=False)
    b2 = side.forward(x, accumulate_hist=False)
    torch.cuda.synchronize()
    for name in ("n", "h_s", "out"):
        np.testing.assert_array_equal(host(b2[name]), host(b1[name]), err_msg=name)


# ---------------------------------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------------------------------
def test_zero_tokens():
    cfg = replace(MID, T=0)
    inp = make_inputs(replace(MID, T=8))
    inp["x"] = inp["x"][:0]
    layer, x = device_layer(cfg, inp, max_tokens=8)
    b = layer.forward(x)
    torch.cuda.synchronize()
    assert host(b["offsets"]).tolist() == [0] * (cfg.n_experts + 1)
    assert b["out"].shape[0] == 0


def test_all_tokens_to_one_expert_and_empty_experts():
    # b_0 = +2 lifts expert 0 above every unbiased score in (0, 1): n_0 = T; large biases on experts
    # 1..k-1 fill the rest, so every other expert is empty.
    cfg = replace(MID, T=640)
    inp = dict(cached_inputs(cfg))
    bias = np.zeros(cfg.n_experts, np.float32)
    bias[: cfg.top_k] = 2.0
    inp["bias"] = bias
    layer, x = device_layer(cfg, inp)
    b = layer.forward(x)
    torch.cuda.synchronize()
    off = host(b["offsets"])
    counts = np.diff(off)
    assert counts[: cfg.top_k].tolist() == [cfg.T] * cfg.top_k and counts[cfg.top_k:].sum() == 0
    ref = O.forward(inp, cfg)
    np.testing.assert_array_equal(host(b["idx"]), ref["idx"])
    assert_out_parity(host(b["out"]), ref["out_pre"], cfg.act_dtype, "single-expert routing")


def test_qb_loop_matches_oracle_step_by_step():
    # Skewed router (Zipf logit offsets); four micro-batches, one update each. Every update is
    # bit-exact given the GPU's histogram, and the load spread shrinks.
    cfg = replace(MID, name="mid_skew", T=2048, zipf_s=1.1)
    inp = make_inputs(cfg)
    layer, _ = device_layer(cfg, inp)
    ratios = []
    for batch in range(4):
        xb = make_inputs(cfg, batch=batch)["x"]
        from latent_space_routed_amd import to_device
        b = layer.forward(to_device(xb, cfg.act_dtype))
        torch.cuda.synchronize()
        load = np.bincount(host(b["idx"]).ravel(), minlength=cfg.n_experts)
        ratios.append(load.max() / load.mean())
        hist = layer.hist.cpu().numpy().view(np.uint32).copy()
        bias_before = layer.bias.cpu().numpy().copy()
        layer.qb_update()
        want, _ = O.qb_update(hist, cfg.T, bias_before, cfg.top_k)
        np.testing.assert_array_equal(layer.bias.cpu().numpy(), want)
    say(f"max/mean expert load per batch: {[round(r, 2) for r in ratios]}")
    assert ratios[-1] < ratios[0]


def test_invalid_arguments_leave_outputs_untouched():
    cfg = MID
    shape = C.make_shape(cfg, 16)
    s = torch.full((16, cfg.n_experts), 7.0, device="cuda")
    x = torch.zeros(16, cfg.d_model, dtype=torch.bfloat16, device="cuda")
    wr = torch.zeros(cfg.n_experts, cfg.d_model, device="cuda")
    bias = torch.zeros(cfg.n_experts, device="cuda")
    idx = torch.full((16, cfg.top_k), -5, dtype=torch.int32, device="cuda")
    w = torch.zeros(16, cfg.top_k, device="cuda")
    thr = torch.zeros(16, 2, device="cuda")
    small_ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(C.LmoeError) as e:
        C.lmoe_route(shape, x, wr, bias, None, s, idx, w, thr, small_ws)
    assert e.value.status == C.LMOE_ERR_WORKSPACE
    bad = C.make_shape(cfg, 16)
    bad.top_k = cfg.n_experts
    ws = torch.empty(C.workspace_bytes(shape, C.LMOE_CALL_ROUTE), dtype=torch.uint8, device="cuda")
    with pytest.raises(C.LmoeError) as e:
        C.lmoe_route(bad, x, wr, bias, None, s, idx, w, thr, ws)
    assert e.value.status == C.LMOE_ERR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    assert bool((s == 7.0).all()) and bool((idx == -5).all())
