"""GPU parity at the K3 layer shape (d_model 7168, d_latent 3584, 896 experts top-16, 2 shared).

* k3_prefill (T=8192), in the launch configuration the benchmark times, with a non-unit RMSNorm
  gain and a non-zero starting bias: routing, histogram, bias update and permutation are checked
  on every token (bit-exact given the GPU's scores); the expert path on 1024 seeded-sampled
  tokens plus every token whose oracle gap between the k-th and (k+1)-th biased score is below
  1e-5, each evaluated by the oracle one by one.
* k3_decode (T=64): every token end to end (about 613 of 896 experts touched).
* k3_stress (T=32768, Zipf(1.1) logit offsets, 0.1% of x entries x50): 8 batches with a bias update
  after each, every step bit-exact given the GPU's scores and histogram, the load spread
  reported; the expert path on the last batch is checked on 1024 sampled tokens plus the 64
  tokens carrying the most outliers and every near-tie token.
"""
from dataclasses import replace

import numpy as np
import pytest
import torch

from latent_space_routed_amd import LatentMoE, to_device, upload_weights
from oracle import lmoe_oracle as O
from workloads import CONFIGS
from workloads.inputs import bf16_bits_to_f32, gain_and_bias, logit_offsets, make_inputs, token_rows

from .gpu_helpers import assert_close_rows, assert_out_parity, host, near_ties, say

pytestmark = pytest.mark.gpu

K3 = CONFIGS["k3_prefill"]
_CACHE = {}


def k3_weights():
    if "w" not in _CACHE:
        say("[k3] generating K3 weights")
        inp = make_inputs(replace(K3, T=0), with_x=False)
        _CACHE["inp"] = inp
        _CACHE["w"] = upload_weights(inp, K3.act_dtype)
        torch.cuda.synchronize()
    return _CACHE["inp"], _CACHE["w"]


N_SAMPLE = 1024  # seeded-sampled tokens of the expert-path checks at K3 scale


def layer_for(cfg, fused: bool = True, gain_bias: bool = False):
    inp_w, w = k3_weights()
    inp = dict(inp_w)
    inp["logit_offset"] = logit_offsets(cfg)
    w = dict(w)
    w["logit_offset"] = to_device(inp["logit_offset"], cfg.act_dtype)
    if gain_bias:  # gamma = 1 + 0.5 N(0,1), b = 0.05 N(0,1)
        inp["gamma"], inp["bias"] = gain_and_bias(cfg)
        w["gamma"] = to_device(inp["gamma"], "f32")
        w["bias"] = to_device(inp["bias"], "f32")
    return inp, LatentMoE(cfg, w, fused=fused)


def sample_tokens(T: int, seed: int, *must) -> np.ndarray:
    """N_SAMPLE seeded tokens, the first and last token, and every token listed in ``must``."""
    rng = np.random.default_rng(seed)
    extra = [np.asarray(m, dtype=np.int64).ravel() for m in must]
    return np.unique(np.concatenate([rng.choice(T, N_SAMPLE, replace=False), [0, T - 1], *extra]))


def check_sampled_tokens(cfg, inp, b, tokens, what):
    """Each stage against the oracle fed the GPU's own inputs to that stage (one rounding step of
    the storage type), then the whole chain end to end within the stated output tolerance."""
    dt = cfg.act_dtype
    T, k = cfg.T, cfg.top_k
    tok = torch.as_tensor(tokens, device="cuda")
    g_idx = host(b["idx"])
    g_w = host(b["w"]).astype(np.float32)
    slot = host(b["slot_of_pair"]).reshape(T, k)[tokens]
    sl = torch.as_tensor(slot.reshape(-1), device="cuda", dtype=torch.long)
    x_lat = host(b["x_lat"][tok])
    h = host(b["h"][sl]).reshape(len(tokens), k, -1)
    y = host(b["y"][sl]).reshape(len(tokens), k, -1)
    n = host(b["n"][tok])
    h_s = host(b["h_s"][tok])[:, : cfg.n_shared * cfg.inter_shared]
    y_sh = host(b["y_sh"][tok]) if b["y_sh"] is not None else None
    out = host(b["out"][tok])
    x = O.to_f64(np.asarray(inp["x"])[tokens], dt)
    assert_close_rows(x_lat, O.down_project(x, O.to_f64(inp["w_down"], dt), dt), dt, f"{what} x_lat")
    sel = g_idx[tokens]
    h_ref = np.zeros_like(h)
    y_ref = np.zeros_like(y)
    for e in np.unique(sel):
        rr, jj = np.nonzero(sel == e)
        w1, w2 = O.to_f64(inp["w1"][e], dt), O.to_f64(inp["w2"][e], dt)
        h_ref[rr, jj], _ = O.situ_glu_ffn(x_lat[rr], w1, w2, cfg.beta1, cfg.beta2, dt)
        y_ref[rr, jj] = O.store(h[rr, jj] @ w2.T, dt)
    assert_close_rows(h, h_ref, dt, f"{what} h")
    assert_close_rows(y, y_ref, dt, f"{what} y")
    z = O.combine(y, g_w[tokens])
    assert_close_rows(n, O.store(O.rms_norm(z, inp["gamma"], cfg.rms_eps), dt), dt, f"{what} n")
    h_s_ref, _ = O.shared_experts(x, O.to_f64(inp["w1s"], dt), O.to_f64(inp["w2s"], dt), cfg.beta1, cfg.beta2, dt)
    assert_close_rows(h_s, h_s_ref, dt, f"{what} h_s")
    w2s_cat = np.concatenate(list(O.to_f64(inp["w2s"], dt)), axis=1)
    if y_sh is not None:  # materialised shared output
        assert_close_rows(y_sh, O.store(h_s @ w2s_cat.T, "f32"), "f32", f"{what} y_sh")
        pre, _ = O.up_project(n, O.to_f64(inp["w_up"], dt), y_sh, dt)
    else:  # shared down-projection accumulated with the up-projection
        pre, _ = O.up_project(n, O.to_f64(inp["w_up"], dt), h_s @ w2s_cat.T, dt)
    assert_close_rows(out, pre, "f32", f"{what} out from the GPU's n")
    ex = O.expert_path(inp, cfg, g_idx, g_w, tokens=tokens)
    return assert_out_parity(out, ex["out_pre"], dt, f"{what} out end to end (GPU routing, {len(tokens)} tokens)")


def check_routing_all_tokens(cfg, inp, x_host, b, bias):
    """Routing, histogram-ready outputs and permutation of every token against the oracle."""
    s = host(b["scores"]).astype(np.float32)
    idx, w, thr = O.select_topk(s, bias, cfg.top_k)
    np.testing.assert_array_equal(host(b["idx"]), idx)
    np.testing.assert_array_equal(host(b["thresh"]).astype(np.float32), thr)
    np.testing.assert_allclose(host(b["w"]), w, rtol=3e-7, atol=0)
    off, st, sp = O.permute(idx, cfg.n_experts)
    np.testing.assert_array_equal(host(b["offsets"]), off)
    np.testing.assert_array_equal(host(b["sorted_token"]), st)
    np.testing.assert_array_equal(host(b["slot_of_pair"]), sp)
    if b["x_perm"] is not None:
        st_dev = torch.as_tensor(st, device="cuda", dtype=torch.long)
        assert torch.equal(b["x_perm"].view(torch.int16), b["x_lat"][st_dev].view(torch.int16))
    return s, idx, thr


def test_k3_prefill():
    cfg = K3
    inp, layer = layer_for(cfg, gain_bias=True)
    x_host = token_rows(cfg)
    inp["x"] = x_host
    x = to_device(x_host, cfg.act_dtype)
    say("[k3_prefill] GPU forward")
    b = layer.forward(x)
    torch.cuda.synchronize()
    hist = layer.hist.cpu().numpy().view(np.uint32).copy()
    s, idx, thr = check_routing_all_tokens(cfg, inp, x_host, b, inp["bias"])
    say("[k3_prefill] routing and permutation bit-exact given the GPU scores")
    np.testing.assert_array_equal(hist, O.qb_histogram(s, inp["bias"], idx, thr, cfg.n_bins))
    bias_before = layer.bias.cpu().numpy().copy()
    layer.qb_update()
    want, _ = O.qb_update(hist, cfg.T, bias_before, cfg.top_k)
    np.testing.assert_array_equal(layer.bias.cpu().numpy(), want)
    say("[k3_prefill] histogram and bias update bit-exact")
    # the oracle's own router on every token (float64 logits)
    s_ref = O.router_scores(O.to_f64(x_host, cfg.act_dtype), inp["w_router"], inp["logit_offset"])
    ds = float(np.abs(s - s_ref).max())
    idx_ref, _, thr_ref = O.select_topk(s_ref, inp["bias"], cfg.top_k)
    same = np.array([set(a) == set(c) for a, c in zip(idx, idx_ref)])
    tie = near_ties(thr_ref)
    say(f"[k3_prefill] max |s_gpu - s_oracle| = {ds:.2e}; near-tie tokens {int(tie.sum())}; "
        f"differing top-k sets {int((~same).sum())}")
    assert ds <= 2e-6 and np.all(same | tie)
    tokens = sample_tokens(cfg.T, 0, np.nonzero(tie)[0])
    say(f"[k3_prefill] expert path on {len(tokens)} tokens ({int(tie.sum())} near-tie tokens included)")
    check_sampled_tokens(cfg, inp, b, tokens, "k3_prefill")


def test_k3_prefill_unfused():
    """The unfused composition at K3 prefill: x_perm materialised, y_sh stored in f32 and added by
    the up-projection's epilogue; sampled tokens against the oracle."""
    cfg = K3
    inp, layer = layer_for(cfg, fused=False)
    x_host = token_rows(cfg)
    inp["x"] = x_host
    say("[k3_prefill unfused] GPU forward")
    b = layer.forward(to_device(x_host, cfg.act_dtype))
    torch.cuda.synchronize()
    check_routing_all_tokens(cfg, inp, x_host, b, inp["bias"])
    s_ref = O.router_scores(O.to_f64(x_host, cfg.act_dtype), inp["w_router"], inp["logit_offset"])
    tie = near_ties(O.select_topk(s_ref, inp["bias"], cfg.top_k)[2])
    tokens = sample_tokens(cfg.T, 1, np.nonzero(tie)[0])
    say(f"[k3_prefill unfused] expert path on {len(tokens)} tokens ({int(tie.sum())} near-tie tokens included)")
    check_sampled_tokens(cfg, inp, b, tokens, "k3_prefill unfused")


def test_k3_decode_every_token():
    cfg = CONFIGS["k3_decode"]
    inp, layer = layer_for(cfg)
    inp["x"] = token_rows(cfg)
    b = layer.forward(to_device(inp["x"], cfg.act_dtype))
    torch.cuda.synchronize()
    s, idx, thr = check_routing_all_tokens(cfg, inp, inp["x"], b, inp["bias"])
    touched = int((np.diff(host(b["offsets"])) > 0).sum())
    say(f"[k3_decode] experts touched: {touched} of {cfg.n_experts}")
    check_sampled_tokens(cfg, inp, b, np.arange(cfg.T), "k3_decode")


def test_k3_stress_qb_updates():
    cfg = CONFIGS["k3_stress"]
    inp, layer = layer_for(cfg)
    loads = []
    for batch in range(cfg.qb_updates):
        x_host = token_rows(cfg, batch=batch)
        b = layer.forward(to_device(x_host, cfg.act_dtype))
        torch.cuda.synchronize()
        bias_before = layer.bias.cpu().numpy().copy()
        s = host(b["scores"]).astype(np.float32)
        idx, _, thr = O.select_topk(s, bias_before, cfg.top_k)
        np.testing.assert_array_equal(host(b["idx"]), idx)
        hist = layer.hist.cpu().numpy().view(np.uint32).copy()
        np.testing.assert_array_equal(hist, O.qb_histogram(s, bias_before, idx, thr, cfg.n_bins))
        load = np.bincount(idx.ravel(), minlength=cfg.n_experts)
        loads.append(float(load.max() / load.mean()))
        if batch == cfg.qb_updates - 1:
            inp["x"] = x_host
            inp["bias"] = bias_before
            # the oracle's router on every token; the expert path on a sample that holds the tokens
            # with the most outlier entries and every near-tie token
            xf = O.to_f64(x_host, cfg.act_dtype)
            s_ref = O.router_scores(xf, inp["w_router"], inp["logit_offset"])
            idx_ref, _, thr_ref = O.select_topk(s_ref, bias_before, cfg.top_k)
            tie = near_ties(thr_ref)
            same = np.array([set(a) == set(c) for a, c in zip(idx, idx_ref)])
            # Rows carrying x50 outliers have products up to ~50x those of Gaussian rows, and the f32
            # accumulation error of their logits follows the partial sums those products leave: the
            # score error is held to the 1e-5 window of the near-tie rule itself (Gaussian rows stay
            # under 2e-6, checked at prefill), on every token, and any top-k set that differs from
            # the oracle's must belong to a near-tie token.
            err = np.abs(s - s_ref)
            say(f"[k3_stress] router on all {cfg.T} tokens: max |s_gpu - s_oracle| = {err.max():.2e} "
                f"(99.9th percentile {np.quantile(err, 0.999):.2e}); differing top-k sets {int((~same).sum())} "
                f"(all near-ties: {bool(np.all(same | tie))}), near-ties {int(tie.sum())}")
            assert err.max() <= 1e-5 and np.all(same | tie)
            big = (np.abs(bf16_bits_to_f32(x_host)) > 20).sum(axis=1)
            heavy = np.argsort(-big, kind="stable")[:64]
            tokens = sample_tokens(cfg.T, 1, heavy, np.nonzero(tie)[0])
            say(f"[k3_stress] expert path on {len(tokens)} tokens (64 outlier-heaviest, "
                f"{int(tie.sum())} near-tie tokens included)")
            check_sampled_tokens(cfg, inp, b, tokens, "k3_stress")
        layer.qb_update()
        want, _ = O.qb_update(hist, cfg.T, bias_before, cfg.top_k)
        np.testing.assert_array_equal(layer.bias.cpu().numpy(), want)
        say(f"[k3_stress] batch {batch}: max/mean expert load {loads[-1]:.2f}; update bit-exact")
    assert loads[-1] < loads[0] and loads[-1] < 1.6
