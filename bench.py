"""Benchmark: tokens/s of one Stable LatentMoE layer forward at K3 shape on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens: route (router GEMM,
top-k), QB histogram, down-projection + permutation, routed grouped SiTU-GLU FFNs, shared experts,
combine + RMSNorm + up-projection, and the QB bias update. Inputs are resident in HBM before the
timed region. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload k3_prefill] [--no-cpu-baseline]
                  [--backward] [--no-mx] [--no-graph] [--no-configs]

Timing: two pre-generated batches alternate step by step (so the timed routing is not the one the
bias was fitted to in warm-up; the bias update runs every step); before each timed step a 512 MB
buffer is written to flush the 256 MB MALL (outside the timed region); every step is bracketed by
HIP events on the launch stream, and ms_per_step is the median (min and mean reported beside it).
The headline line is the bf16 layer at k3_prefill, stepped eagerly. Under "configs" the other
workloads (tiny, mid, K3 decode, K3 stress) are timed the same way. Under "graph" the same step is
replayed from a HIP graph (same kernels, no launch gaps). Under "mx" the same steps are timed with
the routed experts on MXFP4 weights and MXFP8 activations (a variant with its own numerics, never
the headline value).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/s per Stable LatentMoE layer fwd (K3 shape); % bf16 MFMA / HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
DOMINANT = "gemm_glu_grouped"  # routed experts' GEMM1 + SiTU-GLU epilogue
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_glu_grouped_k3_prefill.json")
KERNEL_SOURCES = ("latent_space_routed_amd/csrc/gemm.hip", "latent_space_routed_amd/csrc/common.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def glu_bytes(cfg, offsets) -> tuple[float, float]:
    """Algorithmic HBM bytes and FLOPs of one routed GEMM1 launch: the W1 slices of the experts that
    received tokens, each token's latent row read once (the GEMM gathers rows of x_lat in place),
    and h written once."""
    import numpy as np

    counts = np.diff(offsets)
    touched = int((counts > 0).sum())
    rows = int(offsets[-1])
    esz = 2 if cfg.act_dtype == "bf16" else 4
    w_bytes = touched * 2 * cfg.inter * cfg.d_latent * esz
    a_bytes = cfg.T * cfg.d_latent * esz
    h_bytes = rows * cfg.inter * esz
    flops = 2.0 * rows * cfg.d_latent * 2 * cfg.inter
    return float(w_bytes + a_bytes + h_bytes), flops


def router_fused_splits(cfg) -> int:
    """Number of split-K halves whose partial logits the top-k kernel sums itself (0: the router GEMM
    stores the scores): the library's rule for bf16 router GEMMs whose 256x256 tiles fill between a
    quarter and all of the CUs."""
    if cfg.act_dtype != "bf16":
        return 0
    tiles = -(-cfg.T // 256) * -(-cfg.n_experts // 256)
    if not 64 <= tiles < 256:
        return 0
    K = 3 * cfg.d_model
    for n in range(-(-256 // tiles), 5):
        if K % n == 0 and (K // n) % 64 == 0 and K // n >= 256:
            return n
    return 0


def kernel_work(cfg, offsets, fused: bool = True) -> dict:
    """Algorithmic work of each kernel for one forward: ("mfma", FLOPs) for the contractions,
    ("hbm", bytes) for the rest. GEMM FLOPs count only real rows; routed weights count only the
    experts that received tokens."""
    import numpy as np

    T, D, L, E, k, I = cfg.T, cfg.d_model, cfg.d_latent, cfg.n_experts, cfg.top_k, cfg.inter
    S, Is, NB = cfg.n_shared, cfg.inter_shared, cfg.n_bins
    esz = 2 if cfg.act_dtype == "bf16" else 4
    counts = np.diff(offsets)
    touched = int((counts > 0).sum())
    rows = int(offsets[-1])
    glu_b, _ = glu_bytes(cfg, offsets)
    work = {
        "router_split": ("hbm", E * D * (4 + 6)),
        "gemm_router": ("mfma", (3 if esz == 2 else 1) * 2.0 * T * D * E),
        # algorithmic: the scores [T, E] once, the bias, and idx, w, thresholds written (the split-K
        # partial logits the fused kernel reads are implementation traffic, not counted)
        "route_topk": ("hbm", T * E * 4 + E * 4 + T * k * 8 + T * 8),
        "qb_hist": ("hbm", T * E * 4 + E * 4 + T * 8 + E * NB * 4 * 2),
        "gemm_down": ("mfma", 2.0 * T * D * L),
        "perm_count": ("hbm", T * k * 4),
        "perm_scan": ("hbm", -(-T // 256) * E * 4 * 2 + (E + 1) * 4),
        "perm_scatter": ("hbm", T * k * 12),
        "gemm_glu_grouped": ("hbm", glu_b),
        "gemm_down_grouped": ("hbm", touched * L * I * esz + rows * (I + L) * esz),
        "gemm_glu_dense": ("mfma", 2.0 * T * D * 2 * S * Is),
        "gemm_out_dense": ("mfma", 2.0 * T * S * Is * D),
        "combine_norm": ("hbm", rows * L * esz + T * k * 8 + L * 4 + T * L * esz),
        "gemm_up": ("mfma", 2.0 * T * (L + (S * Is if fused else 0)) * D),
        "qb_update": ("hbm", E * NB * 4 * 2 + E * 8),
    }
    return work


def kernel_roofline(work: dict, kernels_ms: dict) -> dict:
    """Each kernel's achieved rate against the peak of the unit that bounds it."""
    out = {}
    for name, (bound, amount) in work.items():
        ms = kernels_ms.get(name)
        if not ms:
            continue
        if bound == "mfma":
            tf = amount / (ms * 1e-3) / 1e12
            out[name] = {"bound": "mfma", "achieved": round(tf, 1), "unit": "TFLOP/s",
                         "frac": round(tf / BF16_PEAK_TFLOPS, 4)}
        else:
            gbs = amount / (ms * 1e-3) / 1e9
            out[name] = {"bound": "hbm", "achieved": round(gbs, 1), "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def cpu_baseline(cfg, inp, sample_tokens: int) -> dict:
    """The oracle as it stands, on a bounded sample of the same workload (host cores)."""
    import numpy as np

    from oracle import lmoe_oracle as O

    try:
        from threadpoolctl import threadpool_info
        threads = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    sub = dict(inp)
    sub["x"] = inp["x"][:sample_tokens]
    cfg_s = cfg.with_tokens(sample_tokens)
    t0 = time.perf_counter()
    s, idx, w, thr = O.route(sub, cfg_s)
    O.qb_histogram(s, sub["bias"], idx, thr, cfg.n_bins)
    O.permute(idx, cfg.n_experts)
    O.expert_path(sub, cfg_s, idx, w)
    dt = time.perf_counter() - t0
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:  # pragma: no cover
        pass
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": threads, "cpu_model": model, "kind": "oracle",
            "sample": f"first {sample_tokens} tokens of the {cfg.name} batch through the full forward "
                      f"(route, QB histogram, permutation, all touched experts, shared, combine, norm, up): "
                      f"{dt:.1f} s"}


FP8_PEAK_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (the FP8 x FP4 scaled MFMA runs at this rate)
MX_KERNELS = ["mx_quantize", "gemm_glu_mx", "gemm_down_mx"]


def mx_work(cfg, offsets) -> dict:
    """Algorithmic work of the MX routed-expert kernels for one forward: FP4 weight slices (0.5 byte
    per element plus one scale byte per 32) of the experts that received tokens, x_lat's FP8 codes
    and scales read once, h written in bf16, then read as FP8 codes; y written in bf16."""
    import numpy as np

    T, L, k, I = cfg.T, cfg.d_latent, cfg.top_k, cfg.inter
    counts = np.diff(offsets)
    touched = int((counts > 0).sum())
    rows = int(offsets[-1])
    fp4 = lambda n: n / 2 + n / 32  # noqa: E731
    fp8 = lambda n: n + n / 32      # noqa: E731
    return {
        "mx_quantize": ("hbm", 2 * T * L + fp8(T * L) + 2 * rows * I + fp8(rows * I)),
        "gemm_glu_mx": ("hbm", touched * fp4(2 * I * L) + fp8(T * L) + 2 * rows * I,
                        2.0 * rows * L * 2 * I),
        "gemm_down_mx": ("hbm", touched * fp4(L * I) + fp8(rows * I) + 2 * rows * L, 2.0 * rows * I * L),
    }


def mx_steps(cfg, w, xs, args, _lib, torch, LatentMoE, flush) -> dict:
    """Forward steps with the routed experts on MX operands (MXFP4 weights, MXFP8 activations), timed
    like the headline steps."""
    layer = LatentMoE(cfg, w, mx=True, overlap_shared=False if args.one_stream else None)

    def step(i):
        layer.forward(xs[i % 2])
        layer.qb_update()

    for i in range(max(args.warmup, 2)):
        step(i)
    torch.cuda.synchronize()
    t = timed_steps(step, args.steps, flush, torch, _lib, None)
    bd_steps = min(args.steps, 20)  # per-kernel breakdown in a pass of its own, on one stream
    overlap = layer.overlap_shared
    layer.overlap_shared = False
    _lib.profile_reset()
    _lib.profile_enable(True)
    for i in range(bd_steps):
        step(i)
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    _lib.profile_collect()
    layer.overlap_shared = overlap
    kernels, roof = {}, {}
    b = layer.forward(xs[0])
    torch.cuda.synchronize()
    work = mx_work(cfg, b["offsets"].cpu().numpy())
    for n in MX_KERNELS:
        cnt, ms = _lib.profile_get(n)
        if not cnt:
            continue
        kernels[n] = round(ms / bd_steps, 4)
        step_s = ms / bd_steps / 1e3  # the work is per step (the quantize kernel runs twice a step)
        gbs = work[n][1] / step_s / 1e9
        roof[n] = {"bound": "hbm", "achieved": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                   "launches_per_step": round(cnt / bd_steps, 2), "avg_launch_ms": round(ms / cnt, 4)}
        if len(work[n]) > 2:
            tf = work[n][2] / step_s / 1e12
            roof[n].update({"mfma_tflops": round(tf, 1), "mfma_frac_fp8": round(tf / FP8_PEAK_TFLOPS, 4)})
    del layer
    return {"ms_per_step": t["ms_median"], "ms_min": t["ms_min"], "tokens_per_s": cfg.T / (t["ms_median"] / 1e3),
            "kernels_ms_per_step": kernels, "kernels_roofline": roof}


BWD_KERNELS = ["bwd_transpose", "bwd_gemm_dn", "bwd_gemm_dw", "bwd_combine_norm", "bwd_dgamma", "bwd_router_dw",
               "bwd_router_dx", "bwd_gemm_dh", "bwd_gemm_dw_experts", "bwd_gemm_dgu", "bwd_gemm_dx_experts",
               "bwd_unpermute", "bwd_gemm_dx"]


def train_steps(layer, x, cfg, args, _lib, torch) -> dict:
    """Training steps: forward, backward of <dout, out> for a fixed synthetic dout, bias update."""
    g = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn(cfg.T, cfg.d_model, device="cuda", generator=g).to(layer.dt)

    def step():
        b = layer.forward(x)
        layer.backward(x, b, dout)
        layer.qb_update()

    log("[bench] training-step warmup")
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    bd_steps = min(args.steps, 10)  # per-kernel breakdown in a pass of its own
    _lib.profile_reset()
    _lib.profile_enable(True)
    for _ in range(bd_steps):
        step()
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    _lib.profile_collect()
    kernels = {}
    for n in BWD_KERNELS:
        cnt, ms = _lib.profile_get(n)
        if cnt:
            kernels[n] = round(ms / bd_steps, 4)
    ms_step = elapsed / args.steps * 1e3
    return {"ms_per_step": ms_step, "tokens_per_s": cfg.T / (ms_step / 1e3),
            "backward_kernels_ms_per_step": kernels, "backward_kernels_sum_ms": round(sum(kernels.values()), 4)}


def graph_steps(layer, xs, cfg, args, torch, flush) -> dict:
    """The same step (forward + QB update) recorded once as a HIP graph and replayed: the launch
    gaps between the step's kernels go away; the kernels are the same. The graph reads x from one
    buffer, into which the two batches are copied in turn (outside the timed replays)."""
    layer.qb_update()  # close the step of the forward that read the offsets
    xg = xs[0].clone()
    g, _ = layer.capture_step(xg)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    times = []
    for i in range(args.steps):
        xg.copy_(xs[i % len(xs)])
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in times)
    del g
    med = ms[len(ms) // 2]
    return {"ms_per_step": med, "ms_min": ms[0], "tokens_per_s": cfg.T / (med / 1e3)}


def make_flush(torch):
    """A write of 512 MB (twice the 256 MB MALL) that evicts the caches between timed steps."""
    buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    state = {"v": 0}

    def flush():
        state["v"] = (state["v"] + 1) & 0xFF
        buf.fill_(state["v"])
    return flush


def timed_steps(step, n_steps: int, flush, torch, _lib, dominant: str | None) -> dict:
    """n_steps steps, each preceded by a cache flush and bracketed by HIP events on the launch
    stream; the dominant kernel's launches are also bracketed by the library's own events."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_steps)]
    _lib.profile_reset()
    if dominant:
        _lib.profile_only(dominant)
        _lib.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_steps):
        flush()
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    _lib.profile_enable(False)
    _lib.profile_collect()
    _lib.profile_only(None)
    ms = sorted(a.elapsed_time(b) for a, b in evs)
    out = {"ms_median": ms[len(ms) // 2], "ms_min": ms[0], "ms_mean": sum(ms) / len(ms), "wall_s": wall}
    if dominant:
        cnt, tot = _lib.profile_get(dominant)
        out["dominant_avg_ms"] = tot / cnt if cnt else None
    return out


def breakdown(step, n: int, torch, _lib, layer=None) -> dict:
    """Per-kernel milliseconds per step: every kernel between HIP events (a pass of its own). The
    pass runs every kernel on the caller's stream (the layer's side stream off), so that no two of
    the timed kernels overlap."""
    names = ["router_split", "gemm_router", "route_topk", "qb_hist", "gemm_down", "perm_count", "perm_scan",
             "perm_scatter", "gather_rows", "mtile_prefix", "gemm_glu_grouped", "gemm_down_grouped",
             "gemm_glu_dense", "gemm_out_dense", "combine_norm", "gemm_up", "splitk_reduce", "qb_update"]
    overlap = layer.overlap_shared if layer is not None else None
    if layer is not None:
        layer.overlap_shared = False
    _lib.profile_reset()
    _lib.profile_enable(True)
    for i in range(n):
        step(i)
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    _lib.profile_collect()
    if layer is not None:
        layer.overlap_shared = overlap
    out = {}
    for nm in names:
        cnt, ms = _lib.profile_get(nm)
        if cnt:
            out[nm] = round(ms / n, 4)
    return out


def dominant_roofline(cfg, offsets, avg_ms: float) -> dict:
    """The routed experts' GEMM1 + SiTU-GLU against both rooflines; `bound` names the binding one
    (HBM below the ridge intensity, MFMA above it)."""
    bytes_, flops = glu_bytes(cfg, offsets)
    gbs = bytes_ / (avg_ms * 1e-3) / 1e9
    tf = flops / (avg_ms * 1e-3) / 1e12
    intensity = flops / bytes_
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    if intensity < ridge:
        return {"kernel": DOMINANT, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": bytes_, "avg_launch_ms": round(avg_ms, 4),
                "mfma_tflops": round(tf, 1), "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4),
                "intensity_flop_per_byte": round(intensity, 1)}
    return {"kernel": DOMINANT, "bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": flops, "avg_launch_ms": round(avg_ms, 4),
            "hbm_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "intensity_flop_per_byte": round(intensity, 1)}


def k3_weights(cache: dict, torch, upload_weights, make_inputs, K3):
    """The K3-shape weights, drawn and uploaded once for the three K3 workloads."""
    from dataclasses import replace

    if "w" not in cache:
        inp = make_inputs(replace(K3, T=0), with_x=False)
        cache["inp"] = inp
        cache["w"] = upload_weights(inp, K3.act_dtype)
        torch.cuda.synchronize()
    return cache["inp"], cache["w"]


def setup_workload(cfg, cache, torch, np):
    """(host inputs, device weights, two device batches) of a workload; K3 shapes share weights."""
    from latent_space_routed_amd import to_device, upload_weights
    from workloads import CONFIGS
    from workloads.inputs import logit_offsets, make_inputs, token_rows

    if cfg.d_model == CONFIGS["k3_prefill"].d_model:
        inp_w, w = k3_weights(cache, torch, upload_weights, make_inputs, CONFIGS["k3_prefill"])
        inp = dict(inp_w)
        w = dict(w)
        off = logit_offsets(cfg)
        inp["logit_offset"] = off
        w["logit_offset"] = to_device(off, cfg.act_dtype) if off is not None else None
    else:
        inp = make_inputs(cfg, with_x=False)
        w = upload_weights(inp, cfg.act_dtype)
    inp["x"] = token_rows(cfg, 0, 0)
    first = 0 if cfg.qb_updates <= 1 else cfg.qb_updates  # the stress batches after its QB loop
    xs = [to_device(token_rows(cfg, 0, first + b), cfg.act_dtype) for b in range(2)]
    return inp, w, xs


def qb_loop(layer, cfg, torch, np):
    """The QB loop over distinct batches, the bias carried forward (untimed), reporting the load."""
    from latent_space_routed_amd import to_device
    from workloads.inputs import token_rows

    ratios = []
    for bt in range(cfg.qb_updates):
        xb = to_device(token_rows(cfg, 0, bt), cfg.act_dtype)
        counts = np.diff(layer.forward(xb)["offsets"].cpu().numpy())
        ratios.append(round(float(counts.max() / counts.mean()), 3))
        layer.qb_update()
        del xb
    return {"updates": cfg.qb_updates, "max_over_mean_expert_load": ratios,
            "note": "load of each batch's forward, before that batch's bias update"}


def run_workload(cfg, args, cache, flush, torch, np, _lib, headline: bool) -> tuple[dict, object, dict, list]:
    from latent_space_routed_amd import LatentMoE

    log(f"[bench] {cfg.name}: inputs")
    inp, w, xs = setup_workload(cfg, cache, torch, np)
    layer = LatentMoE(cfg, w, overlap_shared=False if args.one_stream else None)
    res = {}
    if cfg.qb_updates > 1:
        log(f"[bench] {cfg.name}: {cfg.qb_updates} QB updates over distinct batches")
        res["qb"] = qb_loop(layer, cfg, torch, np)

    def step(i):
        layer.forward(xs[i % 2])
        layer.qb_update()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] {cfg.name}: {args.steps} timed steps")
    t = timed_steps(step, args.steps, flush, torch, _lib, DOMINANT)
    b = layer.forward(xs[0])
    layer.qb_update()
    torch.cuda.synchronize()
    offsets = b["offsets"].cpu().numpy()
    res.update({"T": cfg.T, "ms_per_step": t["ms_median"], "ms_min": t["ms_min"], "ms_mean": t["ms_mean"],
                "tokens_per_s": cfg.T / (t["ms_median"] / 1e3),
                "roofline": dominant_roofline(cfg, offsets, t["dominant_avg_ms"]) if t["dominant_avg_ms"] else None})
    kernels = breakdown(step, min(args.steps, 20), torch, _lib, layer)
    res["kernels_ms_per_step"] = kernels
    res["kernels_roofline"] = kernel_roofline(kernel_work(cfg, offsets, layer.fused), kernels)
    return res, layer, inp, xs


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="k3_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=2048)
    ap.add_argument("--backward", action="store_true",
                    help="also time training steps (forward + backward + bias update) and report them under 'train'")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the replays of the step recorded as a HIP graph (reported under 'graph')")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the forward steps with MX routed experts (reported under 'mx')")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other workloads (reported under 'configs')")
    ap.add_argument("--one-stream", action="store_true",
                    help="run the shared experts' GEMM1 on the caller's stream too (per-kernel traces: no kernel "
                         "shares the chip with another)")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB 5 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from latent_space_routed_amd import LatentMoE, _lib
    from workloads import CONFIGS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_probe_mb:
        n = args.copy_probe_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 10
        print(json.dumps({"copy_probe_bytes": n, "launches": 15, "ms_per_copy": ms,
                          "read_plus_write_GBs": 2 * n / ms / 1e6}), flush=True)
        return 0
    cfg = CONFIGS[args.workload]
    flush = make_flush(torch)
    cache = {}
    head, layer, inp, xs = run_workload(cfg, args, cache, flush, torch, np, _lib, True)
    roof = dict(head["roofline"])
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_digest") == source_digest() and tr.get("workload") == cfg.name:
            traffic = tr.get("bytes_per_launch")
    roof["traffic"] = traffic
    out = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_min": head["ms_min"],
        "ms_per_step_mean": head["ms_mean"],
        "timing": "median of per-step HIP events; a 512 MB write flushes the MALL before each step, outside "
                  "the events; two batches alternate; the bias update runs every step; the shared experts' "
                  "GEMM1 runs on a second stream up to the routed experts unless --one-stream",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model, "d_latent": cfg.d_latent,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "inter": cfg.inter, "n_shared": cfg.n_shared,
                   "inter_shared": cfg.inter_shared, "n_bins": cfg.n_bins, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "kernels_ms_per_step": head["kernels_ms_per_step"],
        "kernels_note": "a pass of its own after the timed region, every kernel on one stream, HIP events around "
                        "every kernel",
        "kernels_roofline": head["kernels_roofline"],
    }
    if "qb" in head:
        out["qb"] = head["qb"]
    if not args.no_graph:
        log("[bench] graph replays")
        out["graph"] = graph_steps(layer, xs, cfg, args, torch, flush)
    if args.backward:
        out["train"] = train_steps(layer, xs[0], cfg, args, _lib, torch)
    del layer
    torch.cuda.empty_cache()
    if not args.no_mx and cfg.act_dtype == "bf16":
        log("[bench] MX routed experts")
        _, w_mx, _ = setup_workload(cfg, cache, torch, np)
        out["mx"] = mx_steps(cfg, w_mx, xs, args, _lib, torch, LatentMoE, flush)
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {min(args.cpu_sample, cfg.T)} tokens")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_sample, cfg.T))
    if not args.no_configs:
        configs = {}
        for name in ("tiny_f32", "mid_bf16", "k3_decode", "k3_stress"):
            if name == cfg.name:
                continue
            res, lay, _, _ = run_workload(CONFIGS[name], args, cache, flush, torch, np, _lib, False)
            configs[name] = {k: res[k] for k in ("T", "ms_per_step", "ms_min", "tokens_per_s", "roofline")}
            configs[name]["dtype"] = CONFIGS[name].act_dtype
            top = sorted(res["kernels_ms_per_step"].items(), key=lambda kv: -kv[1])[:4]
            configs[name]["top_kernels_ms"] = dict(top)
            if "qb" in res:
                configs[name]["qb"] = res["qb"]
            del lay
            torch.cuda.empty_cache()
        out["configs"] = configs
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
