"""Benchmark: tokens/s of one Stable LatentMoE layer forward at K3 shape on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic tokens: route (router GEMM,
top-k), QB histogram, down-projection + permutation, routed grouped SiTU-GLU FFNs, shared experts,
combine + RMSNorm + up-projection, and the QB bias update. Inputs are resident in HBM before the
timed region. Prints ONE JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload k3_prefill] [--no-cpu-baseline]
                  [--backward] [--no-mx]

The headline line is the bf16 layer, stepped eagerly. Under "graph" the same step is replayed from a
HIP graph (same kernels, no launch gaps). Under "mx" the same steps are timed with the routed experts
on MXFP4 weights and MXFP8 activations (a variant with its own numerics, never the headline value).
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
        # fused: n partial logit matrices read and the scores written; else the scores read
        "route_topk": ("hbm", (router_fused_splits(cfg) + 1 if router_fused_splits(cfg) else 1) * T * E * 4
                       + E * 4 + T * k * 8 + T * 8),
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
    return {"value": sample_tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
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


def mx_steps(cfg, w, x, args, _lib, torch, LatentMoE) -> dict:
    """Forward steps with the routed experts on MX operands (MXFP4 weights, MXFP8 activations)."""
    layer = LatentMoE(cfg, w, mx=True)

    def step():
        layer.forward(x)
        layer.qb_update()

    for _ in range(max(args.warmup, 2)):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    bd_steps = min(args.steps, 20)  # per-kernel breakdown in a pass of its own
    _lib.profile_reset()
    _lib.profile_enable(True)
    for _ in range(bd_steps):
        step()
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    _lib.profile_collect()
    kernels, roof = {}, {}
    b = layer.forward(x)
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
    ms_step = elapsed / args.steps * 1e3
    del layer
    return {"ms_per_step": ms_step, "tokens_per_s": cfg.T / (ms_step / 1e3), "kernels_ms_per_step": kernels,
            "kernels_roofline": roof}


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


def graph_steps(layer, x, cfg, args, torch) -> dict:
    """The same step (forward + QB update) recorded once as a HIP graph and replayed: the launch
    gaps between the step's kernels go away; the kernels are the same."""
    layer.qb_update()  # close the step of the forward that read the offsets
    g, _ = layer.capture_step(x)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        g.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    del g
    return {"ms_per_step": ms, "tokens_per_s": cfg.T / (ms / 1e3)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="k3_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=2048)
    ap.add_argument("--backward", action="store_true",
                    help="also time training steps (forward + backward + bias update) and report them under 'train'")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the replays of the step recorded as a HIP graph (reported under 'graph')")
    ap.add_argument("--no-mx", action="store_true",
                    help="skip the forward steps with MX routed experts (reported under 'mx')")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB 5 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from latent_space_routed_amd import LatentMoE, _lib, to_device, upload_weights
    from workloads import CONFIGS
    from workloads.inputs import make_inputs

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
    log(f"[bench] generating {cfg.name} inputs")
    t0 = time.perf_counter()
    inp = make_inputs(cfg)
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    w = upload_weights(inp, cfg.act_dtype)
    x = to_device(inp["x"], cfg.act_dtype)
    layer = LatentMoE(cfg, w)
    torch.cuda.synchronize()

    def step():
        layer.forward(x)
        layer.qb_update()

    qb_report = None
    if cfg.qb_updates > 1:  # the QB loop over distinct batches, the bias carried forward (untimed)
        from workloads.inputs import token_rows

        log(f"[bench] {cfg.qb_updates} QB updates over batches 0..{cfg.qb_updates - 1}")
        ratios = []
        for bt in range(cfg.qb_updates):
            xb = x if bt == 0 else to_device(token_rows(cfg, 0, bt), cfg.act_dtype)
            counts = np.diff(layer.forward(xb)["offsets"].cpu().numpy())
            ratios.append(round(float(counts.max() / counts.mean()), 3))
            layer.qb_update()
            del xb
        qb_report = {"updates": cfg.qb_updates, "max_over_mean_expert_load": ratios,
                     "note": "load of each batch's forward, before that batch's bias update"}

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: HIP events bracket the dominant kernel only (events around every kernel add
    # ~0.14 ms to a K3 step); the per-kernel breakdown comes from a second pass below.
    _lib.profile_reset()
    _lib.profile_only(DOMINANT)
    _lib.profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    _lib.profile_enable(False)
    _lib.profile_collect()
    _lib.profile_only(None)
    log(f"[bench] timed {args.steps} steps in {elapsed:.3f} s")
    cnt, ms = _lib.profile_get(DOMINANT)
    avg_s = ms / cnt / 1e3

    bd_steps = min(args.steps, 20)  # breakdown pass: every kernel between HIP events
    _lib.profile_reset()
    _lib.profile_enable(True)
    for _ in range(bd_steps):
        step()
    torch.cuda.synchronize()
    _lib.profile_enable(False)
    _lib.profile_collect()

    names = ["router_split", "gemm_router", "route_topk", "qb_hist", "gemm_down", "perm_count", "perm_scan",
             "perm_scatter", "gather_rows", "mtile_prefix", "gemm_glu_grouped", "gemm_down_grouped",
             "gemm_glu_dense", "gemm_out_dense", "combine_norm", "gemm_up", "splitk_reduce", "qb_update"]
    kernels = {}
    for n in names:
        cnt, ms = _lib.profile_get(n)
        if cnt:
            kernels[n] = round(ms / bd_steps, 4)
    b = layer.forward(x)
    torch.cuda.synchronize()
    offsets = b["offsets"].cpu().numpy()
    bytes_, flops = glu_bytes(cfg, offsets)
    achieved = bytes_ / avg_s / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_digest") == source_digest() and tr.get("workload") == cfg.name:
            traffic = tr.get("bytes_per_launch")

    ms_per_step = elapsed / args.steps * 1e3
    out = {
        "metric": METRIC,
        "value": cfg.T * args.steps / elapsed,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.act_dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d_model": cfg.d_model, "d_latent": cfg.d_latent,
                   "n_experts": cfg.n_experts, "top_k": cfg.top_k, "inter": cfg.inter, "n_shared": cfg.n_shared,
                   "inter_shared": cfg.inter_shared, "n_bins": cfg.n_bins, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": DOMINANT, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": bytes_, "avg_launch_ms": round(avg_s * 1e3, 4),
                     "mfma_tflops": round(flops / avg_s / 1e12, 1),
                     "mfma_frac": round(flops / avg_s / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "kernels_ms_per_step": kernels,
        "kernels_note": f"a pass of {bd_steps} steps after the timed region, HIP events around every kernel",
        "kernels_roofline": kernel_roofline(kernel_work(cfg, offsets, layer.fused), kernels),
    }
    if qb_report:
        out["qb"] = qb_report
    if not args.no_graph:
        log("[bench] graph replays")
        out["graph"] = graph_steps(layer, x, cfg, args, torch)
    if args.backward:
        out["train"] = train_steps(layer, x, cfg, args, _lib, torch)
    if not args.no_mx and cfg.act_dtype == "bf16":
        log("[bench] MX routed experts")
        out["mx"] = mx_steps(cfg, w, x, args, _lib, torch, LatentMoE)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle on {min(args.cpu_sample, cfg.T)} tokens")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_sample, cfg.T))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
