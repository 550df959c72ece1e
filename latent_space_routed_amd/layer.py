"""Stable LatentMoE layer forward composed from the C-ABI calls (device memory via PyTorch).

Order of the calls ([vxz] 01-02 and [slm] Latent-Space MoE: route, dispatch in latent space, expert
FFNs, combine, norm, up-project, shared experts added):
  lmoe_route -> lmoe_qb_histogram -> lmoe_permute -> lmoe_grouped_situ_glu (routed experts)
  -> lmoe_grouped_situ_glu (shared experts, one group) -> lmoe_combine_norm_up
and, at a step boundary, lmoe_qb_update. Every step runs in the library's kernels; this module only
allocates buffers and passes pointers.

fused=True (default): the routed GEMM reads x_lat rows through sorted_token (no permuted copy), and
the shared experts' down-projection is folded into the up-projection's accumulation (no y_sh).
fused=False materialises x_perm and y_sh, as separate steps.

mx=True (bf16 layers, [slm] 训练基础设施: MXFP4 weights with MXFP8 activations): the routed experts
run on MX operands. W1 and W2 are quantised to MXFP4 once, at construction; each forward quantises
x_lat to MXFP8 (lmoe_mx_quantize) and calls lmoe_grouped_situ_glu_mx, which reads x_lat's codes
through sorted_token and quantises h itself. Everything else is the bf16 layer.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as C

_TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def to_device(a: np.ndarray | None, act_dtype: str, device="cuda") -> torch.Tensor | None:
    """Host array -> device tensor. uint16 arrays are bfloat16 bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


class LatentMoE:
    """One layer instance: weights on the device, per-batch buffers sized for up to ``max_tokens``."""

    def __init__(self, cfg, weights: dict, max_tokens: int | None = None, device: str = "cuda",
                 out_dtype: torch.dtype = torch.float32, fused: bool = True, mx: bool = False,
                 overlap_shared: bool | None = None):
        self.cfg = cfg
        # Fused path with shared experts: their GEMM1 depends on x alone, so it can run on a side
        # stream forked at the start of the step, beside the router, top-k, histogram,
        # down-projection and permutation, whose small kernels and the down-projection's last
        # partial round of tiles leave CUs idle; the caller's stream waits for it before the routed
        # GEMMs (joining later, before the up-projection, measured 0.01 ms slower at K3 prefill and
        # 0.2 ms slower at 32768 tokens). Outputs are bit-identical either way. Measured (one
        # process, on and off alternating): K3 prefill 4.47-4.48 ms per step against 4.52; K3
        # decode 1.89 against 1.91; the tiny f32 workload 0.112-0.120 against 0.108,
        # where the fork and join cost more than the overlap gives; with MX routed experts at K3
        # prefill 3.64-3.65 against 3.66-3.67; K3 dimensions at 32768 tokens 16.79-16.87 against
        # 16.29-16.32, where the longer shared GEMM still runs when the routed GEMMs start. Forking
        # after the route or after the permutation instead makes the routed GEMMs share the chip
        # (slower). None (the default) turns it on when the shared GEMM1 of the batch is at least
        # 1 GFLOP and the batch holds at most 16384 tokens.
        self.overlap_shared = overlap_shared
        self._side = None
        if mx and (cfg.act_dtype != "bf16" or not fused):
            raise ValueError("MX experts need a bf16 layer on the fused path")
        self.mx = mx
        self.out_dtype = out_dtype
        self.fused = fused
        self.device = device
        self.max_tokens = cfg.T if max_tokens is None else max_tokens
        self.w = weights
        dt = _TORCH_DT[cfg.act_dtype]
        self.dt = dt
        E, NB, D, S, Is = cfg.n_experts, cfg.n_bins, cfg.d_model, cfg.n_shared, cfg.inter_shared
        self.bias = weights["bias"].clone()
        self.hist = torch.zeros(E, NB, dtype=torch.int32, device=device)
        self.n_acc = 0
        shape = C.make_shape(cfg, self.max_tokens)
        self.w1s_packed = torch.empty(2 * S * Is, D, dtype=dt, device=device)
        self.w2s_packed = torch.empty(D, S * Is, dtype=dt, device=device)
        if S > 0:
            C.lmoe_pack_shared(shape, weights["w1s"], weights["w2s"], self.w1s_packed, self.w2s_packed)
        # bf16 layers: the router weights split into three bf16 parts once, not per forward
        self.w_router_split = None
        if cfg.act_dtype == "bf16":
            self.w_router_split = torch.empty(E, 3 * D, dtype=torch.bfloat16, device=device)
            C.lmoe_split_router(shape, weights["w_router"], self.w_router_split)
        if mx:
            self.mx_w = {}
            for name in ("w1", "w2"):
                wt = weights[name]
                G, R, K = wt.shape
                codes = torch.empty(G, R, K // 2, dtype=torch.uint8, device=device)
                scales = torch.empty(G, R, K // 32, dtype=torch.uint8, device=device)
                C.lmoe_mx_quantize(shape, C.LMOE_MX_FP4, G * R, K, wt, codes, scales)
                self.mx_w[name] = (codes, scales)
        self._bufs = {}
        self._alloc(self.max_tokens)

    # -------------------------------------------------------------------------------------------
    def _alloc(self, T: int) -> None:
        cfg, dev, dt = self.cfg, self.device, self.dt
        E, k, L, D, I = cfg.n_experts, cfg.top_k, cfg.d_latent, cfg.d_model, cfg.inter
        S, Is = cfg.n_shared, cfg.inter_shared
        shape = C.make_shape(cfg, T)
        f32, i32 = torch.float32, torch.int32
        b = {
            "scores": torch.empty(T, E, dtype=f32, device=dev),
            "idx": torch.empty(T, k, dtype=i32, device=dev),
            "w": torch.empty(T, k, dtype=f32, device=dev),
            "thresh": torch.empty(T, 2, dtype=f32, device=dev),
            "x_lat": torch.empty(T, L, dtype=dt, device=dev),
            "offsets": torch.empty(E + 1, dtype=i32, device=dev),
            "sorted_token": torch.empty(T * k, dtype=i32, device=dev),
            "slot_of_pair": torch.empty(T * k, dtype=i32, device=dev),
            "x_perm": torch.empty(0 if self.fused else T * k, L, dtype=dt, device=dev),
            "h": torch.empty(T * k, I, dtype=dt, device=dev),
            "y": torch.empty(T * k, L, dtype=dt, device=dev),
            "h_s": torch.empty(T, max(S * Is, 64), dtype=dt, device=dev),
            "y_sh": torch.empty(0 if self.fused else T, D, dtype=f32, device=dev),
            "n": torch.empty(T, L, dtype=dt, device=dev),
            "out": torch.empty(T, D, dtype=self.out_dtype, device=dev),
        }
        if self.mx:
            b["x_lat_codes"] = torch.empty(T, L, dtype=torch.uint8, device=dev)
            b["x_lat_scales"] = torch.empty(T, L // 32, dtype=torch.uint8, device=dev)
            n = C.workspace_bytes(shape, C.LMOE_CALL_GROUPED_GLU_MX)
            b["ws_glu_mx"] = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        for name, which in (("ws_route", C.LMOE_CALL_ROUTE), ("ws_permute", C.LMOE_CALL_PERMUTE),
                            ("ws_glu", C.LMOE_CALL_GROUPED_GLU), ("ws_combine", C.LMOE_CALL_COMBINE_NORM_UP)):
            n = C.workspace_bytes(shape, which)
            b[name] = torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        if self.fused and S > 0 and self._side is None:
            # created whether or not overlap_shared is set, so the flag can change between steps; the
            # side stream's shared GEMM1 uses the grouped-GLU workspace, which the routed GEMMs use
            # only after the join
            self._side = torch.cuda.Stream(device=dev)
        self._bufs = b

    def _overlapped(self, T: int) -> bool:
        cfg = self.cfg
        if not (self.fused and cfg.n_shared > 0) or self.overlap_shared is False:
            return False
        if self.overlap_shared:
            return True
        return T <= 16384 and 4.0 * T * cfg.d_model * cfg.n_shared * cfg.inter_shared >= 1e9

    # -------------------------------------------------------------------------------------------
    def forward(self, x: torch.Tensor, accumulate_hist: bool = True) -> dict:
        """One forward pass over x [T, D]; returns the buffers (views of the first T tokens)."""
        cfg, w = self.cfg, self.w
        T = x.shape[0]
        if T > self.max_tokens:
            self.max_tokens = T
            self._alloc(T)
        b = {k: (v[:T] if k in ("scores", "idx", "w", "thresh", "x_lat", "h_s", "n", "out", "x_lat_codes",
                                "x_lat_scales") else v)
             for k, v in self._bufs.items()}
        b["y_sh"] = self._bufs["y_sh"][:T] if not self.fused else None
        for k in ("sorted_token", "slot_of_pair"):
            b[k] = self._bufs[k][: T * cfg.top_k]
        for k in ("h", "y"):
            b[k] = self._bufs[k][: T * cfg.top_k]
        b["x_perm"] = self._bufs["x_perm"][: T * cfg.top_k] if not self.fused else None
        shape = C.make_shape(cfg, T)
        E, k, L, D, I = cfg.n_experts, cfg.top_k, cfg.d_latent, cfg.d_model, cfg.inter
        S, Is = cfg.n_shared, cfg.inter_shared
        side = self._side if self._overlapped(T) else None
        if side is not None:
            cur = torch.cuda.current_stream()
            side.wait_stream(cur)
            with torch.cuda.stream(side):
                C.lmoe_grouped_situ_glu(shape, 1, T, D, S * Is, D, x, None, self.w1s_packed, None, b["h_s"], None,
                                        b["ws_glu"])
        C.lmoe_route(shape, x, w["w_router"], self.bias, w.get("logit_offset"), b["scores"], b["idx"], b["w"],
                     b["thresh"], b["ws_route"], w_router_split=self.w_router_split)
        if accumulate_hist:
            C.lmoe_qb_histogram(shape, b["scores"], self.bias, b["idx"], b["thresh"], self.hist)
            self.n_acc += T
        fused = self.fused
        C.lmoe_permute(shape, x, w["w_down"], b["idx"], b["x_lat"], b["offsets"], b["sorted_token"],
                       b["slot_of_pair"], None if fused else b["x_perm"], b["ws_permute"])
        if side is not None:
            cur.wait_stream(side)  # h_s is ready, and the routed GEMMs have the chip to themselves
        if self.mx:
            C.lmoe_mx_quantize(shape, C.LMOE_MX_FP8, T, L, b["x_lat"], b["x_lat_codes"], b["x_lat_scales"])
            (w1c, w1s), (w2c, w2s) = self.mx_w["w1"], self.mx_w["w2"]
            C.lmoe_grouped_situ_glu_mx(shape, E, T * k, L, I, L, b["x_lat_codes"], b["x_lat_scales"], T,
                                       b["sorted_token"], b["offsets"], w1c, w1s, w2c, w2s, b["h"], b["y"],
                                       b["ws_glu_mx"])
        elif fused:
            C.lmoe_grouped_situ_glu(shape, E, T * k, L, I, L, b["x_lat"], b["offsets"], w["w1"], w["w2"], b["h"],
                                    b["y"], b["ws_glu"], a_row_index=b["sorted_token"])
        else:
            C.lmoe_grouped_situ_glu(shape, E, T * k, L, I, L, b["x_perm"], b["offsets"], w["w1"], w["w2"], b["h"],
                                    b["y"], b["ws_glu"])
        if S > 0 and fused:
            if side is None:
                C.lmoe_grouped_situ_glu(shape, 1, T, D, S * Is, D, x, None, self.w1s_packed, None, b["h_s"], None,
                                        b["ws_glu"])
            C.lmoe_combine_norm_up(shape, b["y"], b["slot_of_pair"], b["w"], w.get("gamma"), w["w_up"], None,
                                   b["n"], b["out"], h_shared=b["h_s"], w2_shared=self.w2s_packed,
                                   workspace=b["ws_combine"])
        elif S > 0:
            C.lmoe_grouped_situ_glu(shape, 1, T, D, S * Is, D, x, None, self.w1s_packed, self.w2s_packed,
                                    b["h_s"], b["y_sh"], b["ws_glu"])
            C.lmoe_combine_norm_up(shape, b["y"], b["slot_of_pair"], b["w"], w.get("gamma"), w["w_up"], b["y_sh"],
                                   b["n"], b["out"], workspace=b["ws_combine"])
        else:
            C.lmoe_combine_norm_up(shape, b["y"], b["slot_of_pair"], b["w"], w.get("gamma"), w["w_up"], None,
                                   b["n"], b["out"], workspace=b["ws_combine"])
        return b

    # -------------------------------------------------------------------------------------------
    def backward(self, x: torch.Tensor, b: dict, dout: torch.Tensor) -> dict:
        """Gradients of <dout, out> for the batch whose forward buffers are ``b`` (from forward(x)).

        dout [T, D] in the activation type. Returns activation and weight gradients (weight
        gradients, dgamma, dlogit and dx in f32; the shared experts' in their packed layout).
        Calls, in order: transposed weights, up-projection, combine + norm + routing weights, router,
        routed experts, un-permutation + down-projection, shared experts.
        """
        if self.mx:
            raise NotImplementedError("the backward calls take bf16/f32 expert weights, not MX ones")
        cfg, w, dev, dt = self.cfg, self.w, self.device, self.dt
        T = x.shape[0]
        E, k, L, D, I = cfg.n_experts, cfg.top_k, cfg.d_latent, cfg.d_model, cfg.inter
        S, Is = cfg.n_shared, cfg.inter_shared
        Ss = S * Is
        shape = C.make_shape(cfg, T)
        f32 = torch.float32
        if getattr(self, "_wt", None) is None:
            self._wt = {
                "w_up_t": torch.empty(L, D, dtype=dt, device=dev),
                "w_down_t": torch.empty(D, L, dtype=dt, device=dev),
                "w2s_t": torch.empty(max(Ss, 1), D, dtype=dt, device=dev),
                "w1s_t": torch.empty(D, max(2 * Ss, 1), dtype=dt, device=dev),
            }
        wt = self._wt
        shared = S > 0
        C.lmoe_bwd_transpose_weights(shape, w["w_up"], self.w2s_packed if shared else None,
                                     self.w1s_packed if shared else None, w["w_down"], wt["w_up_t"],
                                     wt["w2s_t"] if shared else None, wt["w1s_t"] if shared else None, wt["w_down_t"])
        ws = {name: torch.empty(max(C.workspace_bytes(shape, which), 256), dtype=torch.uint8, device=dev)
              for name, which in (("up", C.LMOE_CALL_BWD_UP), ("comb", C.LMOE_CALL_BWD_COMBINE_NORM),
                                  ("exp", C.LMOE_CALL_BWD_EXPERTS), ("down", C.LMOE_CALL_BWD_DOWN),
                                  ("sh", C.LMOE_CALL_BWD_SHARED))}
        g = {
            "dn": torch.empty(T, L, dtype=dt, device=dev),
            "dh_s": torch.empty(T, max(Ss, 64), dtype=dt, device=dev),
            "dW_up": torch.empty(D, L, dtype=f32, device=dev),
            "dW2s_packed": torch.empty(D, max(Ss, 1), dtype=f32, device=dev),
            "dy": torch.empty(T * k, L, dtype=dt, device=dev),
            "dl": torch.empty(T, k, dtype=f32, device=dev),
            "dl_sorted": torch.empty(T * k, dtype=f32, device=dev),
            "dgamma": torch.empty(L, dtype=f32, device=dev),
            "dW_r": torch.empty(E, D, dtype=f32, device=dev),
            "dx": torch.empty(T, D, dtype=f32, device=dev),
            "dh": torch.empty(T * k, I, dtype=dt, device=dev),
            "dgu": torch.empty(T * k, 2 * I, dtype=dt, device=dev),
            "dx_perm": torch.empty(T * k, L, dtype=dt, device=dev),
            "dW1": torch.empty(E, 2 * I, L, dtype=f32, device=dev),
            "dW2": torch.empty(E, L, I, dtype=f32, device=dev),
            "dx_lat": torch.empty(T, L, dtype=dt, device=dev),
            "dW_dn": torch.empty(L, D, dtype=f32, device=dev),
            "dgu_s": torch.empty(T, max(2 * Ss, 64), dtype=dt, device=dev),
            "dW1s_packed": torch.empty(max(2 * Ss, 1), D, dtype=f32, device=dev),
        }
        C.lmoe_bwd_up(shape, dout, b["n"], b["h_s"] if shared else None, wt["w_up_t"], wt["w2s_t"] if shared else None,
                      g["dn"], g["dh_s"] if shared else None, g["dW_up"], g["dW2s_packed"] if shared else None, ws["up"])
        C.lmoe_bwd_combine_norm(shape, g["dn"], b["y"], b["slot_of_pair"], b["idx"], b["scores"], b["w"],
                                w.get("gamma"), g["dy"], g["dl"], g["dl_sorted"], g["dgamma"], ws["comb"])
        C.lmoe_bwd_router(shape, x, w["w_router"], g["dl"], g["dl_sorted"], b["idx"], b["offsets"], b["sorted_token"],
                          g["dW_r"], g["dx"])
        C.lmoe_bwd_experts(shape, b["x_lat"], b["sorted_token"], b["offsets"], w["w1"], w["w2"], b["h"], g["dy"],
                           g["dh"], g["dgu"], g["dx_perm"], g["dW1"], g["dW2"], ws["exp"])
        C.lmoe_bwd_down(shape, x, g["dx_perm"], b["slot_of_pair"], wt["w_down_t"], g["dx_lat"], g["dW_dn"], g["dx"],
                        ws["down"])
        if shared:
            C.lmoe_bwd_shared(shape, x, self.w1s_packed, wt["w1s_t"], g["dh_s"], g["dgu_s"], g["dW1s_packed"], g["dx"],
                              ws["sh"])
        return g

    def qb_update(self) -> None:
        """Move the selection bias from the accumulated histogram and reset it (a step boundary)."""
        C.lmoe_qb_update(C.make_shape(self.cfg, 0), self.hist, self.n_acc, self.bias)
        self.n_acc = 0

    def capture_step(self, x: torch.Tensor) -> tuple[torch.cuda.CUDAGraph, dict]:
        """Record one step, forward(x) then the QB update, as a HIP graph to replay.

        Every call of the step only enqueues kernels (no host synchronisation, no allocation, no
        memset), so the graph holds the same launches in the same order; a replay recomputes the
        returned buffers from the current contents of x and moves the bias like an eager step. x
        and the layer's buffers must stay where they are while the graph is in use. The histogram
        must be empty at capture (call qb_update first), since each replay updates from one batch.
        """
        if self.n_acc != 0:
            raise RuntimeError("capture_step needs an empty histogram: call qb_update() first")
        if x.shape[0] > self.max_tokens:
            self.max_tokens = x.shape[0]
            self._alloc(x.shape[0])
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            b = self.forward(x)
            self.qb_update()
        return g, b


def upload_weights(inp: dict, act_dtype: str, device: str = "cuda") -> dict:
    """The seeded host inputs (see workloads.inputs) as device tensors."""
    out = {}
    for name, a in inp.items():
        if name == "x":
            continue
        out[name] = to_device(a, act_dtype, device)
    return out
