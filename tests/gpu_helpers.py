"""Helpers shared by the GPU parity tests: uploading the seeded inputs and comparing with the oracle."""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

from latent_space_routed_amd import LatentMoE, to_device, upload_weights
from oracle import lmoe_oracle as O
from workloads.inputs import make_inputs

NEAR_TIE_GAP = 1e-5      # fp32 gap between the k-th and (k+1)-th biased score (tie window)
OUT_TOL = {"bf16": 2e-2, "f32": 1e-4}   # max |out - oracle| / RMS(oracle)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 values exactly), int tensors unchanged."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float32):
        return t.float().numpy().astype(np.float64)
    return t.numpy()


@functools.lru_cache(maxsize=4)
def cached_inputs(cfg, seed: int = 0, batch: int = 0, gain_bias: bool = False):
    return make_inputs(cfg, seed=seed, batch=batch, gain_bias=gain_bias)


def device_layer(cfg, inp: dict, max_tokens=None, fused: bool = True) -> tuple[LatentMoE, torch.Tensor]:
    w = upload_weights(inp, cfg.act_dtype)
    layer = LatentMoE(cfg, w, max_tokens=max_tokens, fused=fused)
    x = to_device(inp["x"], cfg.act_dtype)
    return layer, x


def near_ties(thresh: np.ndarray) -> np.ndarray:
    return (thresh[:, 0].astype(np.float64) - thresh[:, 1].astype(np.float64)) < NEAR_TIE_GAP


def assert_close_rows(got: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> float:
    """Elementwise check of a stored tensor: one rounding step of the storage type plus f32
    accumulation noise relative to the tensor's RMS. Returns the max error over the RMS."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) or 1.0
    rel = 2.0 ** -7 if dtype == "bf16" else 2.0 ** -20
    tol = rel * np.abs(ref) + (1e-3 if dtype == "bf16" else 1e-5) * rms
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} of {bad.size} elements off; worst {err.max():.3g} (rms {rms:.3g})"
    return float(err.max() / rms)


def assert_out_parity(out_gpu: np.ndarray, out_pre: np.ndarray, dtype: str, what: str, mask=None) -> float:
    """Layer output within the stated tolerance of the oracle's value before its final rounding."""
    if mask is not None:
        out_gpu, out_pre = out_gpu[mask], out_pre[mask]
    rms = float(np.sqrt(np.mean(out_pre ** 2)))
    err = float(np.max(np.abs(out_gpu - out_pre))) if out_gpu.size else 0.0
    say(f"{what}: max|err|/RMS = {err / rms:.3e} (tol {OUT_TOL[dtype]:.0e}), max|out| = {np.abs(out_pre).max():.3f}")
    assert err <= OUT_TOL[dtype] * rms, f"{what}: max err {err:.4g} > {OUT_TOL[dtype]} * RMS {rms:.4g}"
    return err / rms
