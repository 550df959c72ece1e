"""Seeded synthetic inputs for the Stable LatentMoE layer (shared by the oracle side and the GPU side).

This module only draws random numbers and stores them in the layer's storage types; it holds none
of the method's arithmetic. Recipe (the pages publish no dataset and no trained weights):

* every tensor has its own stream ``PCG64(SeedSequence([seed, tensor_id, sub_id, ...]))``; per-expert
  tensors use the expert index as ``sub_id`` so a consumer may regenerate one expert alone, and the
  token matrix is drawn in fixed 256-row chunks so the result does not depend on thread count;
* x ~ N(0, 1); every weight W ~ N(0, 1/fan_in) with fan_in the matrix's input dimension;
* the router weight, bias, logit offsets and gamma are float32; everything else is stored as
  bfloat16 (round-to-nearest-even of the float32 draw, kept as uint16 bit patterns) or float32
  for ``act_dtype == "f32"``;
* bias b = 0 and gamma = 1 at the start, or, with ``gain_bias=True`` (parity tests of the gain and
  of a moved bias), gamma = 1 + 0.5 N(0, 1) and b = 0.05 N(0, 1), each from its own stream;
* optional skew: logit offsets o_e = -s * ln(r_e) with r a seeded permutation of 1..E (a Zipf(s)
  preference over experts);
* optional outliers: a Bernoulli(frac) mask of x entries multiplied by ``outlier_scale`` before
  the cast to the storage type.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import LayerConfig

TID_X, TID_WR, TID_WDN, TID_W1, TID_W2, TID_WUP, TID_W1S, TID_W2S, TID_ZIPF, TID_OUTLIER, TID_GAMMA, TID_BIAS = range(12)
X_CHUNK_ROWS = 256


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store(a32: np.ndarray, act_dtype: str) -> np.ndarray:
    if act_dtype == "bf16":
        return f32_to_bf16_bits(a32)
    if act_dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(act_dtype)


def _normal(shape, std: float, *key: int) -> np.ndarray:
    a = _rng(*key).standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def _weight(shape, fan_in: int, act_dtype: str, seed: int, tid: int, sub: int = 0) -> np.ndarray:
    return _store(_normal(shape, 1.0 / np.sqrt(fan_in), seed, tid, sub), act_dtype)


def token_rows(cfg: LayerConfig, seed: int = 0, batch: int = 0, rows: slice | None = None) -> np.ndarray:
    """x [T, D] in the storage type (or a row range of it, drawn chunk by chunk identically)."""
    T, D = cfg.T, cfg.d_model
    r0, r1 = (0, T) if rows is None else (rows.start or 0, T if rows.stop is None else rows.stop)
    c0, c1 = r0 // X_CHUNK_ROWS, (r1 + X_CHUNK_ROWS - 1) // X_CHUNK_ROWS

    def chunk(c: int) -> np.ndarray:
        n = min(X_CHUNK_ROWS, T - c * X_CHUNK_ROWS)
        a = _normal((n, D), 1.0, seed, TID_X, batch, c)
        if cfg.outlier_frac > 0.0:
            mask = _rng(seed, TID_OUTLIER, batch, c).random((n, D), dtype=np.float32) < np.float32(cfg.outlier_frac)
            a[mask] *= np.float32(cfg.outlier_scale)
        return _store(a, cfg.act_dtype)

    with ThreadPoolExecutor(_threads()) as ex:
        parts = list(ex.map(chunk, range(c0, c1)))
    full = np.concatenate(parts, axis=0)
    off = r0 - c0 * X_CHUNK_ROWS
    return np.ascontiguousarray(full[off: off + (r1 - r0)])


def expert_weights(cfg: LayerConfig, e: int, seed: int = 0):
    """(w1_e [2I, L], w2_e [L, I]) of routed expert e: gate rows 0..I-1, up rows I..2I-1."""
    L, I = cfg.d_latent, cfg.inter
    return (_weight((2 * I, L), L, cfg.act_dtype, seed, TID_W1, e),
            _weight((L, I), I, cfg.act_dtype, seed, TID_W2, e))


def logit_offsets(cfg: LayerConfig, seed: int = 0) -> np.ndarray | None:
    if cfg.zipf_s <= 0.0:
        return None
    r = _rng(seed, TID_ZIPF).permutation(cfg.n_experts).astype(np.float64) + 1.0
    return (-cfg.zipf_s * np.log(r)).astype(np.float32)


def gain_and_bias(cfg: LayerConfig, seed: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """A non-unit RMSNorm gain gamma = 1 + 0.5 N(0, 1) [L] and a selection bias b = 0.05 N(0, 1) [E],
    both float32, for tests that exercise the gain and a bias moved away from zero."""
    gamma = (1.0 + 0.5 * _normal((cfg.d_latent,), 1.0, seed, TID_GAMMA)).astype(np.float32)
    bias = (0.05 * _normal((cfg.n_experts,), 1.0, seed, TID_BIAS)).astype(np.float32)
    return gamma, bias


def make_inputs(cfg: LayerConfig, seed: int = 0, batch: int = 0, with_x: bool = True, gain_bias: bool = False) -> dict:
    """All tensors of one layer instance as host arrays (bf16 as uint16 bit patterns)."""
    T, D, L, E, I = cfg.T, cfg.d_model, cfg.d_latent, cfg.n_experts, cfg.inter
    S, Is, dt = cfg.n_shared, cfg.inter_shared, cfg.act_dtype
    edt = np.uint16 if dt == "bf16" else np.float32
    w1 = np.empty((E, 2 * I, L), dtype=edt)
    w2 = np.empty((E, L, I), dtype=edt)

    def fill(e: int) -> None:
        w1[e], w2[e] = expert_weights(cfg, e, seed)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(E)))
    out = {
        "w_router": _normal((E, D), 1.0 / np.sqrt(D), seed, TID_WR),
        "bias": np.zeros(E, dtype=np.float32),
        "logit_offset": logit_offsets(cfg, seed),
        "w_down": _weight((L, D), D, dt, seed, TID_WDN),
        "w1": w1,
        "w2": w2,
        "gamma": np.ones(L, dtype=np.float32),
        "w_up": _weight((D, L), L, dt, seed, TID_WUP),
        "w1s": np.stack([_weight((2 * Is, D), D, dt, seed, TID_W1S, j) for j in range(S)]),
        "w2s": np.stack([_weight((D, Is), Is, dt, seed, TID_W2S, j) for j in range(S)]),
    }
    if gain_bias:
        out["gamma"], out["bias"] = gain_and_bias(cfg, seed)
    if with_x:
        out["x"] = token_rows(cfg, seed, batch)
    return out
