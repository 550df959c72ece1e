"""CPU oracle for the MX-format routed experts (MXFP4 weights, MXFP8 activations).

TEST INFRASTRUCTURE ONLY, like lmoe_oracle: only the test suite, the package's smoke check and the
benchmark's CPU-baseline leg may import it. NumPy only; it shares no code with the GPU kernels.

[slm] 训练基础设施 names MXFP4 weights with MXFP8 activations for the experts (quantisation-aware
training from SFT on); the pages give no format details. The formats are the public OCP
Microscaling (MX) ones, read here as:

  RM1 a block is 32 consecutive elements along the contraction dimension (the row of a weight
      [out, in] or of an activation [token, features]); it shares one E8M0 scale X = 2^(e - 127),
      e in 0..254 (stored as the byte e).
  RM2 the shared exponent is floor(log2(max |v| over the block)) - emax, emax = 2 for FP4 (E2M1,
      largest normal 6 = 1.5 * 2^2) and 8 for FP8 (E4M3, largest normal 448 = 1.75 * 2^8), clamped
      to [-127, 127]; an all-zero block takes e = 0.
  RM3 each element is v / X rounded to the nearest value of the element format, ties to the even
      significand, and saturated to the largest normal (+-6 for E2M1, +-448 for E4M3).
  RM4 FP4 elements are packed two per byte, the even-indexed element in the low nibble; FP8
      elements are one byte each; NaN encodings are never produced.
  RM5 a product of an MX activation row and an MX weight row is the sum over k of
      (X_a p_a)(X_w p_w), evaluated exactly here (float64).
  RM6 in the routed experts both projections take MX operands: the expert's input rows (x_lat,
      stored bf16) and its hidden h (stored bf16 after SiTU-GLU) are quantised to MXFP8 along the
      contraction, W1 and W2 are MXFP4 along theirs; everything else is the bf16 expert.
"""
from __future__ import annotations

import numpy as np

from . import lmoe_oracle as O

F64 = np.float64
BLOCK = 32

# representable magnitudes, indexed by the 3 (E2M1) / 7 (E4M3) magnitude bits
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e4m3_mag_table() -> np.ndarray:
    mags = np.empty(128)
    for code in range(128):
        e, m = code >> 3, code & 7
        mags[code] = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return mags


E4M3_MAG = _e4m3_mag_table()            # code 127 (e = 15, m = 7) is NaN in the format: never produced
E4M3_MAX_CODE = 126                      # 448
FORMATS = {"fp4": (E2M1_MAG, 7, 2), "fp8": (E4M3_MAG[:E4M3_MAX_CODE + 1], E4M3_MAX_CODE, 8)}


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Element codes (sign bit 3 for FP4, bit 7 for FP8) to float64 values."""
    codes = np.asarray(codes).astype(np.int64)
    if fmt == "fp4":
        mag = E2M1_MAG[codes & 7]
        neg = (codes >> 3) & 1
    else:
        mag = E4M3_MAG[codes & 127]
        neg = (codes >> 7) & 1
    return np.where(neg == 1, -mag, mag)


def round_to_format(x: np.ndarray, fmt: str) -> np.ndarray:
    """RM3: nearest representable magnitude code, ties to the even code (codes are ordered by
    magnitude, and an even code has an even significand), saturating at the largest normal."""
    mags, max_code, _ = FORMATS[fmt]
    a = np.abs(np.asarray(x, F64))
    idx = np.clip(np.searchsorted(mags, a, side="left"), 0, max_code)   # first magnitude >= a
    lo = np.clip(idx - 1, 0, max_code)
    hi = idx
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= mags[max_code], max_code, code)                 # saturate
    sign_bit = 8 if fmt == "fp4" else 128
    return np.where((np.asarray(x, F64) < 0) & (code > 0), code + sign_bit, code).astype(np.uint8)


def shared_exponent(block_max: np.ndarray, fmt: str) -> np.ndarray:
    """RM2: the E8M0 byte of each block from its largest magnitude."""
    emax = FORMATS[fmt][2]
    m = np.asarray(block_max, F64)
    _, e = np.frexp(m)                   # m = f * 2^e, 0.5 <= f < 1, so floor(log2 m) = e - 1
    se = np.clip(e - 1 - emax, -127, 127)
    return np.where(m > 0, se + 127, 0).astype(np.uint8)


def quantize(x: np.ndarray, fmt: str):
    """MX-quantise rows of x [..., K] (K a multiple of 32) along the last axis.

    Returns (codes [..., K] uint8 element codes, scales [..., K/32] uint8 E8M0 bytes)."""
    x = np.asarray(x, F64)
    K = x.shape[-1]
    assert K % BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (K // BLOCK, BLOCK))
    sc = shared_exponent(np.max(np.abs(blocks), axis=-1), fmt)
    X = np.ldexp(1.0, sc.astype(np.int64) - 127)
    codes = round_to_format(blocks / X[..., None], fmt)
    return codes.reshape(x.shape), sc


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """RM1: value = 2^(e - 127) * element."""
    codes = np.asarray(codes)
    K = codes.shape[-1]
    v = decode(codes, fmt).reshape(codes.shape[:-1] + (K // BLOCK, BLOCK))
    X = np.ldexp(1.0, np.asarray(scales).astype(np.int64) - 127)
    return (v * X[..., None]).reshape(codes.shape)


def pack_fp4(codes: np.ndarray) -> np.ndarray:
    """RM4: two FP4 codes per byte along the last axis, even index in the low nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mx_matmul(a_codes, a_scales, w_packed, w_scales) -> np.ndarray:
    """deq(a) . deq(w)^T exactly (RM5): a fp8 [M, K], w fp4 packed [N, K/2]."""
    a = dequantize(a_codes, a_scales, "fp8")
    w = dequantize(unpack_fp4(w_packed), w_scales, "fp4")
    return a @ w.T


def mx_glu_stage(a, w1_codes, w1_scales, beta1: float, beta2: float):
    """RM6, first projection: a (float64 values of bf16 rows) quantised to MXFP8, times the
    dequantised FP4 W1 [2I, K] (unpacked codes), SiTU-GLU, stored bf16. Returns (h, a codes, a scales)."""
    aq, asc = quantize(a, "fp8")
    w1 = dequantize(w1_codes, w1_scales, "fp4")
    inter = w1.shape[0] // 2
    gu = dequantize(aq, asc, "fp8") @ w1.T
    h = O.store(O.situ(gu[:, :inter], beta1) * O.softcap(gu[:, inter:], beta2), "bf16")
    return h, aq, asc


def mx_down_stage(h, w2_codes, w2_scales):
    """RM6, second projection: h (float64 values of bf16) quantised to MXFP8 along inter, times the
    dequantised FP4 W2 [N, I] (unpacked codes), stored bf16."""
    hq, hs = quantize(h, "fp8")
    return O.store(dequantize(hq, hs, "fp8") @ dequantize(w2_codes, w2_scales, "fp4").T, "bf16")


def mx_expert_ffn(a, w1_codes, w1_scales, w2_codes, w2_scales, beta1: float, beta2: float):
    """One routed SiTU-GLU expert with MX operands (RM6); returns (h, y)."""
    h, _, _ = mx_glu_stage(a, w1_codes, w1_scales, beta1, beta2)
    return h, mx_down_stage(h, w2_codes, w2_scales)
