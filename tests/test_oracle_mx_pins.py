"""Pins of the MX oracle (CPU): the element formats against their bit-field definitions, rounding
ties, saturation, the shared exponent, error bounds, packing order and the block-scaled product.

Format facts used (OCP Microscaling formats, as read in the oracle's RM1-RM5): E2M1 has 1 sign,
2 exponent (bias 1) and 1 mantissa bit; E4M3 has 1 sign, 4 exponent (bias 7) and 3 mantissa bits,
no infinities and a NaN at exponent and mantissa all ones; E8M0 is 2^(e - 127).
"""
import numpy as np
import pytest

from oracle import lmoe_oracle_mx as M


def field_value(code, ebits, mbits, bias):
    """Value of a sign/exponent/mantissa code written out from the bit fields."""
    s = code >> (ebits + mbits)
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if e == 0:
        v = (m / 2 ** mbits) * 2.0 ** (1 - bias)
    else:
        v = (1 + m / 2 ** mbits) * 2.0 ** (e - bias)
    return -v if s else v


def test_element_tables():
    for c in range(16):
        assert M.decode(np.array([c]), "fp4")[0] == field_value(c, 2, 1, 1)
    for c in range(256):
        if (c & 127) == 127:
            continue                                   # NaN encodings
        assert M.decode(np.array([c]), "fp8")[0] == field_value(c, 4, 3, 7)
    assert list(M.E2M1_MAG) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert M.E4M3_MAG[126] == 448.0 and M.E4M3_MAG[1] == 2.0 ** -9 and M.E4M3_MAG[8] == 2.0 ** -6
    assert M.E4M3_MAG[0x38] == 1.0                     # the byte the GPU reads as 1.0


def test_rounding_ties_and_saturation_fp4():
    # block max 4 -> floor(log2 4) - 2 = 0 -> X = 1; ties go to the even significand
    vals = np.array([4.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 0.3, 2.9] + [0.0] * 20)
    codes, sc = M.quantize(vals[None, :], "fp4")
    assert sc[0, 0] == 127
    got = M.decode(codes, "fp4")[0, :12]
    np.testing.assert_array_equal(got, [4, 0, 1, 1, 2, 2, 4, 4, 0, -4, 0.5, 3])
    assert codes[0, 8] == 0                            # -0.25 rounds to +0 (no negative zero code)
    # max 7.9: X = 1 and 7.9 saturates to 6
    v = np.zeros((1, 32)); v[0, 0] = 7.9; v[0, 1] = -7.0
    c, sc = M.quantize(v, "fp4")
    assert sc[0, 0] == 127 and M.decode(c, "fp4")[0, 0] == 6.0 and M.decode(c, "fp4")[0, 1] == -6.0


def test_shared_exponent_and_saturation_fp8():
    v = np.zeros((1, 32)); v[0, 0] = 1000.0; v[0, 1] = 3.0
    c, sc = M.quantize(v, "fp8")
    assert sc[0, 0] == 127 + 1                         # floor(log2 1000) - 8 = 1
    d = M.dequantize(c, sc, "fp8")[0]
    assert d[0] == 896.0                               # 500 saturates to 448, times 2
    assert d[1] == 3.0
    z, zs = M.quantize(np.zeros((2, 64)), "fp8")
    assert not z.any() and not zs.any()                # all-zero blocks: e = 0, codes 0
    tiny = np.full((1, 32), 2.0 ** -140)
    _, ts = M.quantize(tiny, "fp4")
    assert ts[0, 0] == 0                               # exponent clamped at -127


@pytest.mark.parametrize("fmt,frac", [("fp4", 0.25), ("fp8", 1.0 / 8)])
def test_error_bound(fmt, frac):
    # max/X lies in [2^emax, 2^(emax+1)), above the largest normal (6 or 448) for the top of that
    # range: saturation costs at most 2X (fp4, 8 - 6) or 64X (fp8, 512 - 448), i.e. max/4 and max/8;
    # rounding below the largest normal costs at most half a spacing (X and 16X), which is less
    rng = np.random.default_rng(0)
    x = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    c, sc = M.quantize(x, fmt)
    d = M.dequantize(c, sc, fmt)
    bmax = np.repeat(np.max(np.abs(x.reshape(64, 8, 32)), axis=2), 32, axis=1)
    assert np.all(np.abs(d - x) <= frac * bmax)
    # values on the grid survive exactly
    c2, sc2 = M.quantize(d, fmt)
    np.testing.assert_array_equal(M.dequantize(c2, sc2, fmt), d)


def test_pack_order_and_block_product():
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    p = M.pack_fp4(codes)
    assert p.shape == (3, 32) and p[0, 0] == codes[0, 0] | (codes[0, 1] << 4)
    np.testing.assert_array_equal(M.unpack_fp4(p), codes)
    a, as_ = M.quantize(rng.standard_normal((5, 128)), "fp8")
    wc, ws = M.quantize(rng.standard_normal((7, 128)), "fp4")
    got = M.mx_matmul(a, as_, M.pack_fp4(wc), ws)
    # the same product with the scales factored out of each 32-element block
    want = np.zeros((5, 7))
    for b in range(4):
        pa = M.decode(a[:, 32 * b:32 * b + 32], "fp8")
        pw = M.decode(wc[:, 32 * b:32 * b + 32], "fp4")
        xa = 2.0 ** (as_[:, b].astype(np.int64) - 127)
        xw = 2.0 ** (ws[:, b].astype(np.int64) - 127)
        want += np.outer(xa, xw) * (pa @ pw.T)
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=0)


def on_grid(rng, rows, K, fmt):
    """Rows of MX-representable values: random codes and scales with one element per block at a
    top-binade magnitude, so quantisation returns every value unchanged (and the same scale)."""
    mags, max_code, emax = M.FORMATS[fmt]
    codes = rng.integers(0, max_code + 1, (rows, K))
    top = np.nonzero(mags >= 2.0 ** emax)[0]                  # codes in the largest binade
    codes[:, ::32] = rng.choice(top, (rows, K // 32))
    sign = 8 if fmt == "fp4" else 128
    codes = np.where(rng.random((rows, K)) < 0.5, codes + sign * (codes > 0), codes).astype(np.uint8)
    scales = rng.integers(120, 134, (rows, K // 32)).astype(np.uint8)
    return codes, scales, M.dequantize(codes, scales, fmt)


def test_mx_glu_stage_on_grid_is_the_bf16_expert():
    """With operands already on the MX grids the first projection is the (pinned) bf16 expert's:
    quantisation is the identity there, so h must match situ_glu_ffn's h exactly."""
    from oracle import lmoe_oracle as O
    rng = np.random.default_rng(21)
    I, K, rows = 64, 128, 40
    w1c, w1s, w1 = on_grid(rng, 2 * I, K, "fp4")
    ac, asc, a = on_grid(rng, rows, K, "fp8")
    a = a * 2.0 ** -10                                       # keep the products in a sane range
    asc = (asc.astype(np.int64) - 10).astype(np.uint8)
    q, qs = M.quantize(a, "fp8")
    assert np.array_equal(q, ac) and np.array_equal(qs, asc)
    h, aq, _ = M.mx_glu_stage(a, w1c, w1s, 4.0, 25.0)
    h_ref, _ = O.situ_glu_ffn(a, w1, np.zeros((8, I)), 4.0, 25.0, "bf16")
    assert np.array_equal(aq, ac)
    assert np.array_equal(h, h_ref)


def test_mx_down_stage_brute_force():
    """Second projection on a tiny case against a scalar loop written from the format fields:
    y[r, n] = bf16(sum_k 2^(ea-127) fp8(h code) * 2^(ew-127) fp4(w code))."""
    from oracle import lmoe_oracle as O
    rng = np.random.default_rng(22)
    rows, N, I = 3, 5, 64
    h = O.store(rng.standard_normal((rows, I)) * 3.0, "bf16")
    w2c, w2s, _ = on_grid(rng, N, I, "fp4")
    y = M.mx_down_stage(h, w2c, w2s)
    hq, hs = M.quantize(h, "fp8")
    for r in range(rows):
        for n in range(N):
            acc = 0.0
            for k in range(I):
                va = field_value(int(hq[r, k]), 4, 3, 7) * 2.0 ** (int(hs[r, k // 32]) - 127)
                vw = field_value(int(w2c[n, k]), 2, 1, 1) * 2.0 ** (int(w2s[n, k // 32]) - 127)
                acc += va * vw
            assert y[r, n] == O.store(np.array([acc]), "bf16")[0], (r, n)
