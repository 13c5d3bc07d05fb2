"""Pins of the oracle's 8-bit comparator quantizer (oracle/kvc_int8.c):
exact rational values of the printed formulas away from rounding ties, the
special points (group min and max, clamped zero points, constant groups),
the reconstruction error bound, exact dequantized values, and the page's
own dequantize expression evaluated by torch in float32 (bit for bit)."""
from fractions import Fraction

import numpy as np
import pytest

import kvgen
import oracle


def f16(vals):
    return np.asarray(vals, dtype=np.float16).view(np.uint16)


def _as_kv(groups, g):
    """Rows of whole groups as a [1][2][T][C] fp16-bit array (K and V the same)."""
    flat = np.concatenate([np.asarray(x, np.float16) for x in groups])
    C = g * 2
    rows = flat.reshape(-1, C)
    kv = np.stack([rows, rows])[None]
    return kv.view(np.uint16), rows.astype(np.float64)


def test_exact_rational_values_away_from_ties():
    rng = np.random.default_rng(3)
    g = 16
    groups = [rng.standard_normal(g) * rng.uniform(0.01, 50) + rng.uniform(-5, 5) for _ in range(400)]
    kv, rows = _as_kv(groups, g)
    q, scale, zp = oracle.int8_quantize(kv, g)
    checked = 0
    for r in range(rows.shape[0]):
        for k in range(rows.shape[1] // g):
            x = [Fraction(float(v)) for v in rows[r, k * g:(k + 1) * g]]
            mn, mx = min(x), max(x)
            if mx == mn:
                continue
            z = -mn * 255 / (mx - mn)
            if abs(z - round(z)) > Fraction(1, 100) and 0 <= z <= 255:
                assert zp[0, 0, r, k] == round(z)
                checked += 1
            for i, xi in enumerate(x):
                u = (xi - mn) * 255 / (mx - mn)
                if abs(u - int(u) - Fraction(1, 2)) > Fraction(1, 100):
                    assert q[0, 0, r, k * g + i] == int(u + Fraction(1, 2)), (r, k, i)
                    checked += 1
    assert checked > 5000


def test_special_points_and_clamps():
    g = 8
    groups = [
        [-3.0, -1.0, 0.0, 0.5, 1.0, 2.0, 4.0, 5.0],      # mixed signs
        [1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0],         # all positive: zero point clamps to 0
        [-8.0, -7.0, -6.0, -5.0, -4.0, -3.0, -2.0, -1.0],  # all negative: zero point clamps to 255
        [2.5] * 8,                                         # constant
    ]
    kv, rows = _as_kv(groups, g)
    q, scale, zp = oracle.int8_quantize(kv, g)
    q, scale, zp = q[0, 0].reshape(-1, g), scale[0, 0].reshape(-1), zp[0, 0].reshape(-1)
    for k, grp in enumerate(groups[:3]):
        assert q[k][int(np.argmin(grp))] == 0 and q[k][int(np.argmax(grp))] == 255
        assert scale[k] == np.float32(np.float32(max(grp) - min(grp)) / np.float32(255))
    assert zp[1] == 0 and zp[2] == 255
    assert scale[3] == 0 and zp[3] == 0 and not q[3].any()
    y = oracle.int8_dequantize(q.reshape(1, 2, -1, 2 * g)[:, :1].repeat(2, axis=1),
                               scale.reshape(1, 1, -1, 2).repeat(2, axis=1),
                               zp.reshape(1, 1, -1, 2).repeat(2, axis=1), g)
    assert not y.reshape(-1, g)[3].any()  # the constant group decodes to 0


def test_dequantize_order_exact():
    # scale a power of two: (q - zp) * scale is exact, then rounded to fp16
    q = np.array([0, 1, 127, 128, 255, 64, 200, 3], np.uint8).reshape(1, 1, 1, 8).repeat(2, axis=1)
    scale = np.array([[[[2.0 ** -4]]]], np.float32).repeat(2, axis=1)
    zp = np.array([[[[128]]]], np.uint8).repeat(2, axis=1)
    y = oracle.int8_dequantize(q, scale, zp, 8)
    want = f16([(v - 128) * 2.0 ** -4 for v in [0, 1, 127, 128, 255, 64, 200, 3]])
    assert np.array_equal(y[0, 0, 0], want)


def test_error_bound_on_kv_like_data():
    cfg = kvgen.CONFIGS["c5"].scaled(n_tokens=24, n_layers=2, n_channels=256,
                                     layer_bins=((0, 2, 16),))
    kv, _ = kvgen.generate(cfg)
    g = 128
    q, scale, zp = oracle.int8_quantize(kv, g)
    y = oracle.int8_dequantize(q, scale, zp, g).view(np.float16).astype(np.float64)
    x = kv.view(np.float16).astype(np.float64)
    s = np.repeat(scale.astype(np.float64), g, axis=-1)
    # q and the zero point each round by at most half a step; y then rounds to fp16
    bound = s * (1 + 1e-5) + np.abs(y) * 2.0 ** -11 + 2.0 ** -25
    assert (np.abs(y - x) <= bound).all()
    assert (np.abs(y - x) > 0.49 * s).any()  # the bound is not vacuous


def test_nonfinite_and_bad_group_rejected():
    kv = np.zeros((1, 2, 1, 8), np.uint16)
    kv[0, 0, 0, 3] = 0x7C00
    with pytest.raises(oracle.OracleError):
        oracle.int8_quantize(kv, 8)
    with pytest.raises(oracle.OracleError):
        oracle.int8_quantize(np.zeros((1, 2, 1, 12), np.uint16), 8)


def test_exact_ties_round_to_even():
    # scale = range / 255 = 1/16 exactly; (x - mn) / scale lands on k + 1/2 for the tie entries
    s = 1.0 / 16
    mn = -2.5 * s  # -mn / scale = 2.5: the zero point ties too
    grp = [mn, mn + 255 * s, mn + 0.5 * s, mn + 2.5 * s, mn + 16.5 * s, mn + 1.5 * s, mn + 3.0 * s,
           mn + 254.5 * s]
    kv, rows = _as_kv([grp, grp], 8)
    assert np.array_equal(rows[0, :8], np.asarray(grp, np.float64))  # all exact in fp16
    q, scale, zp = oracle.int8_quantize(kv, 8)
    assert scale[0, 0, 0, 0] == np.float32(s)
    assert zp[0, 0, 0, 0] == 2  # 2.5 -> 2
    assert q[0, 0, 0, :8].tolist() == [0, 255, 0, 2, 16, 2, 3, 254]  # 0.5->0, 2.5->2, 16.5->16, 1.5->2, 254.5->254


def test_dequantize_page_code_pin_fp32():
    """The page's dequantize_key ([KVM] 四): q and the zero point converted
    with .float(), subtracted, times the float scale.  Evaluated by torch on
    CPU float32 tensors it must equal the oracle's fp32 output bit for bit;
    the fp16 output is that value rounded to nearest even.  Includes groups
    spanning +-65504 (the 70B workload's saturated channels), where the fp32
    result stays finite and the fp16 one overflows."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(21)
    g = 16
    groups = [rng.standard_normal(g) * rng.uniform(0.01, 3000) for _ in range(300)]
    groups += [[65504.0, -65504.0] * (g // 2), [65504.0] + [-3.0] * (g - 1)]
    kv, _ = _as_kv(groups, g)
    q, scale, zp = oracle.int8_quantize(kv, g)
    y32 = oracle.int8_dequantize(q, scale, zp, g, fp32=True)
    y16 = oracle.int8_dequantize(q, scale, zp, g)
    qt = torch.from_numpy(q.astype(np.uint8))
    zt = torch.from_numpy(np.repeat(zp, g, axis=-1).astype(np.uint8))
    st = torch.from_numpy(np.repeat(scale, g, axis=-1))
    page = (qt.float() - zt.float()) * st
    assert page.dtype == torch.float32
    assert np.array_equal(page.numpy().view(np.uint32), y32.view(np.uint32))
    assert np.array_equal(page.half().numpy().view(np.uint16), y16)
    assert np.isfinite(y32).all() and not np.isfinite(y16.view(np.float16)).all()
