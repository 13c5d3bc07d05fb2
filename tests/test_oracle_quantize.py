"""Pins of the oracle's quantizer and dequantizer.

The write-up's encoder ("2.3 Encoder pipeline", step 1) quantizes each group
by its max |x|: MAX = bins/2 - 1, q = round(x * MAX/max1 + MAX) in [0, 2*MAX];
its decoder ("2.4 Decoder pipeline", step 2) inverts that: (q - MAX)/MAX*max1.
What fixes these functions here, apart from the oracle itself:
  * the symbol range [0, 2*MAX] and the special points x = -m, 0, +m;
  * round-half-to-even on constructed exact ties;
  * exact rational rounding away from ties (brute force with Fractions);
  * the reconstruction error bound max|x|/(2*MAX), exhaustively over fp16,
    plus the fp32 rounding slack derived in the test below;
  * fp16 output equal to numpy's RNE conversion of the fp32 output;
  * the page's own quantize and dequantize expressions, evaluated by torch on
    CPU float32 tensors, agree bit for bit (operation order pins).
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle

F16_FINITE = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)  # non-negative finite fp16


def f16(vals):
    return np.asarray(vals, dtype=np.float32).astype(np.float16).view(np.uint16)


def as_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def quant_rows(rows_bits, nbins):
    """rows_bits: uint16 [R][C] -> sym [R][C], max1 [R] (K and V both use nbins)."""
    R, C = rows_bits.shape
    kv = np.ascontiguousarray(np.broadcast_to(rows_bits[None, None], (1, 2, R, C)))
    bins = np.array([[nbins, nbins]], dtype=np.int32)
    sym, max1 = oracle.quantize(kv, bins)
    assert np.array_equal(sym[0, 0], sym[0, 1])
    return sym[0, 0], max1[0, 0], bins


@pytest.mark.parametrize("nbins", [4, 6, 16, 32, 64, 100, 256])
def test_range_and_special_points(nbins):
    MAX = nbins // 2 - 1
    rng = np.random.default_rng(nbins)
    x = (rng.standard_normal((64, 96)) * np.exp2(rng.uniform(-20, 12, (64, 1)))).astype(np.float32)
    x = np.clip(x, -60000, 60000)
    bits = f16(x)
    sym, max1, _ = quant_rows(bits, nbins)
    xf = as_f32(bits)
    m = np.abs(xf).max(axis=1)
    assert np.array_equal(as_f32(max1), m)  # max1 is exact
    assert sym.min() >= 0 and sym.max() <= 2 * MAX
    # the row maximum lands on an end symbol, a zero lands on MAX
    for r in range(x.shape[0]):
        c = int(np.argmax(np.abs(xf[r])))
        assert sym[r, c] == (2 * MAX if xf[r, c] > 0 else 0)
    zrow = np.zeros((1, 8), dtype=np.uint16)
    zrow[0, 3] = f16([2.5])[0]
    s, _, _ = quant_rows(zrow, nbins)
    assert s[0, 0] == MAX and s[0, 3] == 2 * MAX


def test_zero_row_reading():
    """A row of zeros: max1 = 0, every symbol = MAX, and it dequantizes to 0."""
    rows = np.zeros((3, 16), dtype=np.uint16)
    rows[1, :] = 0x8000  # -0.0
    sym, max1, bins = quant_rows(rows, 32)
    assert (sym == 15).all() and (max1 & 0x7FFF == 0).all()
    kv_sym = np.ascontiguousarray(np.broadcast_to(sym[None, None], (1, 2, 3, 16)))
    y = oracle.dequantize(kv_sym, np.broadcast_to(max1[None, None], (1, 2, 3)).copy(), bins)
    assert (y == 0).all()


@pytest.mark.parametrize("nbins", [4, 16, 32, 64, 256])
def test_ties_round_half_to_even(nbins):
    """With max1 = MAX (exact in fp16) the factor is exactly 1, so x + MAX is an
    exact half-integer for x = k + 1/2, and the symbol must be the even neighbour.
    With max1 = 2*MAX the factor is exactly 1/2 and odd integers x give ties."""
    MAX = nbins // 2 - 1
    ks = np.arange(-MAX, MAX)
    for scale, xs in ((1, ks + 0.5), (2, 2 * ks + 1)):
        row = np.concatenate([[scale * MAX], xs]).astype(np.float32)
        sym, _, _ = quant_rows(f16(row)[None, :], nbins)
        z = xs / scale + MAX  # exact half-integers
        want = np.where(np.floor(z) % 2 == 0, np.floor(z), np.floor(z) + 1)
        assert np.array_equal(sym[0, 1:], want.astype(np.uint8))


def test_exact_rational_rounding():
    """Away from ties, q equals the exact rational round(x*MAX/m + MAX)."""
    rng = np.random.default_rng(7)
    checked = 0
    for nbins in (4, 16, 32, 64, 256):
        MAX = nbins // 2 - 1
        x = (rng.standard_normal((40, 64)) * np.exp2(rng.uniform(-24, 15, (40, 1)))).astype(np.float32)
        bits = f16(np.clip(x, -65504, 65504))
        sym, max1, _ = quant_rows(bits, nbins)
        for r in range(bits.shape[0]):
            m = Fraction(float(as_f32(max1[r])))
            if m == 0:
                continue
            for c in range(bits.shape[1]):
                z = Fraction(float(as_f32(bits[r, c]))) * MAX / m + MAX
                fl = z.numerator // z.denominator
                frac = z - fl
                if abs(frac - Fraction(1, 2)) > Fraction(1, 10000):
                    assert sym[r, c] == (fl + 1 if frac > Fraction(1, 2) else fl)
                    checked += 1
                else:
                    assert sym[r, c] in (fl, fl + 1)
    assert checked > 10000


def test_monotone_in_x():
    rng = np.random.default_rng(3)
    x = np.sort(rng.standard_normal(4000).astype(np.float32) * 3)
    sym, _, _ = quant_rows(f16(x)[None, :], 32)
    assert (np.diff(sym[0].astype(int)) >= 0).all()


def _roundtrip_bound(m, MAX):
    """|y - x| bound for fp32 output.  With u = 2^-24 (binary32 unit roundoff):
    factor = M/m (1+d1); p1 = x*factor (1+d2); p2 = (p1 + M)(1+d3) so that
    |p2 - z| <= 4*M*u (1 + O(u)) for z = x*M/m + M, |x| <= m; rounding adds 1/2.
    Dequant: y = fl(fl((q-M)/M)*m) is within 2u|y| of (q-M)*m/M.  Altogether
    |y - x| <= m/(2M) + 4*m*u + 2*m*u + O(u^2)  <=  m/(2M) + 8*m*u."""
    return m / (2.0 * MAX) + 8.0 * m * 2.0**-24


@pytest.mark.parametrize("nbins", [4, 16, 32, 64, 256])
def test_error_bound_exhaustive_fp16(nbins):
    """Every finite fp16 x with |x| <= m, for a spread of m (normal, subnormal,
    the largest fp16, m = MAX, and random), quantize then dequantize."""
    MAX = nbins // 2 - 1
    rng = np.random.default_rng(100 + nbins)
    ms = [65504.0, 1.0, 0.1, 2.0**-24, 2.0**-14, 6.1e-5, float(MAX), 7.0, 127.0, 3.14159, 1000.5]
    ms += list(np.exp2(rng.uniform(-24, 15.9, 6)))
    pos = as_f32(F16_FINITE)
    worst = 0.0
    for mv in ms:
        mbits = f16([mv])[0]
        m = float(as_f32(mbits))
        xs = pos[pos <= m]
        row_vals = np.concatenate([[m], xs, -xs]).astype(np.float32)
        row = f16(row_vals)[None, :]
        sym, max1, bins = quant_rows(row, nbins)
        assert float(as_f32(max1[0])) == m
        kv_sym = np.ascontiguousarray(np.broadcast_to(sym[None, None], (1, 2) + sym.shape))
        mx = np.ascontiguousarray(np.broadcast_to(max1[None, None], (1, 2, 1)))
        y = oracle.dequantize(kv_sym, mx, bins, fp32=True)[0, 0, 0].astype(np.float64)
        err = np.abs(y - row_vals.astype(np.float64))
        assert (err <= _roundtrip_bound(m, MAX)).all(), (mv, float(err.max()), m / (2 * MAX))
        if m > 0:
            worst = max(worst, float(err.max() / (m / (2 * MAX))))
        # fp16 output is numpy's RNE conversion of the fp32 output
        y16 = oracle.dequantize(kv_sym, mx, bins, fp32=False)[0, 0, 0]
        assert np.array_equal(y16, y.astype(np.float32).astype(np.float16).view(np.uint16))
    assert worst <= 1.0 + 16 * MAX * 2.0**-24


@pytest.mark.parametrize("nbins", [4, 32, 256])
def test_dequant_special_values(nbins):
    """q = MAX -> 0, q = 0 -> -m, q = 2*MAX -> +m exactly; y(MAX+d) = -y(MAX-d)."""
    MAX = nbins // 2 - 1
    q = np.arange(0, 2 * MAX + 1, dtype=np.uint8)[None, :]
    m = f16([3.7])
    sym = np.ascontiguousarray(np.broadcast_to(q[None, None], (1, 2, 1, q.shape[1])))
    mx = np.ascontiguousarray(np.broadcast_to(m[None, None], (1, 2, 1)))
    bins = np.array([[nbins, nbins]], dtype=np.int32)
    y = oracle.dequantize(sym, mx, bins, fp32=True)[0, 0, 0]
    mf = float(as_f32(m[0]))
    assert y[MAX] == 0 and y[0] == -np.float32(mf) and y[2 * MAX] == np.float32(mf)
    assert np.array_equal(y[MAX:], -y[MAX::-1])


def test_nonfinite_and_bad_bins_rejected():
    row = f16([1.0, 2.0, 3.0])[None, :]
    for bad in (np.inf, -np.inf, np.nan):
        r = row.copy()
        r[0, 1] = f16([bad])[0]
        with pytest.raises(oracle.OracleError) as ei:
            quant_rows(r, 32)
        assert ei.value.code == oracle.ORC_ERR_NONFINITE
    for nb in (2, 3, 31, 258, 0):
        with pytest.raises(oracle.OracleError):
            quant_rows(row, nb)


def _edge_maxes():
    """fp16 row maxima: subnormals (smallest, largest), the smallest normal,
    1.0, values with long mantissas, 65504, and a spread of random finite ones."""
    fixed = [0x0001, 0x0003, 0x02AB, 0x03FF, 0x0400, 0x0401, 0x1E66, 0x3BFF, 0x3C00, 0x3C01,
             0x4247, 0x4E00, 0x57FF, 0x6AAA, 0x7800, 0x7BFE, 0x7BFF]
    rng = np.random.default_rng(1234)
    rand = rng.integers(1, 0x7C00, 200)
    return np.array(fixed + list(rand), dtype=np.uint16)


DEQ_BINS = [4, 6, 16, 32, 64, 256]


@pytest.mark.parametrize("nbins", DEQ_BINS)
def test_dequantize_page_code_pin(nbins):
    """Pin of the dequantizer's operation order: the write-up's decoder
    ("2.4 Decoder pipeline", step 2) undoes the offset (integer subtraction of
    C = bins//2 - 1), converts to float and divides by C, then multiplies by
    the stored maxima.  That expression, evaluated by torch on CPU float32
    tensors (each operation rounded on its own), must equal the oracle bit for
    bit for every symbol q in [0, 2*MAX] and every row maximum in the sweep,
    in fp32 and after RNE to fp16.  The sweep is chosen so that the two
    plausible reorderings, (q-MAX)*m/MAX and (q-MAX)*(m/MAX), disagree with
    the page's order somewhere (asserted, so the pin is known to catch them)."""
    torch = pytest.importorskip("torch")
    MAX = nbins // 2 - 1
    maxes = _edge_maxes()
    R, Q = maxes.size, 2 * MAX + 1
    q = np.ascontiguousarray(np.broadcast_to(np.arange(Q, dtype=np.uint8)[None, :], (R, Q)))
    sym = np.ascontiguousarray(np.broadcast_to(q[None, None], (1, 2, R, Q)))
    mx = np.ascontiguousarray(np.broadcast_to(maxes[None, None], (1, 2, R)))
    bins = np.array([[nbins, nbins]], dtype=np.int32)
    want32 = oracle.dequantize(sym, mx, bins, fp32=True)[0, 0]
    want16 = oracle.dequantize(sym, mx, bins, fp32=False)[0, 0]

    # the page's expression, groups along the first axis as its [:, None, None] broadcast
    t = torch.from_numpy(q.astype(np.int64))[None]                      # [1, R, Q] integer indices
    maxt = torch.from_numpy(maxes.view(np.float16).astype(np.float32))[None, :, None]  # [1, R, 1]
    Ct = (torch.tensor([nbins], dtype=torch.int64) // 2 - 1)[:, None, None]
    y = t - Ct
    y = y.float() / Ct
    y = y * maxt
    got32 = y[0].numpy()
    assert got32.dtype == np.float32
    assert np.array_equal(got32.view(np.uint32), want32.view(np.uint32))
    got16 = y[0].half().numpy().view(np.uint16)
    assert np.array_equal(got16, want16)

    # the sweep tells the page's order from the two reorderings
    d = (t - Ct).float()
    Mf = Ct.float()
    alt1 = (d * maxt / Mf)[0].numpy()
    alt2 = (d * (maxt / Mf))[0].numpy()
    if MAX & (MAX - 1):  # dividing by a power of two is exact: then every order agrees
        assert not np.array_equal(alt1.view(np.uint32), want32.view(np.uint32))
        assert not np.array_equal(alt2.view(np.uint32), want32.view(np.uint32))


def test_quantize_page_code_pin():
    """Pin of the quantizer's operation order: the write-up's encoder
    ("2.3 Encoder pipeline", step 1) computes MAX = bins//2 - 1 per group, the
    group's max |x|, factor = MAX / max1, then round(x * factor + MAX).  That
    expression, evaluated by torch on CPU float32 tensors (each operation
    rounded on its own; torch.round is half-to-even), must give the oracle's
    symbols bit for bit.  Rows span 2^-24 .. 65504 in scale, include
    subnormal-only rows and rows whose max is 65504.  A reordered factor,
    round((x * MAX) / max1 + MAX), is asserted to differ on this data."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((2, 2, 50, 128)) * np.exp2(rng.uniform(-10, 8, (2, 2, 50, 1)))).astype(np.float32)
    x[0, 0, 0] = rng.standard_normal(128) * 2.0**-20          # subnormal fp16 values only
    x[0, 1, 1, :3] = [65504, -65504, 1.0]                     # the largest finite max
    x[1, 0, 2] = np.clip(rng.standard_normal(128) * 30000, -65504, 65504)
    bits = f16(x)
    bins = np.array([[32, 16], [64, 4]], dtype=np.int32)
    sym, _ = oracle.quantize(bits, bins)
    L = bins.shape[0]
    groups = torch.from_numpy(as_f32(bits)).reshape(L * 2, 50, 128)   # one group per (layer, K|V)
    bt = torch.from_numpy(bins.reshape(-1).astype(np.int64))
    MAXt = (bt // 2 - 1)[:, None, None]
    max1 = torch.amax(torch.abs(groups), dim=-1, keepdim=True)
    factor = MAXt / max1
    xq = torch.round(groups * factor + MAXt)
    assert xq.dtype == torch.float32
    got = xq.to(torch.uint8).numpy().reshape(sym.shape)
    assert np.array_equal(got, sym)
    alt = torch.round((groups * MAXt) / max1 + MAXt).to(torch.uint8).numpy().reshape(sym.shape)
    assert not np.array_equal(alt, sym)
