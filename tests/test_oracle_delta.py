"""Pins of the oracle's token-delta transform (oracle/kvc_delta.c): one-token
groups are the identity; a hand-worked example whose anchors lie on the
quantizer grid (so every delta is exact) and one whose anchor does not (so
the reference must be the reconstruction, not the input); chunks stand
alone; on AR(1) inputs the deltas are smaller than the rows; and through the
whole codec the error is bounded by the delta row's own quantization step,
which fails if an anchor's error carried into its tokens."""
import numpy as np
import pytest

import kvgen
import oracle


def f16(rows):
    return np.asarray(rows, dtype=np.float16).view(np.uint16)


def test_one_token_groups_are_identity():
    cfg = kvgen.CONFIGS["c1"].scaled(n_tokens=70, chunk_tokens=32)
    kv, _ = kvgen.generate(cfg)
    d = oracle.delta_forward(kv, cfg.bins(), 32, 1)
    assert np.array_equal(d, kv)
    assert np.array_equal(oracle.delta_inverse(kv, 32, 1), kv)


def _hand_example():
    # L = 1, T = 5, C = 4, one chunk of 5 tokens, G = 3: anchors are tokens 0 and 3.
    # bins 6: MAX = 2.  K anchors are on the grid (x = m (q - 2) / 2): reconstruction exact.
    K = [[2.0, -1.0, 0.0, 1.0],      # anchor: m = 2, factor 1, q = [4, 1, 2, 3] -> itself
         [2.5, -0.75, 0.25, 1.0],
         [1.5, -1.5, 0.5, 0.5],
         [4.0, 2.0, -2.0, 0.0],      # anchor: m = 4, factor 0.5, q = [4, 3, 1, 2] -> itself
         [3.0, 3.0, -1.0, 0.5]]
    # V's first anchor is off the grid: 0.3 quantizes to q = rint(2.3) = 2 -> 0
    V = [[2.0, 0.3, 0.0, 0.0],
         [2.0, 0.3, 0.0, 0.0],
         [1.0, 0.3, 0.0, 0.0],
         [1.0, 1.0, 1.0, 1.0],       # anchor: m = 1, q = [3, 3, 3, 3] -> itself
         [1.0, 1.0, 1.0, 1.0]]
    kv = np.stack([f16(K), f16(V)])[None]
    return kv, np.array([[6, 6]], np.int32)


def test_hand_worked_example():
    kv, bins = _hand_example()
    d = oracle.delta_forward(kv, bins, 5, 3)
    want_K = f16([[2.0, -1.0, 0.0, 1.0],
                  [0.5, 0.25, 0.25, 0.0],     # token 1 - token 0
                  [-0.5, -0.5, 0.5, -0.5],    # token 2 - token 0 (not token 1)
                  [4.0, 2.0, -2.0, 0.0],
                  [-1.0, 1.0, 1.0, 0.5]])     # token 4 - token 3
    assert np.array_equal(d[0, 0], want_K)
    # V: the reference is the reconstruction [2, 0, 0, 0], so 0.3 stays in the delta
    assert np.array_equal(d[0, 1, 0], kv[0, 1, 0])
    assert np.array_equal(d[0, 1, 1], f16([0.0, 0.3, 0.0, 0.0]))
    assert np.array_equal(d[0, 1, 2], f16([-1.0, 0.3, 0.0, 0.0]))
    assert np.array_equal(d[0, 1, 4], f16([0.0, 0.0, 0.0, 0.0]))
    # without coding, the inverse adds the anchor rows back (exact here)
    back = d.copy()
    back[0, 1, 0] = f16([2.0, 0.0, 0.0, 0.0])  # the decoder's anchor row is the reconstruction
    y = oracle.delta_inverse(back, 5, 3)
    assert np.array_equal(y[0, 0], kv[0, 0])
    assert np.array_equal(y[0, 1, 1:], kv[0, 1, 1:])


def test_chunks_stand_alone():
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=300, n_layers=2, n_channels=64, chunk_tokens=128,
                                     layer_bins=((0, 2, 16),))
    kv, _ = kvgen.generate(cfg)
    bins, Tc, G = cfg.bins(), cfg.chunk_tokens, 5
    d = oracle.delta_forward(kv, bins, Tc, G)
    for j in range(oracle.n_chunks(300, Tc)):
        nj = oracle.chunk_tokens(300, Tc, j)
        part = np.ascontiguousarray(kv[:, :, j * Tc:j * Tc + nj])
        assert np.array_equal(oracle.delta_forward(part, bins, Tc, G), d[:, :, j * Tc:j * Tc + nj])


def test_deltas_are_smaller_on_ar1_rows():
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=256, n_layers=2, n_channels=256)
    kv, _ = kvgen.generate(cfg)
    d = oracle.delta_forward(kv, cfg.bins(), 256, 4)
    x = kv.view(np.float16).astype(np.float64)
    dd = d.view(np.float16).astype(np.float64)
    non_anchor = np.arange(256) % 4 != 0
    ms_x = np.mean(x[:, :, non_anchor] ** 2)
    ms_d = np.mean(dd[:, :, non_anchor] ** 2)
    assert ms_d < 0.5 * ms_x  # rho = 0.95: about 2 (1 - rho^k) of the rows' power for k <= 3


@pytest.mark.parametrize("G", [2, 4, 16])
def test_codec_error_is_the_delta_step_only(G):
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=200, n_layers=2, n_channels=128, chunk_tokens=64,
                                     layer_bins=((0, 1, 32), (1, 2, 16)))
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    d = oracle.delta_forward(kv, bins, Tc, G)
    r = oracle.codec(d, bins, Tc)
    xh = oracle.delta_inverse(r["out_f16"], Tc, G)
    x = kv.view(np.float16).astype(np.float64)
    y = xh.view(np.float16).astype(np.float64)
    yd = r["out_f16"].view(np.float16).astype(np.float64)
    mD = r["max1"].view(np.float16).astype(np.float64)[..., None]  # each delta row's own max
    MAX = (bins // 2 - 1).astype(np.float64)[:, :, None, None]
    # the codec's step on the delta row, the fp16 rounding of the delta, of the decoded delta
    # and of the sum; nothing from the anchor's own quantization
    bound = (mD / (2 * MAX) + mD * (2.0**-11 + 2.0**-20) + np.abs(yd) * 2.0**-11
             + np.abs(y) * 2.0**-11 + 2.0**-23)
    assert (np.abs(y - x) <= bound).all()
    plain = oracle.codec(kv, bins, Tc)["out_f16"].view(np.float16).astype(np.float64)
    if G <= 4:  # close anchors: the delta rows carry less error than the rows coded themselves
        na = (np.arange(200) % Tc) % G != 0
        assert np.mean((y - x)[:, :, na] ** 2) < 0.5 * np.mean((plain - x)[:, :, na] ** 2)


def test_rejects_bad_arguments_and_nonfinite():
    kv, bins = _hand_example()
    with pytest.raises(oracle.OracleError):
        oracle.delta_forward(kv, bins, 5, 0)
    for t in (0, 1):  # Inf in an anchor row, then in a delta row
        bad = np.zeros((1, 2, 2, 4), np.uint16)
        bad[0, 1, t, 2] = f16([np.inf])[0]
        with pytest.raises(oracle.OracleError):
            oracle.delta_forward(bad, np.array([[6, 6]], np.int32), 2, 2)


def saturation_example():
    """L = 1, T = 2, C = 4, G = 2, bins 6 (MAX = 2): the anchor row
    [-65504, 65504, 0, 32752] is on the quantizer grid (max1 = 65504, codes
    0, 4, 2, 3), so its reconstruction is itself; the token row
    [16, -16, 0, -32752] has differences 65520, -65520, 0, -65504, whose
    fp16 roundings without the clamp would be +Inf, -Inf (65520 is half way to
    the next power of two and rounds up), and which saturate to +-65504."""
    kv = np.zeros((1, 2, 2, 4), np.uint16)
    kv[0, 0, 0] = f16([-65504.0, 65504.0, 0.0, 32752.0])
    kv[0, 0, 1] = f16([16.0, -16.0, 0.0, -32752.0])
    kv[0, 1, 0] = f16([1.0, 2.0, 3.0, 4.0])
    kv[0, 1, 1] = f16([1.0, 2.0, 3.0, 4.0])
    return kv, np.array([[6, 6]], np.int32)


def test_saturating_delta_pin():
    kv, bins = saturation_example()
    d = oracle.delta_forward(kv, bins, 2, 2)
    assert np.array_equal(d[0, 0, 0], kv[0, 0, 0])
    assert np.array_equal(d[0, 0, 1], f16([65504.0, -65504.0, 0.0, -65504.0]))
    # the V half: anchor [1, 2, 3, 4] at max1 4, codes rint(x / 2 + 2) -> [2, 3, 4, 4]
    # (2.5 rounds to even), reconstruction [0, 2, 4, 4], so the deltas are [1, 0, -1, 0]
    assert np.array_equal(d[0, 1, 1], f16([1.0, 0.0, -1.0, 0.0]))
    # the inverse on these deltas taken as decoded: anchor + clamped delta; the first two
    # elements come back 16 away from the input (the clamp's error), the last exactly
    y = oracle.delta_inverse(d, 2, 2)
    assert np.array_equal(y[0, 0, 1], f16([0.0, 0.0, 0.0, -32752.0]))
    # a sum past the fp16 range saturates too: 65504 + 32 would round to Inf
    z = np.zeros((1, 2, 2, 4), np.uint16)
    z[0, 0, 0] = f16([65504.0, -65504.0, 65504.0, 1.0])
    z[0, 0, 1] = f16([32.0, -32.0, -1.0, 1.0])
    w = oracle.delta_inverse(z, 2, 2)
    assert np.array_equal(w[0, 0, 1], f16([65504.0, -65504.0, 65504.0, 2.0]))
