"""The shared input generator: deterministic, thread-count independent, the
configured shapes and statistics."""
import numpy as np

import kvgen


def test_deterministic_and_thread_independent():
    cfg = kvgen.CONFIGS["c2"].scaled(n_layers=2, layer_bins=((0, 2, 32),), n_tokens=300)
    a, _ = kvgen.generate(cfg, threads=1)
    b, _ = kvgen.generate(cfg, threads=5)
    c, _ = kvgen.generate(cfg.scaled(seed=1), threads=3)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert kvgen.checksum(a) == kvgen.checksum(b)


def test_statistics_and_outliers():
    cfg = kvgen.CONFIGS["c4"].scaled(n_layers=1, layer_bins=((0, 1, 32),), n_tokens=2000)
    kv, sat = kvgen.generate(cfg)
    x = kv.view(np.float16).astype(np.float64)
    assert np.isfinite(x).all() and sat == 0
    sd = x.std(axis=2)  # per (layer, kv, channel)
    n_out = round(0.02 * cfg.n_channels)
    # the outlier channels have 20x the scale: they are the largest spreads
    top = np.sort(sd[0, 0])[::-1]
    assert top[n_out - 1] > 20 * np.median(sd[0, 0]) * 0.2
    # AR(1) with rho = 0.97: strong lag-1 correlation
    z = x[0, 0, :, 5]
    r1 = np.corrcoef(z[:-1], z[1:])[0, 1]
    assert 0.9 < r1 < 0.995


def test_configs_cover_all_layers():
    for cfg in kvgen.CONFIGS.values():
        b = cfg.bins()
        assert b.shape == (cfg.n_layers, 2) and (b % 2 == 0).all() and b.min() >= 4
