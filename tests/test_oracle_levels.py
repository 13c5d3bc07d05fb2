"""Pins of the oracle's streaming units: a chunk's own container decodes to
the rows the whole-tensor decode gives for that chunk (every chunk, the last
one ragged), chunk payloads partition the whole payload, and quality levels
(bins tables) trade size against error monotonically on KV-like data."""
import numpy as np

import kvgen
import oracle


def test_chunk_containers_decode_like_the_whole():
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=300, n_layers=3, n_channels=64, chunk_tokens=128,
                                     layer_bins=((0, 1, 32), (1, 3, 16)))
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, _, T, C = kv.shape
    r = oracle.codec(kv, bins, Tc)
    total, sizes = 0, []
    for j in range(oracle.n_chunks(T, Tc)):
        nj = oracle.chunk_tokens(T, Tc, j)
        data = oracle.serialize_chunk(r, j, bins, T, Tc)
        back = oracle.deserialize(data, L, C, nj, Tc, bins)
        o, n = back["payload_offset"], back["payload_bytes"]
        sym, bad = oracle.decode(data[o:], back["slab_off"], back["stream_len"], back["cdf"],
                                 L, C, nj, Tc, int(bins.max()))
        assert not bad
        assert np.array_equal(sym, r["dec_sym"][:, :, j * Tc:j * Tc + nj])
        out = oracle.dequantize(sym, back["max1"], bins, fp32=False)
        assert np.array_equal(out, r["out_f16"][:, :, j * Tc:j * Tc + nj])
        assert data.size == oracle.container_bytes(L, C, nj, Tc, bins, n)
        total += n
        sizes.append(nj)
    assert total == r["payload"].size
    assert sizes == [128, 128, 44]


def test_levels_trade_size_for_error():
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=256, n_layers=4, n_channels=128)
    kv, _ = kvgen.generate(cfg)
    x = kv.view(np.float16).astype(np.float64)
    L = cfg.n_layers
    sizes, errs = [], []
    for b in (64, 32, 16, 8):
        bins = np.full((L, 2), b, np.int32)
        r = oracle.codec(kv, bins, cfg.chunk_tokens)
        sizes.append(r["payload"].size)
        y = r["out_f16"].view(np.float16).astype(np.float64)
        errs.append(np.sqrt(np.mean((y - x) ** 2)))
    assert sizes == sorted(sizes, reverse=True) and len(set(sizes)) == 4
    assert errs == sorted(errs) and len(set(errs)) == 4
