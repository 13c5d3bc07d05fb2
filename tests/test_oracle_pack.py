"""Pins of stream order and packing (slab offsets = exclusive scan of stream
lengths, streams concatenated in (chunk, layer, K|V, token) order), and of the
whole CPU hot path on ragged shapes."""
import numpy as np
import pytest

import kvgen
import oracle


def small_cfg(L=3, C=40, T=300, Tc=128, seed=1):
    return kvgen.KVConfig(name="t", workload="t", n_layers=L, n_channels=C, n_tokens=T,
                          chunk_tokens=Tc, layer_bins=((0, 1, 32), (1, L, 16)) if L > 1 else ((0, 1, 32),),
                          rho=0.9, innov="normal", scale_lo=0.1, scale_hi=4.0, seed=seed)


@pytest.mark.parametrize("L,C,T,Tc", [(3, 40, 300, 128), (1, 7, 5, 256), (2, 16, 64, 256), (2, 33, 257, 256)])
def test_packing_order_and_offsets(L, C, T, Tc):
    cfg = small_cfg(L, C, T, Tc)
    kv, _ = kvgen.generate(cfg)
    r = oracle.codec(kv, cfg.bins(), Tc)
    A = r["A"]
    NC = oracle.n_chunks(T, Tc)
    lens, offs, pay = r["stream_len"], r["slab_off"], r["payload"]
    assert offs[0] == 0 and offs[-1] == pay.size and offs.size == NC * L * 2 + 1
    sid, slab = 0, 0
    for j in range(NC):
        nj = oracle.chunk_tokens(T, Tc, j)
        for l in range(L):
            for kvi in range(2):
                pos = int(offs[slab])
                for t in range(nj):
                    want = oracle.encode_stream(r["sym"][l, kvi, j * Tc + t], r["cdf"][j, l, kvi])
                    assert lens[sid] == len(want)
                    assert pay[pos:pos + len(want)].tobytes() == want
                    pos += len(want)
                    sid += 1
                assert pos == int(offs[slab + 1])
                slab += 1
    assert sid == lens.size == 2 * L * T
    assert np.array_equal(r["dec_sym"], r["sym"]) and not r["corrupt"]


def test_empty_input():
    cfg = small_cfg(T=0)
    kv = np.zeros((cfg.n_layers, 2, 0, cfg.n_channels), np.uint16)
    r = oracle.codec(kv, cfg.bins(), 256)
    assert r["payload"].size == 0 and list(r["slab_off"]) == [0] and r["stream_len"].size == 0


def test_payload_capacity_reported():
    cfg = small_cfg()
    kv, _ = kvgen.generate(cfg)
    sym, _ = oracle.quantize(kv, cfg.bins())
    tab = oracle.cdf(sym, 128, 32)
    _, _, pay = oracle.encode(sym, tab, 128, 32)
    with pytest.raises(oracle.OracleError) as ei:
        oracle.encode(sym, tab, 128, 32, payload_cap=pay.size - 1)
    assert ei.value.code == oracle.ORC_ERR_CAPACITY
    oracle.encode(sym, tab, 128, 32, payload_cap=pay.size)


def test_constant_input_degenerate():
    """All-equal rows: every symbol is the top one, the CDF puts nearly all mass
    there, streams are tiny and decode exactly."""
    cfg = small_cfg(L=1, C=64, T=256, Tc=256)
    kv = np.full((1, 2, 256, 64), np.float16(1.5).view(np.uint16), np.uint16)
    r = oracle.codec(kv, cfg.bins(), 256)
    assert (r["sym"] == 30).all()
    assert r["payload"].size <= 2 * 256 * 2
    y = r["out_f16"].view(np.float16)
    assert (y == np.float16(1.5)).all()
