"""Pins of the oracle's byte container (oracle/kvc_container.c): a hand-built
byte string for a tiny case (every field placed from the format description,
not from the oracle), round trips of the whole codec through it, the size
arithmetic of the compact CDF rows, and refusal of tables or headers it
cannot represent."""
import struct

import numpy as np
import pytest

import kvgen
import oracle


def r16(x):
    return (x + 15) // 16 * 16


@pytest.mark.parametrize("S", [1, 2, 7])
def test_hand_built_container_of_a_tiny_case(S):
    # L=1, C=2, T=3, Tc=2 -> chunks of 2 and 1 tokens; bins K=6, V=4 -> A=6, K=65530.
    # S chunks per CDF table: 1 -> two tables; 2, or 7 (stored as 2 = NC) -> one table
    L, C, T, Tc = 1, 2, 3, 2
    bins = np.array([[6, 4]], np.int32)
    A, Kc = 6, 65536 - 6
    NC = 2
    S_stored = min(S, NC)
    NG = -(-NC // S_stored)
    cdf = np.zeros((NG, L, 2, C, A), np.uint16)
    inner = {}
    for j in range(NG):
        for kv in range(2):
            b = int(bins[0, kv])
            for c in range(C):
                row = [0] + [100 * (j + 1) + 10 * kv + c + k for k in range(1, b - 1)]
                row += [k + Kc for k in range(b - 1, A)]
                cdf[j, 0, kv, c] = row
                inner[(j, kv, c)] = row[1:b - 1]
    max1 = np.array([[[0x3C00, 0x4000, 0x7BFF], [0x0001, 0x8000, 0x1234]]], np.uint16)
    # stream order (chunk, layer, K|V, token): j0 K t0, t1 | j0 V t0, t1 | j1 K t2 | j1 V t2
    stream_len = np.array([2, 1, 0, 2, 0, 0], np.uint16)
    payload = np.frombuffer(b"\x11\x22\x33\x44\x55", np.uint8)

    got = oracle.serialize(cdf, max1, stream_len, payload, bins, Tc, tab_chunks=S)

    # offsets by hand: header 64, bins at 64 (2 bytes), CDF at 80:
    # per table 2 channels x (6-2) + 2 channels x (4-2) = 12 entries = 24 bytes
    o_cdf = 80
    o_max1 = r16(o_cdf + 24 * NG)
    o_len = o_max1 + 16  # 6 max1 values = 12 bytes, padded
    o_pay = o_len + 16
    total = o_pay + 16
    want = bytearray(total)
    struct.pack_into("<IIIIQIIQQI", want, 0, 0x3143564B, 1, L, C, T, Tc, A, payload.size, total, S_stored)
    want[64:66] = bytes([6, 4])
    p = o_cdf
    for j in range(NG):
        for kv in range(2):
            for c in range(C):
                for v in inner[(j, kv, c)]:
                    struct.pack_into("<H", want, p, v)
                    p += 2
    assert p == o_cdf + 24 * NG
    for i, v in enumerate(max1.reshape(-1)):
        struct.pack_into("<H", want, o_max1 + 2 * i, int(v))
    for i, v in enumerate(stream_len):
        struct.pack_into("<H", want, o_len + 2 * i, int(v))
    want[o_pay:o_pay + 5] = payload.tobytes()
    assert got.tobytes() == bytes(want)
    assert oracle.container_payload_offset(L, C, T, Tc, bins, S) == o_pay
    assert oracle.container_bytes(L, C, T, Tc, bins, 5, S) == total

    back = oracle.deserialize(got, L, C, T, Tc, bins, S)
    assert np.array_equal(back["cdf"], cdf)
    assert np.array_equal(back["max1"], max1)
    assert np.array_equal(back["stream_len"], stream_len)
    with pytest.raises(oracle.OracleError):  # the header's S must match the reader's
        oracle.deserialize(got, L, C, T, Tc, bins, 1 if S_stored == 2 else 2)
    assert back["slab_off"].tolist() == [0, 3, 5, 5, 5]
    assert back["payload_bytes"] == 5


@pytest.mark.parametrize("cfg", [
    kvgen.CONFIGS["c1"],
    kvgen.CONFIGS["c2"].scaled(n_tokens=70, n_layers=3, layer_bins=((0, 1, 32), (1, 3, 16))),
    kvgen.CONFIGS["c5"].scaled(n_tokens=40, n_layers=3, n_channels=64,
                               layer_bins=((0, 1, 64), (1, 2, 32), (2, 3, 16))),
])
def test_codec_round_trips_through_the_container(cfg):
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    r = oracle.codec(kv, bins, Tc)
    data = oracle.serialize(r["cdf"], r["max1"], r["stream_len"], r["payload"], bins, Tc)
    L, _, T, C = kv.shape
    back = oracle.deserialize(data, L, C, T, Tc, bins)
    for key in ("cdf", "max1", "stream_len", "slab_off"):
        assert np.array_equal(back[key], r[key]), key
    o, n = back["payload_offset"], back["payload_bytes"]
    assert n == r["payload"].size
    assert np.array_equal(data[o:o + n], r["payload"])
    # decode straight from the container's payload section
    sym, bad = oracle.decode(data[o:], back["slab_off"], back["stream_len"], back["cdf"],
                             L, C, T, Tc, int(np.max(bins)))
    assert not bad and np.array_equal(sym, r["sym"])


def test_size_follows_the_per_layer_alphabet():
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=300)  # two chunks, bins 32 (layers 0-9) / 16
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, C, T = cfg.n_layers, cfg.n_channels, cfg.n_tokens
    entries = 2 * C * (10 * (32 - 2) + 22 * (16 - 2))  # per chunk, K and V
    o_cdf = r16(64 + 2 * L)
    o_max1 = r16(o_cdf + 2 * 2 * entries)
    o_len = r16(o_max1 + 2 * 2 * L * T)
    o_pay = r16(o_len + 2 * 2 * L * T)
    assert oracle.container_payload_offset(L, C, T, Tc, bins) == o_pay
    assert oracle.container_bytes(L, C, T, Tc, bins, 1000) == o_pay + 1008
    assert oracle.container_bytes(L, C, T, Tc, bins, 3) == o_pay + 16
    # the compact rows take (10*30 + 22*14) / (32*32) of the full tables
    full = 2 * 2 * L * C * 32 * 2
    assert (o_max1 - o_cdf) / full == pytest.approx((10 * 30 + 22 * 14) / (32 * 32), abs=1e-4)


def _small():
    cfg = kvgen.CONFIGS["c1"]
    kv, _ = kvgen.generate(cfg)
    bins = cfg.bins()
    r = oracle.codec(kv, bins, cfg.chunk_tokens)
    return cfg, kv, bins, r


def test_rows_the_format_cannot_carry_are_refused():
    cfg, kv, bins, r = _small()
    Tc = cfg.chunk_tokens
    for (c, k, v) in ((3, 20, 1234), (5, 0, 7)):  # layer 1 has 16 bins: entry 20 is implied
        bad = r["cdf"].copy()
        bad[0, 1, 0, c, k] = v
        with pytest.raises(oracle.OracleError):
            oracle.serialize(bad, r["max1"], r["stream_len"], r["payload"], bins, Tc)


def test_headers_that_do_not_match_are_refused():
    cfg, kv, bins, r = _small()
    L, _, T, C = kv.shape
    Tc = cfg.chunk_tokens
    data = oracle.serialize(r["cdf"], r["max1"], r["stream_len"], r["payload"], bins, Tc)
    for args in ((L, C + 1, T, Tc, bins), (L, C, T - 1, Tc, bins), (L, C, T, Tc + 1, bins),
                 (L, C, T, Tc, np.array([[32, 16], [16, 16]], np.int32))):
        with pytest.raises(oracle.OracleError):
            oracle.deserialize(data, *args)
    for pos, val in ((0, 0x4C), (4, 2), (40, 0)):  # magic, version, total size
        bad = data.copy()
        bad[pos] = val
        with pytest.raises(oracle.OracleError):
            oracle.deserialize(bad, L, C, T, Tc, bins)
    with pytest.raises(oracle.OracleError):
        oracle.deserialize(data[:-1], L, C, T, Tc, bins)
    bad = data.copy()  # a stream length that no longer sums to the payload size
    o = oracle.container_payload_offset(L, C, T, Tc, bins) - 16
    bad[o] ^= 1
    with pytest.raises(oracle.OracleError):
        oracle.deserialize(bad, L, C, T, Tc, bins)
