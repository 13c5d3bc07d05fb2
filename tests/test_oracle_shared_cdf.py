"""Pins of the oracle's shared CDF tables (one table per S consecutive
chunks): a group's table is the one-chunk table of the group's tokens (the
per-chunk CDF, already pinned, over a chunk S times as long); every stream of
chunk j is the stream the single-table coder writes for the same row with
table floor(j / S); the tables match a brute-force count with exact rational
floors on a tiny case; decode inverts encode; and S at or past the chunk
count means one table per (layer, K|V, channel)."""
from fractions import Fraction

import numpy as np
import pytest

import kvgen
import oracle


def _case(L, C, T, Tc, seed):
    cfg = kvgen.CONFIGS["c1"].scaled(n_layers=L, n_channels=C, n_tokens=T, chunk_tokens=Tc,
                                     layer_bins=((0, 1, 32), (1, L, 16)), seed=seed, rho=0.9)
    kv, _ = kvgen.generate(cfg)
    bins = cfg.bins()
    sym, max1 = oracle.quantize(kv, bins)
    return kv, bins, sym, int(bins.max())


@pytest.mark.parametrize("S", [1, 2, 3, 5, 99])
def test_group_table_is_the_one_chunk_table_of_its_tokens(S):
    L, C, T, Tc = 2, 24, 330, 32  # 11 chunks, the last of 10 tokens
    _, bins, sym, A = _case(L, C, T, Tc, 41)
    tab = oracle.cdf(sym, Tc, A, S)
    Se, NG = oracle.tables_of(T, Tc, S)
    assert Se == min(S, 11) and NG == -(-11 // Se) and tab.shape[0] == NG
    span = Se * Tc
    for g in range(NG):
        part = np.ascontiguousarray(sym[:, :, g * span:(g + 1) * span])
        one = oracle.cdf(part, part.shape[2], A)  # one chunk holding the group's tokens
        assert one.shape[0] == 1
        assert np.array_equal(tab[g], one[0]), g


@pytest.mark.parametrize("S", [2, 4, 99])
def test_streams_use_their_groups_table(S):
    L, C, T, Tc = 2, 24, 200, 16  # 13 chunks, the last of 8 tokens
    _, bins, sym, A = _case(L, C, T, Tc, 42)
    tab = oracle.cdf(sym, Tc, A, S)
    stream_len, slab_off, payload = oracle.encode(sym, tab, Tc, A, tab_chunks=S)
    Se, _ = oracle.tables_of(T, Tc, S)
    NC = oracle.n_chunks(T, Tc)
    sid = 0
    for j in range(NC):
        nj = oracle.chunk_tokens(T, Tc, j)
        for l in range(L):
            for kv in range(2):
                off = int(slab_off[(j * L + l) * 2 + kv])
                for t in range(nj):
                    n = int(stream_len[sid])
                    want = oracle.encode_stream(sym[l, kv, j * Tc + t], tab[j // Se, l, kv])
                    assert payload[off:off + n].tobytes() == want, (j, l, kv, t)
                    off += n
                    sid += 1
    # the whole tensor with one shared table equals the one-chunk coding of it
    if S >= NC:
        one_tab = oracle.cdf(sym, T, A)
        one_len, _, one_pay = oracle.encode(sym, one_tab, T, A)
        assert np.array_equal(tab, one_tab)
        assert sorted(stream_len.tolist()) == sorted(one_len.tolist())
        assert payload.size == one_pay.size
    dsym, bad = oracle.decode(payload, slab_off, stream_len, tab, L, C, T, Tc, A, S)
    assert not bad and np.array_equal(dsym, sym)
    # coded with per-chunk tables the bytes differ: the index is not ignored
    tab1 = oracle.cdf(sym, Tc, A, 1)
    _, _, pay1 = oracle.encode(sym, tab1, Tc, A)
    assert pay1.tobytes() != payload.tobytes()


def test_tables_match_brute_force_counts():
    # L = 1, C = 2, T = 7, Tc = 2, S = 3: groups of tokens [0, 6) and [6, 7)
    A = 6
    rng = np.random.default_rng(5)
    sym = rng.integers(0, A - 1, size=(1, 2, 7, 2)).astype(np.uint8)  # symbols up to A - 2
    sym[0, 0, :6, 0] = 2  # one constant column in the first group
    tab = oracle.cdf(sym, 2, A, 3)
    assert tab.shape == (2, 1, 2, 2, A)
    K = 65536 - A
    for g, (t0, t1) in enumerate([(0, 6), (6, 7)]):
        for kv in range(2):
            for c in range(2):
                col = sym[0, kv, t0:t1, c].tolist()
                N = len(col)
                for k in range(A):
                    Ck = sum(1 for s in col if s < k)
                    assert tab[g, 0, kv, c, k] == k + int(Fraction(Ck * K, N)), (g, kv, c, k)
    # the constant column: every token is symbol 2, so entries jump by K at k = 3
    assert tab[0, 0, 0, 0].tolist() == [0, 1, 2, 3 + K, 4 + K, 5 + K]


def test_codec_round_trip_and_container_with_shared_tables():
    L, C, T, Tc = 2, 16, 150, 32  # 5 chunks
    kv, bins, sym, A = _case(L, C, T, Tc, 43)
    for S in (1, 2, 5):
        r = oracle.codec(kv, bins, Tc, S)
        assert not r["corrupt"] and np.array_equal(r["dec_sym"], r["sym"])
        blob = oracle.serialize(r["cdf"], r["max1"], r["stream_len"], r["payload"], bins, Tc, S)
        back = oracle.deserialize(blob, L, C, T, Tc, bins, S)
        assert np.array_equal(back["cdf"], r["cdf"])
        assert np.array_equal(back["slab_off"], r["slab_off"])
        # fewer tables, smaller container section: NG tables of the per-chunk size
        NG = oracle.tables_of(T, Tc, S)[1]
        per_table = C * int((bins - 2).sum()) * 2
        assert blob.size == oracle.container_bytes(L, C, T, Tc, bins, r["payload"].size, S)
        assert oracle.container_payload_offset(L, C, T, Tc, bins, 1) - \
            oracle.container_payload_offset(L, C, T, Tc, bins, S) == \
            (-(-(80 + 5 * per_table) // 16) - -(-(80 + NG * per_table) // 16)) * 16
        # a chunk's own container carries its group's table and decodes alone
        for j in range(oracle.n_chunks(T, Tc)):
            c = oracle.serialize_chunk(r, j, bins, T, Tc, S)
            nj = oracle.chunk_tokens(T, Tc, j)
            d = oracle.deserialize(c, L, C, nj, Tc, bins)
            assert np.array_equal(d["cdf"][0], r["cdf"][j // S])
            pay = c[d["payload_offset"]:d["payload_offset"] + d["payload_bytes"]]
            ds, bad = oracle.decode(pay, d["slab_off"], d["stream_len"], d["cdf"], L, C, nj, Tc, A)
            assert not bad and np.array_equal(ds, r["sym"][:, :, j * Tc:j * Tc + nj])
