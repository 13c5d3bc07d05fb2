"""Pins of the oracle's range coder.

The write-up entropy-codes the symbols with GPU-parallel arithmetic coding
("1.2 Core challenges and solutions", design point 3; "2.1 Core components";
"2.4 Decoder pipeline", step 1) but prints no coder; the 32-bit range coder
with 16-bit totals, byte renormalisation and a carry cache is the reading
taken.  Pins:
  * byte-identical output of an exact big-integer model (tests/coder_model.py)
    that has no carry cache at all, on random, skewed, carry-heavy and
    exhaustive tiny inputs, with a coverage check that carries through runs of
    0xFF bytes really happen;
  * decode(encode(s)) == s on all of them;
  * the final coding interval contains the number the stream spells;
  * code length within 1% + 4 bytes of the empirical entropy of the chunk;
  * corrupt / truncated streams: defined behaviour, flag raised.
"""
import itertools
import math

import numpy as np
import pytest

import oracle
from coder_model import exact_encode, interval_of


def cdf_from_counts(counts):
    """A valid 16-bit CDF row (f >= 1, total 65536) built from arbitrary counts
    by largest-remainder apportionment: independent of the oracle's formula."""
    A = len(counts)
    budget = 65536 - A
    tot = sum(counts)
    raw = [c * budget / tot for c in counts] if tot else [budget / A] * A
    f = [1 + int(math.floor(r)) for r in raw]
    rem = 65536 - sum(f)
    order = sorted(range(A), key=lambda k: raw[k] - math.floor(raw[k]), reverse=True)
    for k in order[:rem]:
        f[k] += 1
    assert sum(f) == 65536 and min(f) >= 1
    row = np.zeros(A, dtype=np.uint16)
    acc = 0
    for k in range(A):
        row[k] = acc
        acc += f[k]
    return row


def roundtrip(q, rows):
    q = np.asarray(q, dtype=np.uint8)
    rows = np.asarray(rows, dtype=np.uint16)
    data = oracle.encode_stream(q, rows)
    ref, stats = exact_encode(q.tolist(), rows.tolist())
    assert data == ref, (q.tolist(), data.hex(), ref.hex())
    dq, bad = oracle.decode_stream(data, rows)
    assert not bad
    assert np.array_equal(dq, q)
    return data, stats


def test_exhaustive_tiny_alphabets():
    """Every sequence of length <= 5 over A = 4 and A = 5 with skewed, flat and
    extreme (frequency-1) CDFs."""
    shapes = {
        4: [[1, 1, 1, 1], [1000, 1, 1, 1], [1, 1, 1, 1000], [0, 5, 0, 0], [3, 100, 7, 1]],
        5: [[1, 1, 1, 1, 1], [0, 0, 1, 0, 0], [50, 1, 1, 1, 50], [1, 2, 4, 8, 16]],
    }
    n = 0
    for A, shp in shapes.items():
        for counts in shp:
            row = cdf_from_counts(counts)
            for length in range(0, 6):
                rows = np.tile(row, (length, 1)) if length else np.zeros((0, A), np.uint16)
                for q in itertools.product(range(A), repeat=length):
                    if length == 0:
                        continue
                    roundtrip(q, rows)
                    n += 1
    assert n > 8000


def test_carry_heavy_random_matches_big_integer_model():
    """Skewed CDFs where the coded value keeps landing near byte boundaries."""
    rng = np.random.default_rng(2024)
    carries = ff2 = longest = 0
    for trial in range(1500):
        A = int(rng.choice([2, 3, 4, 8, 32, 64]))
        C = int(rng.integers(1, 200))
        rows = []
        for _ in range(C):
            counts = rng.integers(0, 3, A) * rng.integers(1, 40000, A)
            counts[rng.integers(0, A)] += int(rng.integers(0, 60000))
            rows.append(cdf_from_counts(counts.tolist()))
        rows = np.array(rows, dtype=np.uint16)
        if trial % 3 == 0:
            q = rng.integers(0, A, C)  # uniform symbols: many low-probability codes
        else:
            q = np.array([int(rng.choice(A, p=np.diff(np.append(r.astype(np.int64), 65536)) / 65536))
                          for r in rows])
        _, st = roundtrip(q, rows)
        carries += st["carries"]
        ff2 += st["max_ff_run"] >= 2
        longest = max(longest, st["max_ff_run"])
    # random inputs carry often, but rarely through 0xFF runs (see the forced test)
    assert carries > 500, (carries, ff2, longest)


def _straddling_sequence(rows, rng, n_straddle, resolve_up):
    """Symbols that keep the coding interval across the byte boundary B (which
    makes every byte shifted out 0xFF), then one step above B (carry through
    the whole run) or below it (the run stays 0xFF), then random symbols."""
    A = rows.shape[1]
    low, rw, B = 0, 0xFFFFFFFF, 0x80000000
    q = []
    for c in range(rows.shape[0]):
        row = [int(v) for v in rows[c]] + [65536]
        r = rw >> 16
        if c < n_straddle and low <= B < low + r * 65536:
            k = max(i for i in range(A) if low + r * row[i] <= B)
        elif c == n_straddle and low <= B < low + r * 65536:
            k0 = max(i for i in range(A) if low + r * row[i] <= B)
            k = min(k0 + 1, A - 1) if resolve_up else max(k0 - 1, 0)
        else:
            k = int(rng.integers(0, A))
        q.append(k)
        low += r * row[k]
        rw = r * (row[k + 1] - row[k])
        while rw < (1 << 24):
            rw <<= 8
            low <<= 8
            B <<= 8
    return np.array(q, dtype=np.uint8)


def test_forced_ff_runs():
    rng = np.random.default_rng(77)
    longest, carried = 0, 0
    for trial in range(300):
        A = int(rng.choice([2, 4, 16, 32, 64]))
        C = int(rng.integers(20, 160))
        rows = np.array([cdf_from_counts((rng.integers(0, 4, A) * rng.integers(1, 30000, A) + 1).tolist())
                         for _ in range(C)], dtype=np.uint16)
        q = _straddling_sequence(rows, rng, int(rng.integers(1, C)), resolve_up=bool(trial % 2))
        _, st = roundtrip(q, rows)
        longest = max(longest, st["max_ff_run"])
        carried += st["max_ff_run"] >= 3
    assert longest >= 8 and carried > 50, (longest, carried)


def test_interval_contains_stream_value():
    rng = np.random.default_rng(9)
    for _ in range(200):
        A, C = 32, int(rng.integers(1, 300))
        rows = np.array([cdf_from_counts(rng.integers(0, 50, A).tolist()) for _ in range(C)])
        q = rng.integers(0, A, C)
        data = oracle.encode_stream(q.astype(np.uint8), rows)
        low, rng_w, nshift = interval_of(q.tolist(), rows.tolist())
        # the stream spells V = 0.b1 b2 ... in units where the initial window is 2^32
        nb = nshift + 4
        v = int.from_bytes(data.ljust(nb, b"\0")[:nb], "big") if nb else 0
        assert len(data) <= nshift + 1
        assert low <= v < low + rng_w


def test_edge_streams():
    # all symbols at cumulative 0 -> the value is 0 -> an empty stream
    rows = np.tile(cdf_from_counts([10, 1, 1, 1]), (50, 1))
    data, _ = roundtrip(np.zeros(50, np.uint8), rows)
    assert data == b""
    # every symbol of frequency 1: the longest possible stream, <= 2*C + 1 bytes
    rows = np.tile(np.array([0, 65533, 65534, 65535], np.uint16), (300, 1))  # f = 65533, 1, 1, 1
    data, st = roundtrip(np.full(300, 2, np.uint8), rows)
    assert st["nshift"] == 2 * 300 and len(data) <= 2 * 300 + 1
    # a single channel
    roundtrip([1], cdf_from_counts([1, 1])[None, :])


def test_entropy_bound_on_kv_like_data():
    """len <= 1.01 * H/8 + 4 bytes per stream, H = sum_c log2(N / n_{c,q_c}) with
    the chunk's own counts, on generator output quantized by the oracle."""
    import kvgen
    for name, Ls in (("c2", [0, 15]), ("c1", [0, 1])):
        cfg = kvgen.CONFIGS[name].scaled(n_layers=max(Ls) + 1, layer_bins=((0, max(Ls) + 1, 32),))
        kv, _ = kvgen.generate(cfg)
        bins = cfg.bins()
        sym, _ = oracle.quantize(kv, bins)
        A = int(bins.max())
        tab = oracle.cdf(sym, cfg.chunk_tokens, A)
        T, C = cfg.n_tokens, cfg.n_channels
        for l in Ls:
            for kvi in range(2):
                counts = np.stack([np.bincount(sym[l, kvi, :, c], minlength=A) for c in range(C)])
                for t in range(0, T, max(1, T // 32)):
                    q = sym[l, kvi, t]
                    data = oracle.encode_stream(q, tab[0, l, kvi])
                    H = float(np.sum(np.log2(T / counts[np.arange(C), q])))
                    assert len(data) <= 1.01 * H / 8 + 4, (name, l, kvi, t, len(data), H / 8)


def test_corrupt_and_truncated_streams():
    rows = np.tile(cdf_from_counts([5, 20, 5, 1]), (64, 1))
    q, bad = oracle.decode_stream(b"\xff" * 16, rows)
    assert bad and q.shape == (64,)
    rng = np.random.default_rng(1)
    good = oracle.encode_stream(rng.integers(0, 4, 64).astype(np.uint8), rows)
    for cut in range(len(good)):
        q, _ = oracle.decode_stream(good[:cut], rows)  # defined: C symbols, no overrun
        assert q.shape == (64,) and q.max() < 4
