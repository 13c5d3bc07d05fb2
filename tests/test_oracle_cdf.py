"""Pins of the oracle's per-(chunk, layer, K|V, channel) histogram + CDF.

The write-up computes symbol frequencies of the quantized tensor and turns
them into a CDF whose width is the largest bins value ("2.3 Encoder
pipeline", step 2), per 256-token chunk (step 3).  The 16-bit total with a
minimum frequency of 1 is the reading taken here: cdf_k = k + floor(C_k * K / N)
with K = 65536 - A.  Pins, none of which re-types that formula:
  * counts: numpy.bincount of each column (a library routine);
  * cdf_0 = 0, strictly increasing, last frequency 65536 - cdf_{A-1} >= 1;
  * n_s*K/N < f_s < n_s*K/N + 2 for every symbol (floor arithmetic);
  * a constant column puts 65536-(A-1) on its symbol and 1 elsewhere;
  * equal counts with A | 65536 give exactly uniform frequencies 65536/A.
"""
import numpy as np
import pytest

import oracle


def freqs(row):
    row = row.astype(np.int64)
    return np.diff(np.concatenate([row, [65536]]))


def check_slab(col_syms, row, A):
    """col_syms: symbols of one channel over the chunk's tokens; row: its CDF."""
    N = col_syms.size
    K = 65536 - A
    n = np.bincount(col_syms, minlength=A)[:A]
    f = freqs(row)
    assert row[0] == 0
    assert (f >= 1).all()
    lo = n * K / N
    assert (f > lo - 1e-9).all() and (f < lo + 2).all()
    assert f.sum() == 65536


@pytest.mark.parametrize("T,Tc", [(256, 256), (300, 256), (64, 256), (1000, 100), (7, 3)])
@pytest.mark.parametrize("A", [4, 32, 64, 256])
def test_invariants_random(T, Tc, A):
    rng = np.random.default_rng(T * 7 + A)
    L, C = 2, 24
    # peaked symbols like real quantized KV, plus a few uniform channels
    center = A // 2
    sym = np.clip(np.rint(rng.standard_normal((L, 2, T, C)) * rng.uniform(0.3, A / 4, (L, 2, 1, C)) + center),
                  0, A - 1).astype(np.uint8)
    sym[:, :, :, 0] = rng.integers(0, A, (L, 2, T))
    tab = oracle.cdf(sym, Tc, A)
    NC = oracle.n_chunks(T, Tc)
    assert tab.shape == (NC, L, 2, C, A)
    for j in range(NC):
        t0, nj = j * Tc, oracle.chunk_tokens(T, Tc, j)
        for l in range(L):
            for kv in range(2):
                for c in range(C):
                    check_slab(sym[l, kv, t0:t0 + nj, c], tab[j, l, kv, c], A)


@pytest.mark.parametrize("A", [4, 16, 32, 64, 256])
def test_constant_column(A):
    T = 256
    sym = np.zeros((1, 2, T, A), dtype=np.uint8)
    for c in range(A):
        sym[0, :, :, c] = c  # channel c is constant at symbol c
    tab = oracle.cdf(sym, 256, A)
    for c in range(A):
        f = freqs(tab[0, 0, 0, c])
        want = np.ones(A, dtype=np.int64)
        want[c] = 65536 - (A - 1)
        assert np.array_equal(f, want)


@pytest.mark.parametrize("A", [4, 16, 32, 64, 256])
def test_uniform_counts(A):
    reps = 2
    T = A * reps
    col = np.repeat(np.arange(A, dtype=np.uint8), reps)
    sym = np.ascontiguousarray(np.broadcast_to(col[None, None, :, None], (1, 2, T, 3)))
    tab = oracle.cdf(sym, T, A)
    assert all((freqs(tab[0, 0, kv, c]) == 65536 // A).all() for kv in range(2) for c in range(3))


def test_chunks_are_independent():
    """Changing tokens of chunk 1 leaves chunk 0's CDFs alone."""
    rng = np.random.default_rng(5)
    sym = rng.integers(0, 16, (1, 2, 512, 8)).astype(np.uint8)
    a = oracle.cdf(sym, 256, 16)
    sym2 = sym.copy()
    sym2[:, :, 300:] = 3
    b = oracle.cdf(sym2, 256, 16)
    assert np.array_equal(a[0], b[0]) and not np.array_equal(a[1], b[1])


def test_symbol_out_of_alphabet_rejected():
    sym = np.full((1, 2, 4, 4), 16, dtype=np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.cdf(sym, 256, 16)


def test_floor_reading_worked_by_hand():
    """The normalisation reading is floor, not round-to-nearest.  Worked by hand
    for N = 7 tokens, A = 4, counts (3, 2, 2, 0), K = 65532:
      C = 0, 3, 5, 7;  3*65532/7 = 28085.14..;  5*65532/7 = 46808.57..;  7*65532/7 = 65532
      cdf = 0, 1 + 28085, 2 + 46808, 3 + 65532 = 0, 28086, 46810, 65535."""
    col = np.array([0, 0, 0, 1, 1, 2, 2], dtype=np.uint8)
    sym = np.ascontiguousarray(np.broadcast_to(col[None, None, :, None], (1, 2, 7, 1)))
    tab = oracle.cdf(sym, 256, 4)
    assert tab[0, 0, 0, 0].tolist() == [0, 28086, 46810, 65535]
