"""The CDF kernels compute floor(Ck * K / N) (K = 65536 - A, N tokens of a
chunk) as the integer part of fl(fl(x * rn) + 2^-18) with x = Ck * K and
rn = 1/N rounded to double (kvc_common.h, kvc_cdf_entry), instead of an
integer division.  These checks run the same IEEE double operations with
numpy against exact integer division: every N that a chunk can have, the
counts that matter most (0, 1, N - 1, N and random ones) for several
alphabets, and every count for the chunk sizes the workloads use."""
import numpy as np

BIAS = 2.0 ** -18


def device_floor(x, n):
    rn = 1.0 / n.astype(np.float64)
    return np.floor(x.astype(np.float64) * rn + BIAS).astype(np.int64)


def test_every_chunk_size_edge_counts():
    rng = np.random.default_rng(0)
    n = np.arange(1, 65536, dtype=np.int64)
    for A in (4, 16, 32, 64, 256):
        K = 65536 - A
        for ck in (np.zeros_like(n), np.ones_like(n), n - 1, n, n // 2, n // 3 + 1,
                   rng.integers(0, n + 1)):
            x = ck * K
            assert x.max() < 2 ** 32
            np.testing.assert_array_equal(device_floor(x, n), x // n)


def test_all_counts_for_workload_chunk_sizes():
    for N in (1, 2, 3, 7, 64, 128, 255, 256, 1000, 4096, 65535):
        ck = np.arange(0, N + 1, dtype=np.int64)
        for A in (16, 32, 64):
            x = ck * (65536 - A)
            np.testing.assert_array_equal(device_floor(x, np.full_like(ck, N)), x // N)


def test_exact_multiples_are_not_rounded_down():
    # x = m * N exactly: the product may fall just below m without the bias
    n = np.arange(1, 65536, dtype=np.int64)
    for m in (1, 255, 65535, 65532):
        x = m * n
        keep = x < 2 ** 32
        np.testing.assert_array_equal(device_floor(x[keep], n[keep]), np.full(keep.sum(), m))
