"""Exact big-integer model of the range coder, used to pin the oracle's
byte-wise coder (carry cache, pending 0xFF bytes, flush and trimming).

The model never emits bytes while coding.  It keeps `low` as one unbounded
Python integer, so a carry simply propagates through integer addition, and
only at the end writes the number out in base 256.  It shares the coder's
interval rule (r = range >> 16; low += r*cdf_s; range = r*f_s; scale by 256
while range < 2^24; round low up to a multiple of 2^24 at the end) but none of
its byte-emission mechanics, which is what it checks.

It also counts the carries that reach bytes already shifted out of the 32-bit
window, and the longest run of 0xFF bytes such a carry rippled through, so a
test can show that its inputs exercise the carry path.
"""
from __future__ import annotations


def _cdf(row, A, k):
    return 65536 if k >= A else int(row[k])


def exact_encode(q, cdf_rows):
    """q: sequence of symbols; cdf_rows: [C][A] ints.  Returns (bytes, stats)."""
    A = len(cdf_rows[0]) if len(cdf_rows) else 2
    low, rng, nshift = 0, 0xFFFFFFFF, 0
    carries, max_run = 0, 0
    for c, s in enumerate(q):
        row = cdf_rows[c]
        lo, hi = _cdf(row, A, s), _cdf(row, A, s + 1)
        r = rng >> 16
        before = low >> 32
        low += r * lo
        after = low >> 32
        if after != before:
            carries += 1
            # the bytes above the window that flipped: trailing 0xFF of `before`
            run, b = 0, before
            while b & 0xFF == 0xFF:
                run += 1
                b >>= 8
            max_run = max(max_run, run)
        rng = r * (hi - lo)
        while rng < (1 << 24):
            rng <<= 8
            low <<= 8
            nshift += 1
    v = (low + (1 << 24) - 1) >> 24
    raw = v.to_bytes(nshift + 2, "big")
    assert raw[0] == 0, "leading byte must be zero"
    return raw[1:].rstrip(b"\0"), dict(carries=carries, max_ff_run=max_run, nshift=nshift)


def interval_of(q, cdf_rows):
    """Exact final coding interval [low, low+range) scaled to 256^nshift, and nshift."""
    A = len(cdf_rows[0])
    low, rng, nshift = 0, 0xFFFFFFFF, 0
    for c, s in enumerate(q):
        row = cdf_rows[c]
        lo, hi = _cdf(row, A, s), _cdf(row, A, s + 1)
        r = rng >> 16
        low += r * lo
        rng = r * (hi - lo)
        while rng < (1 << 24):
            rng <<= 8
            low <<= 8
            nshift += 1
    return low, rng, nshift
