"""The GPU lane coder (entropy_coding_02_amd/csrc/lane_coder.h) compiled for
the host and compared with the oracle stream by stream: byte-identical
encodes (including carries into bytes already written and the trailing-zero
trim reaching back into them) and identical decodes from streams placed at
every byte alignment, up against the exact end of the buffer (the decoder's
buffers are whole dwords, at least 16 bytes)."""
import ctypes
import os
import subprocess

import numpy as np
import pytest

import oracle
from test_oracle_coder import _straddling_sequence, cdf_from_counts

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hostsim", "hostsim.hip")
SANITIZE = os.environ.get("KVC_SANITIZE") == "1"  # host code with AddressSanitizer + UBSan
LIB = os.path.join(HERE, "hostsim", "libhostsim_san.so" if SANITIZE else "libhostsim.so")
HDR = os.path.join(os.path.dirname(HERE), "entropy_coding_02_amd", "csrc", "lane_coder.h")
COMMON = os.path.join(os.path.dirname(HERE), "entropy_coding_02_amd", "csrc", "kvc_common.h")


@pytest.fixture(scope="module")
def hs():
    newest = max(os.path.getmtime(SRC), os.path.getmtime(HDR), os.path.getmtime(COMMON))
    if not os.path.exists(LIB) or os.path.getmtime(LIB) < newest:
        tmp = LIB + f".tmp{os.getpid()}"
        san = []
        if SANITIZE:  # the host side only: each sanitizer flag goes to the host compilation
            san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g",
                   "-shared-libsan"]
        subprocess.check_call(["/opt/rocm/bin/hipcc", "-std=c++17", "-O2", "--offload-arch=gfx950",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", *san,
                               "-fPIC", "-shared", "-o", tmp, SRC])
        os.replace(tmp, LIB)
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    lib.hostsim_encode_stream.restype = ctypes.c_int64
    lib.hostsim_encode_stream.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P]
    lib.hostsim_decode_stream.restype = ctypes.c_int
    lib.hostsim_decode_stream.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32]
    lib.hostsim_encode_stream_split.restype = ctypes.c_int64
    lib.hostsim_encode_stream_split.argtypes = [P, ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32]
    lib.hostsim_xcd_block.restype = ctypes.c_int64
    lib.hostsim_xcd_block.argtypes = [ctypes.c_int64, ctypes.c_int64]
    lib.hostsim_decode_stream_n.restype = ctypes.c_int
    lib.hostsim_decode_stream_n.argtypes = [P, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int32, ctypes.c_int32, P, P, ctypes.c_int32, P]
    lib.hostsim_bytes_ge.restype = ctypes.c_uint32
    lib.hostsim_bytes_ge.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
    return lib


def h_encode(lib, q, rows):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    C, A = rows.shape
    slot = np.full((2 * C + 16 + 15) // 16 * 16, 0xAB, dtype=np.uint8)
    n = lib.hostsim_encode_stream(q.ctypes.data, C, A, rows.ctypes.data, slot.ctypes.data)
    return slot[:n].tobytes()


def h_decode(lib, buf, off, length, rows, cap=None, search=0):
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    C, A = rows.shape
    q = np.empty(C, dtype=np.uint8)
    cap = buf.size if cap is None else cap
    bad = lib.hostsim_decode_stream(buf.ctypes.data, cap, off, length, C, A, rows.ctypes.data,
                                    q.ctypes.data, search)
    assert bad >= 0
    return q, bool(bad)


def h_encode_split(lib, q, rows, G):
    q = np.ascontiguousarray(q, dtype=np.uint8)
    rows = np.ascontiguousarray(rows, dtype=np.uint16)
    C, A = rows.shape
    slot = np.full((2 * C + 16 + 15) // 16 * 16, 0xAB, dtype=np.uint8)
    n = lib.hostsim_encode_stream_split(q.ctypes.data, C, A, rows.ctypes.data, slot.ctypes.data, G)
    return slot[:n].tobytes()


def check(lib, q, rows):
    """The lane coder, and the split coder with 2, 3, 4 and 8 lanes, against the oracle."""
    want = oracle.encode_stream(np.asarray(q, np.uint8), rows)
    got = h_encode(lib, q, rows)
    assert got == want, (len(got), len(want))
    for G in (2, 3, 4, 8):
        got = h_encode_split(lib, q, rows, G)
        assert got == want, (G, len(got), len(want))
    return want


def test_random_and_skewed_streams(hs):
    """Encodes byte-identical to the oracle; decodes (both table searches) give
    the symbols back."""
    rng = np.random.default_rng(31)
    for trial in range(800):
        A = int(rng.choice([2, 4, 6, 8, 12, 16, 32, 40, 64, 256]))
        C = int(rng.integers(1, 300))
        rows = np.array([cdf_from_counts((rng.integers(0, 3, A) * rng.integers(1, 40000, A)).tolist())
                         for _ in range(C)], dtype=np.uint16)
        q = rng.integers(0, A, C).astype(np.uint8)
        data = check(hs, q, rows)
        buf = np.frombuffer(data + bytes(max(16, (len(data) + 4) // 4 * 4) - len(data)), np.uint8).copy()
        for search in (0, 1, 2):
            got, bad = h_decode(hs, buf, 0, len(data), rows, search=search)
            assert not bad and np.array_equal(got, q), (trial, search)


def test_forced_carries_through_written_bytes(hs):
    """Straddling sequences: runs of 0xFF long enough that the carry reaches
    dwords the lane has already written."""
    rng = np.random.default_rng(77)
    for trial in range(600):
        A = int(rng.choice([2, 4, 16, 32, 64]))
        C = int(rng.integers(20, 200))
        rows = np.array([cdf_from_counts((rng.integers(0, 4, A) * rng.integers(1, 30000, A) + 1).tolist())
                         for _ in range(C)], dtype=np.uint16)
        q = _straddling_sequence(rows, rng, int(rng.integers(1, C)), resolve_up=bool(trial % 2))
        check(hs, q, rows)


def test_zero_tail_trim_reaches_written_dwords(hs):
    rows = np.tile(cdf_from_counts([10, 1, 1, 1]), (400, 1))
    for n_tail in range(0, 40):
        q = np.zeros(400, np.uint8)
        q[: 400 - n_tail - 1] = np.random.default_rng(n_tail).integers(0, 4, 400 - n_tail - 1)
        check(hs, q, rows)  # the final all-zero symbols give trailing zero bytes
    check(hs, np.zeros(400, np.uint8), rows)  # empty stream


@pytest.mark.parametrize("search", [0, 1, 2])
def test_decode_every_alignment_up_to_buffer_end(hs, search):
    """Streams at every byte alignment; the buffer ends right after the last
    stream (rounded up to whole dwords, the padding filled with junk that
    must be masked off), so the reader's clamped loads are exercised."""
    rng = np.random.default_rng(5)
    A, C = 32, 96
    rows = np.array([cdf_from_counts(rng.integers(0, 60, A).tolist()) for _ in range(C)], dtype=np.uint16)
    streams, syms = [], []
    for i in range(40):
        q = rng.integers(0, A, C).astype(np.uint8)
        syms.append(q)
        streams.append(check(hs, q, rows))
    streams.append(b"")  # an empty stream at the very end
    syms.append(None)
    for lead in range(8):  # stream start at every byte alignment
        body = bytes(lead) + b"".join(streams)
        pad = (-len(body)) % 4
        buf = np.frombuffer(body + b"\xa5" * pad, dtype=np.uint8).copy()
        off = lead
        for q, s in zip(syms, streams):
            got, bad = h_decode(hs, buf, off, len(s), rows, search=search)
            if q is not None:
                assert not bad and np.array_equal(got, q)
            off += len(s)


@pytest.mark.parametrize("search", [0, 1, 2])
def test_corrupt_streams_match_oracle_flag(hs, search):
    for rows in (np.tile(cdf_from_counts([5, 20, 5, 1]), (64, 1)),
                 np.tile(np.array([0] + list(range(65504, 65535)), np.uint16), (64, 1))):  # f=1 tail
        A = rows.shape[1]
        for data in (b"\xff" * 16, b"\xfe\xff\xff\xff\x00", bytes(range(200, 256)), b"\xff\xfe" * 9):
            buf = np.frombuffer(data + bytes(max(16 - len(data), (-len(data)) % 4)), np.uint8).copy()
            q_o, bad_o = oracle.decode_stream(data, rows)
            q_h, bad_h = h_decode(hs, buf, 0, len(data), rows, search=search)
            assert bad_o == bad_h and np.array_equal(q_o, q_h)


def test_xcd_block_renumbering_is_a_bijection(hs):
    """The kernels' XCD-aware block numbering covers every block exactly once
    and gives the blocks of one XCD (b % 8) consecutive numbers."""
    for nb in list(range(0, 70)) + [255, 256, 257, 1024, 4099, 16384]:
        got = [hs.hostsim_xcd_block(b, nb) for b in range(nb)]
        assert sorted(got) == list(range(nb)), nb
        per = nb // 8
        for x in range(8):
            mine = sorted(got[b] for b in range(x, 8 * per, 8))
            assert mine == list(range(x * per, (x + 1) * per)), (nb, x)


def test_bytes_ge_exhaustive(hs):
    """The kernels' packed check for symbol bytes >= A (what raises
    KVC_DEV_BAD_SYMBOL in the CDF and encoder kernels): for every even A in
    [4, 256] and every byte value in every byte position (the other bytes
    0 or A - 1, the largest valid symbol), bit 7 of exactly the bytes >= A is
    set; plus random dwords against a byte-by-byte comparison."""
    rng = np.random.default_rng(5)
    rand = rng.integers(0, 2**32, 400, dtype=np.uint64)
    for A in range(4, 257, 2):
        for fill in (0, A - 1):
            for pos in range(4):
                for b in range(256):
                    w = 0
                    for k in range(4):
                        w |= (b if k == pos else fill) << (8 * k)
                    got = hs.hostsim_bytes_ge(w, A)
                    want = (0x80 << (8 * pos)) if b >= A else 0
                    assert got == want, (A, fill, pos, b, hex(got))
        for w in rand:
            w = int(w)
            want = 0
            for k in range(4):
                if ((w >> (8 * k)) & 0xFF) >= A:
                    want |= 0x80 << (8 * k)
            assert hs.hostsim_bytes_ge(w, A) == want, (A, hex(w))


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_mode_first_decoder_on_kv_streams(hs, name):
    """The mode-first decoder (search 2: the mode record's symbol tried first,
    the exact two-level search otherwise, bits from the byte-position window)
    decodes every stream of a KV-shaped slab set back to the oracle's
    symbols, streams packed back to back at their payload offsets, and takes
    its fast path for most symbols of these workloads."""
    import kvgen
    cfg = kvgen.CONFIGS[name].scaled(n_layers=4, n_tokens=300, layer_bins=((0, 2, int(kvgen.CONFIGS[name].bins().max())), (2, 4, 16)))
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    r = oracle.codec(kv, bins, Tc)
    L, T, C, A = cfg.n_layers, cfg.n_tokens, cfg.n_channels, r["A"]
    pay = r["payload"]
    buf = np.concatenate([pay, np.full((-pay.size) % 4 + 16, 0xA5, np.uint8)])
    fast = ctypes.c_int64(0)
    sid, total = 0, 0
    for j in range((T + Tc - 1) // Tc):
        nj = min(Tc, T - j * Tc)
        for lk in range(2 * L):
            rows = np.ascontiguousarray(r["cdf"][j, lk // 2, lk % 2])
            off = int(r["slab_off"][j * 2 * L + lk])
            for t in range(nj):
                n = int(r["stream_len"][sid])
                q = np.empty(C, np.uint8)
                bad = hs.hostsim_decode_stream_n(buf.ctypes.data, pay.size + (-pay.size) % 4, off, n, C, A,
                                                 rows.ctypes.data, q.ctypes.data, 2, ctypes.byref(fast))
                assert bad == 0
                assert np.array_equal(q, r["sym"][lk // 2, lk % 2, j * Tc + t]), (j, lk, t)
                off += n
                sid += 1
                total += C
    assert fast.value > 0.3 * total, (fast.value, total)
