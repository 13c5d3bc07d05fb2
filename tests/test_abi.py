"""libkvc.so loads and exports every entry point include/kvc.h declares, and
its host-side size queries and argument checks behave (no GPU needed: these
calls return before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "kvc.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvc_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kvc.LIB_PATH):
        from entropy_coding_02_amd import build
        build.build()
    return kvc.lib()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kvc.EXPORTED)
    assert kvc.kvc_version() == 1


def test_sizes_match_layout(lib):
    for name, cfg in kvgen.CONFIGS.items():
        d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.bins(), cfg.chunk_tokens)
        NC = -(-cfg.n_tokens // cfg.chunk_tokens)
        A = int(cfg.bins().max())
        assert d.alphabet == A
        assert d.n_chunks == NC
        assert d.n_slabs == NC * 2 * cfg.n_layers
        assert d.n_streams == 2 * cfg.n_layers * cfg.n_tokens
        assert d.cdf_bytes == NC * 2 * cfg.n_layers * cfg.n_channels * A * 2
        slot = (2 * cfg.n_channels + 16 + 15) // 16 * 16
        lanes = d.n_slabs * -(-cfg.chunk_tokens // 256) * 256
        assert d.scratch_bytes == lanes * slot + 8 * d.n_slabs
        assert d.max_payload_bytes == d.n_streams * (2 * cfg.n_channels + 1)
    # the write-up's validation shape: 256 tokens = one chunk, 16,384 streams
    c2 = kvgen.CONFIGS["c2"]
    d = kvc.Desc(c2.n_layers, c2.n_channels, c2.n_tokens, c2.bins())
    assert d.n_chunks == 1 and d.n_streams == 16384 and d.cdf_bytes == 4194304


@pytest.mark.parametrize("T,bins,lanes", [
    (256, 32, 4),      # 16384 streams, rows of 32: four lanes per stream
    (257, 32, 1),      # one stream more: one lane
    (256, 64, 8),      # rows of 64: eight lanes (slices of 8 entries)
    (256, 16, 4), (256, 6, 4),
    (256, 4, 1),       # rows of 4: binary lifting, one lane
    (256, 256, 1),     # rows of 256
])
def test_decode_lanes_rule(lib, T, bins, lanes):
    d = kvc.Desc(32, 1024, T, np.full((32, 2), bins, np.int32))
    assert d.decode_lanes == lanes
    bad = kvc.Desc(1, 0, 64, [[32, 16]])
    assert lib.kvc_decode_lanes(bad.ref) == kvc.KVC_ERR_ARG


@pytest.mark.parametrize("bad", [
    dict(bins=[[3, 16]]), dict(bins=[[2, 16]]), dict(bins=[[258, 16]]), dict(bins=[[31, 16]]),
    dict(n_channels=0), dict(n_channels=16385), dict(chunk_tokens=0), dict(chunk_tokens=65536),
    dict(n_tokens=-1),
])
def test_invalid_descriptors_rejected(lib, bad):
    args = dict(n_layers=1, n_channels=16, n_tokens=64, bins=[[32, 16]], chunk_tokens=256)
    args.update(bad)
    d = kvc.Desc(args["n_layers"], args["n_channels"], args["n_tokens"], args["bins"], args["chunk_tokens"])
    assert lib.kvc_alphabet(d.ref) == kvc.KVC_ERR_ARG
    assert lib.kvc_scratch_bytes(d.ref) == kvc.KVC_ERR_ARG
    # compute entry points reject before touching the GPU
    assert lib.kvc_quantize(d.ref, 16, 16, 16, None, None, None) == kvc.KVC_ERR_ARG


def test_null_and_misaligned_pointers_rejected(lib):
    d = kvc.Desc(1, 16, 64, [[32, 16]])
    assert lib.kvc_quantize(d.ref, None, 64, 64, None, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_quantize(d.ref, 66, 64, 64, None, None, None) == kvc.KVC_ERR_ARG  # kv % 4 != 0
    assert lib.kvc_encode(d.ref, 64, 64, 64, 1, 64, 64, 64, 100, None, None) == kvc.KVC_ERR_CAPACITY
    assert lib.kvc_decode(d.ref, 64, 16, 64, 64, 64, 64, None, 64, 7, None, None) == kvc.KVC_ERR_ARG
    # payload_bytes must be a whole number of dwords, at least four
    for nb in (0, 2, 4, 10, 12, 18):
        assert lib.kvc_decode(d.ref, 64, nb, 64, 64, 64, 64, None, 64, 0, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_dequantize(d.ref, 64, 64, 64, 9, None) == kvc.KVC_ERR_ARG
    # kvc_cdf: null symbols, misaligned CDF or status
    assert lib.kvc_cdf(d.ref, None, 64, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_cdf(d.ref, 64, 66, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_cdf(d.ref, 64, 64, 66, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_status_string(kvc.KVC_ERR_CAPACITY) == b"buffer too small"


def test_container_sizes_agree_with_the_oracle(lib):
    import oracle
    cases = [(c.n_layers, c.n_channels, c.n_tokens, c.chunk_tokens, c.bins()) for c in kvgen.CONFIGS.values()]
    cases += [(3, 40, 0, 256, np.array([[32, 16], [8, 6], [256, 4]], np.int32)),
              (1, 7, 70, 32, np.array([[16, 16]], np.int32))]
    for L, C, T, Tc, bins in cases:
        for S in (0, 1, 4, 1 << 30):  # a table per chunk (0 and 1), per 4 chunks, per tensor
            d = kvc.Desc(L, C, T, bins, Tc, cdf_chunks=S)
            So = max(S, 1)
            assert d.container_payload_offset == oracle.container_payload_offset(L, C, T, Tc, bins, So)
            assert d.container_payload_offset % 16 == 0
            for pb in (0, 1, 15, 16, 17, 123457):
                assert d.container_bytes(pb) == oracle.container_bytes(L, C, T, Tc, bins, pb, So)
            NG = oracle.tables_of(T, Tc, So)[1]
            assert d.cdf_bytes == NG * 2 * L * C * int(np.max(bins)) * 2


def test_container_calls_reject_bad_arguments(lib):
    d = kvc.Desc(1, 16, 64, [[32, 16]])
    need = d.container_bytes(0)
    ok = 1 << 20  # a 16-byte aligned stand-in address; nothing is launched on these paths
    # null or misaligned container, capacity below the empty container
    assert lib.kvc_serialize(d.ref, ok, ok, ok, ok, ok, None, need, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_serialize(d.ref, ok, ok, ok, ok, ok, ok + 4, need, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_serialize(d.ref, ok, ok, ok, ok, ok, ok, need - 1, None, None) == kvc.KVC_ERR_CAPACITY
    assert lib.kvc_serialize(d.ref, None, ok, ok, ok, ok, ok, need, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_deserialize(d.ref, None, need, ok, ok, ok, ok, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_deserialize(d.ref, ok + 8, need, ok, ok, ok, ok, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_deserialize(d.ref, ok, need - 16, ok, ok, ok, ok, None, None) == kvc.KVC_ERR_CAPACITY
    assert lib.kvc_deserialize(d.ref, ok, need, ok, ok, ok, ok + 4, None, None) == kvc.KVC_ERR_ARG
    assert lib.kvc_container_bytes(d.ref, -1) == kvc.KVC_ERR_ARG


def test_stream_work_bytes_and_argument_checks(lib):
    """kvc_stream_work_bytes: the automatic unit is the larger of about
    sqrt(2 NC) chunks and about 2^17 streams (at most NC chunks), the
    workspace grows with the unit, mismatched levels are refused;
    kvc_stream_encode refuses null arguments and out-of-range levels before
    any HIP call."""
    L, C, T, Tc = 2, 64, 1000, 64  # 16 chunks of 256 streams
    a, b = kvc.Desc(L, C, T, [[32, 16], [16, 8]], Tc), kvc.Desc(L, C, T, [[8, 8], [4, 4]], Tc)
    w = [kvc.kvc_stream_work_bytes([a, b], u) for u in range(1, 17)]
    assert all(x < y for x, y in zip(w, w[1:]))
    assert kvc.kvc_stream_work_bytes([a, b], 0) == w[-1]      # 2^17 streams > 16 chunks: all of them
    assert kvc.kvc_stream_work_bytes([a, b], 99) == w[-1]     # capped at NC
    assert kvc.kvc_stream_work_bytes([a], 4) <= kvc.kvc_stream_work_bytes([a, b], 4)
    big = kvc.Desc(32, 1024, 80000, np.full((32, 2), 32, np.int32), 256)  # 16384 streams a chunk, 313 chunks
    assert kvc.kvc_stream_work_bytes([big], 0) == kvc.kvc_stream_work_bytes([big], 25)  # floor(sqrt(626))
    mid = kvc.Desc(32, 1024, 8192, np.full((32, 2), 32, np.int32), 256)  # 32 chunks: 2^17 streams = 8 of them
    assert kvc.kvc_stream_work_bytes([mid], 0) == kvc.kvc_stream_work_bytes([mid], 8)
    for bad in ([a, kvc.Desc(L, C, T + 1, [[32, 16], [16, 8]], Tc)], [a, kvc.Desc(L, 32, T, [[32, 16], [16, 8]], Tc)]):
        with pytest.raises(kvc.KvcError):
            kvc.kvc_stream_work_bytes(bad, 1)
    arr = (kvc.KvcDesc * 2)(a.c, b.c)
    assert lib.kvc_stream_work_bytes(arr, 0, 1) == kvc.KVC_ERR_ARG
    assert lib.kvc_stream_work_bytes(arr, 5, 1) == kvc.KVC_ERR_ARG
    assert lib.kvc_stream_work_bytes(arr, 2, -1) == kvc.KVC_ERR_ARG
    ok = 1 << 20
    ptrs = (ctypes.c_void_p * 2)(ok, ok)
    levels = np.zeros(16, np.int32)
    none_fn = ctypes.cast(None, kvc.CHUNK_FN)

    def call(level_ptr, syms=ptrs, max1=ok, work=ok, host=ok, sizes=ok):
        return lib.kvc_stream_encode(arr, 2, level_ptr, syms, ptrs, max1, 1, work, 1 << 40, host, 1 << 30,
                                     sizes, None, None, None, none_fn, None)
    assert call(None) == kvc.KVC_ERR_ARG
    assert call(levels.ctypes.data, max1=None) == kvc.KVC_ERR_ARG
    assert call(levels.ctypes.data, work=ok + 16) == kvc.KVC_ERR_ARG   # not 256-byte aligned
    assert call(levels.ctypes.data, host=None) == kvc.KVC_ERR_ARG
    assert call(levels.ctypes.data, sizes=ok + 4) == kvc.KVC_ERR_ARG
    assert call(levels.ctypes.data, syms=(ctypes.c_void_p * 2)(ok, None)) == kvc.KVC_ERR_ARG
    for lv in (-1, 2):
        bad = levels.copy()
        bad[7] = lv
        assert call(bad.ctypes.data) == kvc.KVC_ERR_ARG


def test_shared_table_limits(lib):
    """cdf_chunks < 0 is refused; a table may count at most 2^21 tokens."""
    b = np.full((1, 2), 16, np.int32)
    assert kvc.Desc(1, 8, 100, b, 10, cdf_chunks=-1).c and \
        lib.kvc_cdf_bytes(kvc.Desc(1, 8, 100, b, 10, cdf_chunks=-1).ref) == kvc.KVC_ERR_ARG
    T = (1 << 21) + 256
    assert lib.kvc_cdf_bytes(kvc.Desc(1, 8, T, b, 256, cdf_chunks=1 << 20).ref) == kvc.KVC_ERR_ARG
    ok = kvc.Desc(1, 8, T, b, 256, cdf_chunks=(1 << 21) // 256)  # exactly 2^21 tokens per table
    assert ok.cdf_bytes == 2 * 2 * 8 * 16 * 2
    assert lib.kvc_cdf_bytes(kvc.Desc(1, 8, 1 << 21, b, 256, cdf_chunks=1 << 30).ref) > 0
