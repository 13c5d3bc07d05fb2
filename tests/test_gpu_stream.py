"""GPU streaming encoder (kvc_stream_encode): encode a unit of chunks on one
stream while the containers of the unit before copy to page-locked host
memory on another, each chunk at the level a schedule gives it.  Every
container that lands in host memory must be byte-identical to the oracle's
container of that chunk at that level (oracle.serialize_chunk), with units of
one chunk, of several, and the automatic size; on two streams and on one;
the callbacks come in chunk order with the same bytes; a host buffer that is
too small is refused mid-stream without a copy past its end."""
import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


def _cfg(L, C, T, Tc, seed):
    return kvgen.CONFIGS["c1"].scaled(n_layers=L, n_channels=C, n_tokens=T, chunk_tokens=Tc,
                                      layer_bins=((0, 1, 32), (1, L, 16)), seed=seed, rho=0.95)


def _tables(b0):
    out = [b0, np.maximum(b0 // 2, 4), np.maximum(b0 // 4, 4)]
    return [(t + (t % 2)).astype(np.int32) for t in out]


CASES = {
    # ragged last chunk (300 = 4 x 64 + 44), 16-byte symbol rows
    "L3_C64_T300_Tc64": _cfg(3, 64, 300, 64, 31),
    # channels not a multiple of 16: the encoder's scalar staging
    "L2_C24_T130_Tc32": _cfg(2, 24, 130, 32, 32),
    # 17 chunks: many units through the two staging halves
    "L2_C128_T1050_Tc64": _cfg(2, 128, 1050, 64, 33),
}


class _Setup:
    def __init__(self, cfg):
        import torch
        kv, _ = kvgen.generate(cfg)
        self.kv = kv
        L, _, T, C = kv.shape
        self.T, self.Tc = T, cfg.chunk_tokens
        self.tables = _tables(cfg.bins())
        self.descs = [kvc.Desc(L, C, T, t, self.Tc) for t in self.tables]
        self.nc = kvc.lib().kvc_n_chunks(self.descs[0].ref)
        x = torch.from_numpy(kv.view(np.int16)).cuda()
        self.syms = [torch.empty(kv.size, dtype=torch.uint8, device="cuda") for _ in self.tables]
        self.cdfs = [torch.empty(d.cdf_bytes // 2, dtype=torch.int16, device="cuda") for d in self.descs]
        self.max1 = torch.empty(2 * L * T, dtype=torch.int16, device="cuda")
        self.st = torch.zeros(1, dtype=torch.int32, device="cuda")
        kvc.kvc_quantize_levels(self.descs, x, self.syms, self.max1, self.cdfs, self.st)
        torch.cuda.synchronize()
        assert int(self.st.item()) == 0
        self._want = {}

    def want(self, level, j):
        """The oracle's container of chunk j at `level`."""
        if level not in self._want:
            self._want[level] = oracle.codec(self.kv, self.tables[level], self.Tc)
        return oracle.serialize_chunk(self._want[level], j, self.tables[level], self.T, self.Tc)

    def run(self, schedule, U, two_streams, host_cap=None, on_chunk=None):
        import torch
        wb = kvc.kvc_stream_work_bytes(self.descs, U)
        work = torch.empty(wb, dtype=torch.uint8, device="cuda")
        cap = sum(len(self.want(int(schedule[j]), j)) for j in range(self.nc)) if host_cap is None else host_cap
        host = torch.zeros(max(cap, 1), dtype=torch.uint8).pin_memory()
        sizes = torch.zeros(self.nc, dtype=torch.int64).pin_memory()
        cs = torch.cuda.Stream()
        xs = torch.cuda.Stream() if two_streams else cs
        self.st.zero_()
        torch.cuda.synchronize()
        kvc.kvc_stream_encode(self.descs, schedule, self.syms, self.cdfs, self.max1, work, host, sizes,
                              self.st, cs, xs, chunks_per_unit=U, on_chunk=on_chunk, host_cap=cap)
        torch.cuda.synchronize()
        assert int(self.st.item()) == 0
        return host.numpy(), sizes.numpy().copy()


def _schedule(nc, seed, n_levels=3):
    """Runs of one level, as a sender following the link would pick them."""
    rng = np.random.default_rng(seed)
    out, lv = [], 0
    while len(out) < nc:
        out += [lv] * int(rng.integers(1, 4))
        lv = int(rng.integers(n_levels))
    return np.array(out[:nc], np.int32)


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("U,two", [(1, True), (2, True), (3, False), (0, True)])
def test_stream_containers_equal_oracle(name, U, two):
    s = _Setup(CASES[name])
    say(f"[gpu] stream {name} U={U} two_streams={two} chunks={s.nc}")
    sched = _schedule(s.nc, 7 + U)
    seen = []
    host, sizes = s.run(sched, U, two, on_chunk=lambda j, lv, b: seen.append((j, lv, bytes(b))))
    off = 0
    for j in range(s.nc):
        w = s.want(int(sched[j]), j)
        assert sizes[j] == len(w), j
        assert np.array_equal(host[off:off + len(w)], w), j
        assert seen[j] == (j, int(sched[j]), w.tobytes()), j
        off += len(w)
    assert len(seen) == s.nc


def test_stream_one_level_equals_whole_tensor_chunks():
    """Every chunk at level 0: the containers are the chunks of the one
    encoded tensor, as kvc_serialize_chunk cuts them from kvc_encode's output."""
    import torch
    s = _Setup(CASES["L3_C64_T300_Tc64"])
    sched = np.zeros(s.nc, np.int32)
    host, sizes = s.run(sched, 2, True)
    d = s.descs[0]
    buf = kvc.alloc(d)
    kvc.kvc_encode(d, s.syms[0], s.cdfs[0], buf.scratch, buf.stream_len, buf.slab_off, buf.payload,
                   buf.dev_status)
    off = 0
    for j in range(s.nc):
        out = torch.zeros(int(sizes[j]), dtype=torch.uint8, device="cuda")
        kvc.kvc_serialize_chunk(d, j, s.cdfs[0], s.max1, buf.stream_len, buf.slab_off, buf.payload, out,
                                buf.dev_status)
        torch.cuda.synchronize()
        assert np.array_equal(host[off:off + sizes[j]], out.cpu().numpy()), j
        off += int(sizes[j])
    assert int(buf.dev_status.item()) == 0


def test_stream_host_capacity_refused():
    """A host buffer that holds the first two containers only: KVC_ERR_CAPACITY,
    those two intact, nothing written past the buffer's end."""
    import torch
    s = _Setup(CASES["L2_C128_T1050_Tc64"])
    sched = np.zeros(s.nc, np.int32)
    n01 = len(s.want(0, 0)) + len(s.want(0, 1))
    wb = kvc.kvc_stream_work_bytes(s.descs, 1)
    work = torch.empty(wb, dtype=torch.uint8, device="cuda")
    host = torch.zeros(n01 + 4096, dtype=torch.uint8).pin_memory()
    sizes = torch.zeros(s.nc, dtype=torch.int64).pin_memory()
    with pytest.raises(kvc.KvcError) as ei:
        kvc.kvc_stream_encode(s.descs, sched, s.syms, s.cdfs, s.max1, work, host, sizes, s.st,
                              chunks_per_unit=1, host_cap=n01 + 100)
    assert ei.value.status == kvc.KVC_ERR_CAPACITY
    h = host.numpy()
    assert np.array_equal(h[:n01], np.concatenate([s.want(0, 0), s.want(0, 1)]))
    assert not h[n01 + 100:].any()


def test_stream_rejects_pageable_host_memory():
    import ctypes
    import torch
    s = _Setup(CASES["L2_C24_T130_Tc32"])
    wb = kvc.kvc_stream_work_bytes(s.descs, 0)
    work = torch.empty(wb, dtype=torch.uint8, device="cuda")
    host = np.zeros(1 << 20, np.uint8)  # pageable
    sizes = np.zeros(s.nc, np.int64)
    sched = np.zeros(s.nc, np.int32)
    n = len(s.descs)
    arr = (kvc.KvcDesc * n)(*[d.c for d in s.descs])
    ps = (ctypes.c_void_p * n)(*[t.data_ptr() for t in s.syms])
    pc = (ctypes.c_void_p * n)(*[t.data_ptr() for t in s.cdfs])
    rc = kvc.lib().kvc_stream_encode(arr, n, sched.ctypes.data, ps, pc, s.max1.data_ptr(), 0, work.data_ptr(),
                                     wb, host.ctypes.data, host.size, sizes.ctypes.data, None, None, None,
                                     ctypes.cast(None, kvc.CHUNK_FN), None)
    assert rc == kvc.KVC_ERR_ARG
    assert not host.any() and not sizes.any()
