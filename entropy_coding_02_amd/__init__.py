"""CacheGen-style KV-cache codec for AMD MI355X: Python binding of libkvc.so.

The functions named kvc_* mirror the C ABI in include/kvc.h one to one and
only marshal arguments (torch tensors -> device pointers, the caller's HIP
stream).  Every step of the codec runs in the HIP kernels of libkvc.so; there
is no CPU path.  `encode` / `decode` chain those calls for convenience.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvc.so")

KVC_OK, KVC_ERR_ARG, KVC_ERR_CAPACITY, KVC_ERR_HIP = 0, -1, -2, -3
KVC_DEV_NONFINITE, KVC_DEV_CORRUPT, KVC_DEV_PAYLOAD_OVERFLOW = 1, 2, 4
KVC_DEV_BAD_CDF, KVC_DEV_BAD_CONTAINER, KVC_DEV_BAD_SYMBOL = 8, 16, 32
KVC_F16, KVC_F32 = 0, 1

EXPORTED = (
    "kvc_version", "kvc_status_string", "kvc_alphabet", "kvc_n_chunks", "kvc_n_slabs",
    "kvc_n_streams", "kvc_cdf_bytes", "kvc_scratch_bytes", "kvc_max_payload_bytes",
    "kvc_quantize", "kvc_cdf", "kvc_encode", "kvc_decode", "kvc_dequantize",
    "kvc_container_bytes", "kvc_container_payload_offset", "kvc_serialize", "kvc_deserialize",
    "kvc_int8_quantize", "kvc_int8_dequantize", "kvc_serialize_chunk", "kvc_quantize_levels",
    "kvc_decode_lanes", "kvc_delta_forward", "kvc_delta_inverse", "kvc_encode_noalloc",
    "kvc_stream_work_bytes", "kvc_stream_encode",
)
KVC_NOALLOC_SCRATCH_BYTES = 64 << 20


class KvcDesc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("n_channels", ctypes.c_int32),
        ("n_tokens", ctypes.c_int64),
        ("chunk_tokens", ctypes.c_int32),
        ("cdf_chunks", ctypes.c_int32),
        ("bins", ctypes.POINTER(ctypes.c_int32)),
    ]


# void on_chunk(void *user, int64_t chunk, int32_t level, const uint8_t *container, int64_t n_bytes)
CHUNK_FN = ctypes.CFUNCTYPE(None, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                            ctypes.c_int64)


class KvcError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = _load().kvc_status_string(status).decode() if _lib else str(status)
        super().__init__(f"{fn} failed: {msg} ({status})")


_lib = None


def _load():
    """Load libkvc.so; fail loudly when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m entropy_coding_02_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        D = ctypes.POINTER(KvcDesc)
        lib.kvc_version.restype = ctypes.c_int
        lib.kvc_status_string.restype = ctypes.c_char_p
        lib.kvc_status_string.argtypes = [ctypes.c_int]
        lib.kvc_alphabet.restype = I32
        lib.kvc_decode_lanes.restype = I32
        lib.kvc_decode_lanes.argtypes = [D]
        lib.kvc_delta_forward.restype = ctypes.c_int
        lib.kvc_delta_forward.argtypes = [D, I32, P, P, P, P]
        lib.kvc_delta_inverse.restype = ctypes.c_int
        lib.kvc_delta_inverse.argtypes = [D, I32, P, P]
        for n in ("kvc_n_chunks", "kvc_n_slabs", "kvc_n_streams", "kvc_cdf_bytes",
                  "kvc_scratch_bytes", "kvc_max_payload_bytes"):
            getattr(lib, n).restype = I64
        for n in ("kvc_alphabet", "kvc_n_chunks", "kvc_n_slabs", "kvc_n_streams", "kvc_cdf_bytes",
                  "kvc_scratch_bytes", "kvc_max_payload_bytes"):
            getattr(lib, n).argtypes = [D]
        lib.kvc_quantize.restype = ctypes.c_int
        lib.kvc_quantize.argtypes = [D, P, P, P, P, P, P]
        lib.kvc_cdf.restype = ctypes.c_int
        lib.kvc_cdf.argtypes = [D, P, P, P, P]
        lib.kvc_encode.restype = ctypes.c_int
        lib.kvc_encode.argtypes = [D, P, P, P, I64, P, P, P, I64, P, P]
        lib.kvc_encode_noalloc.restype = ctypes.c_int
        lib.kvc_encode_noalloc.argtypes = [D, P, P, P, P, P, I64, P, P]
        lib.kvc_decode.restype = ctypes.c_int
        lib.kvc_decode.argtypes = [D, P, I64, P, P, P, P, P, P, I32, P, P]
        lib.kvc_dequantize.restype = ctypes.c_int
        lib.kvc_dequantize.argtypes = [D, P, P, P, I32, P]
        lib.kvc_container_bytes.restype = I64
        lib.kvc_container_bytes.argtypes = [D, I64]
        lib.kvc_container_payload_offset.restype = I64
        lib.kvc_container_payload_offset.argtypes = [D]
        lib.kvc_serialize.restype = ctypes.c_int
        lib.kvc_serialize.argtypes = [D, P, P, P, P, P, P, I64, P, P]
        lib.kvc_deserialize.restype = ctypes.c_int
        lib.kvc_deserialize.argtypes = [D, P, I64, P, P, P, P, P, P]
        lib.kvc_quantize_levels.restype = ctypes.c_int
        lib.kvc_quantize_levels.argtypes = [D, I32, P, P, P, P, P, P]
        lib.kvc_serialize_chunk.restype = ctypes.c_int
        lib.kvc_serialize_chunk.argtypes = [D, I64, P, P, P, P, P, P, I64, P, P]
        lib.kvc_int8_quantize.restype = ctypes.c_int
        lib.kvc_int8_quantize.argtypes = [D, I32, P, P, P, P, P, P]
        lib.kvc_int8_dequantize.restype = ctypes.c_int
        lib.kvc_int8_dequantize.argtypes = [D, I32, P, P, P, P, I32, P]
        lib.kvc_stream_work_bytes.restype = I64
        lib.kvc_stream_work_bytes.argtypes = [D, I32, I32]
        lib.kvc_stream_encode.restype = ctypes.c_int
        lib.kvc_stream_encode.argtypes = [D, I32, P, P, P, P, I32, P, I64, P, I64, P, P, P, P,
                                          CHUNK_FN, P]
        _lib = lib
    return _lib


def lib():
    return _load()


class Desc:
    """A kvc_desc plus the host bins array it points to."""

    def __init__(self, n_layers: int, n_channels: int, n_tokens: int, bins,
                 chunk_tokens: int = 256, cdf_chunks: int = 0):
        """cdf_chunks: chunks sharing one CDF table (0 or 1: a table per chunk)."""
        self.bins = np.ascontiguousarray(np.asarray(bins, dtype=np.int32).reshape(n_layers, 2))
        self.c = KvcDesc(n_layers, n_channels, n_tokens, chunk_tokens, cdf_chunks,
                         self.bins.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        self.n_layers, self.n_channels, self.n_tokens = n_layers, n_channels, n_tokens
        self.chunk_tokens, self.cdf_chunks = chunk_tokens, cdf_chunks

    @property
    def ref(self):
        return ctypes.byref(self.c)

    def _q(self, name):
        v = getattr(_load(), name)(self.ref)
        if v < 0:
            raise KvcError(name, int(v))
        return int(v)

    @property
    def alphabet(self): return self._q("kvc_alphabet")
    @property
    def n_chunks(self): return self._q("kvc_n_chunks")
    @property
    def n_slabs(self): return self._q("kvc_n_slabs")
    @property
    def n_streams(self): return self._q("kvc_n_streams")
    @property
    def decode_lanes(self): return self._q("kvc_decode_lanes")
    @property
    def cdf_bytes(self): return self._q("kvc_cdf_bytes")
    @property
    def scratch_bytes(self): return self._q("kvc_scratch_bytes")
    @property
    def max_payload_bytes(self): return self._q("kvc_max_payload_bytes")
    @property
    def container_payload_offset(self): return self._q("kvc_container_payload_offset")

    def container_bytes(self, payload_bytes: int) -> int:
        v = _load().kvc_container_bytes(self.ref, payload_bytes)
        if v < 0:
            raise KvcError("kvc_container_bytes", int(v))
        return int(v)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("kvc: device tensors only (there is no CPU path)")
    if not t.is_contiguous():
        raise ValueError("kvc: tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, rc: int):
    if rc != KVC_OK:
        raise KvcError(fn, rc)


# --------------------------------------------------------------- C ABI, 1:1

def kvc_version() -> int:
    return int(_load().kvc_version())


def kvc_quantize(desc: Desc, kv, sym, max1, cdf=None, dev_status=None, stream=None):
    _check("kvc_quantize", _load().kvc_quantize(desc.ref, _ptr(kv), _ptr(sym), _ptr(max1), _ptr(cdf),
                                                _ptr(dev_status), _stream(stream)))


def kvc_quantize_levels(descs, kv, syms, max1, cdfs, dev_status=None, stream=None):
    """descs: Desc per level; syms, cdfs: device tensors per level."""
    n = len(descs)
    arr = (KvcDesc * n)(*[d.c for d in descs])  # the Desc objects keep their bins alive
    ps = (ctypes.c_void_p * n)(*[_ptr(t) for t in syms])
    pc = (ctypes.c_void_p * n)(*[_ptr(t) for t in cdfs])
    _check("kvc_quantize_levels", _load().kvc_quantize_levels(arr, n, _ptr(kv), ps, _ptr(max1), pc,
                                                              _ptr(dev_status), _stream(stream)))


def kvc_cdf(desc: Desc, sym, cdf, dev_status=None, stream=None):
    _check("kvc_cdf", _load().kvc_cdf(desc.ref, _ptr(sym), _ptr(cdf), _ptr(dev_status), _stream(stream)))


def kvc_encode(desc: Desc, sym, cdf, scratch, stream_len, slab_off, payload, dev_status=None,
               stream=None, scratch_bytes=None, payload_cap=None):
    sb = scratch.numel() * scratch.element_size() if scratch_bytes is None else scratch_bytes
    pc = payload.numel() * payload.element_size() if payload_cap is None else payload_cap
    _check("kvc_encode", _load().kvc_encode(desc.ref, _ptr(sym), _ptr(cdf), _ptr(scratch), sb,
                                            _ptr(stream_len), _ptr(slab_off), _ptr(payload), pc,
                                            _ptr(dev_status), _stream(stream)))


def kvc_encode_noalloc(desc: Desc, sym, cdf, stream_len, slab_off, payload, dev_status=None, stream=None,
                       payload_cap=None):
    pc = payload.numel() * payload.element_size() if payload_cap is None else payload_cap
    _check("kvc_encode_noalloc", _load().kvc_encode_noalloc(desc.ref, _ptr(sym), _ptr(cdf), _ptr(stream_len),
                                                            _ptr(slab_off), _ptr(payload), pc,
                                                            _ptr(dev_status), _stream(stream)))


def kvc_decode(desc: Desc, payload, slab_off, stream_len, cdf, max1=None, sym_out=None, out=None,
               out_dtype=KVC_F16, dev_status=None, stream=None, payload_bytes=None):
    pb = payload.numel() * payload.element_size() if payload_bytes is None else payload_bytes
    _check("kvc_decode", _load().kvc_decode(desc.ref, _ptr(payload), pb, _ptr(slab_off),
                                            _ptr(stream_len), _ptr(cdf), _ptr(max1), _ptr(sym_out),
                                            _ptr(out), out_dtype, _ptr(dev_status), _stream(stream)))


def kvc_dequantize(desc: Desc, sym, max1, out, out_dtype=KVC_F16, stream=None):
    _check("kvc_dequantize", _load().kvc_dequantize(desc.ref, _ptr(sym), _ptr(max1), _ptr(out),
                                                    out_dtype, _stream(stream)))


def kvc_serialize(desc: Desc, cdf, max1, stream_len, slab_off, payload, out, dev_status=None,
                  stream=None, out_cap=None):
    oc = out.numel() * out.element_size() if out_cap is None else out_cap
    _check("kvc_serialize", _load().kvc_serialize(desc.ref, _ptr(cdf), _ptr(max1), _ptr(stream_len),
                                                  _ptr(slab_off), _ptr(payload), _ptr(out), oc,
                                                  _ptr(dev_status), _stream(stream)))


def kvc_serialize_chunk(desc: Desc, chunk: int, cdf, max1, stream_len, slab_off, payload, out,
                        dev_status=None, stream=None, out_cap=None):
    oc = out.numel() * out.element_size() if out_cap is None else out_cap
    _check("kvc_serialize_chunk", _load().kvc_serialize_chunk(desc.ref, chunk, _ptr(cdf), _ptr(max1),
                                                              _ptr(stream_len), _ptr(slab_off),
                                                              _ptr(payload), _ptr(out), oc,
                                                              _ptr(dev_status), _stream(stream)))


def kvc_stream_work_bytes(descs, chunks_per_unit: int = 0) -> int:
    n = len(descs)
    arr = (KvcDesc * n)(*[d.c for d in descs])
    v = int(_load().kvc_stream_work_bytes(arr, n, chunks_per_unit))
    if v < 0:
        raise KvcError("kvc_stream_work_bytes", v)
    return v


def _host_ptr(t) -> int:
    if t.is_cuda or not t.is_pinned() or not t.is_contiguous():
        raise ValueError("kvc: page-locked contiguous host tensors only (torch pin_memory)")
    return t.data_ptr()


def kvc_stream_encode(descs, chunk_level, syms, cdfs, max1, work, host_out, chunk_bytes, dev_status=None,
                      compute_stream=None, copy_stream=None, chunks_per_unit: int = 0, on_chunk=None,
                      work_bytes=None, host_cap=None):
    """descs: Desc per level; chunk_level: host int32 [NC]; syms, cdfs: device
    tensors per level; work: device buffer; host_out (uint8) and chunk_bytes
    (int64 [NC]): pinned host tensors; on_chunk(chunk, level, memoryview) or
    None.  Returns once every container is in host_out."""
    import torch
    n = len(descs)
    arr = (KvcDesc * n)(*[d.c for d in descs])
    ps = (ctypes.c_void_p * n)(*[_ptr(t) for t in syms])
    pc = (ctypes.c_void_p * n)(*[_ptr(t) for t in cdfs])
    lv = np.ascontiguousarray(np.asarray(chunk_level, dtype=np.int32))
    wb = work.numel() * work.element_size() if work_bytes is None else work_bytes
    hc = host_out.numel() * host_out.element_size() if host_cap is None else host_cap
    if chunk_bytes.dtype != torch.int64:
        raise ValueError("kvc: chunk_bytes must be int64")
    if on_chunk is None:
        cb = ctypes.cast(None, CHUNK_FN)
    else:
        def _cb(_user, chunk, level, ptr, nbytes):
            on_chunk(int(chunk), int(level), (ctypes.c_uint8 * nbytes).from_address(ptr))
        cb = CHUNK_FN(_cb)
    cs = _stream(compute_stream)
    xs = cs if copy_stream is None else _stream(copy_stream)
    _check("kvc_stream_encode", _load().kvc_stream_encode(
        arr, n, lv.ctypes.data, ps, pc, _ptr(max1), chunks_per_unit, _ptr(work), wb, _host_ptr(host_out), hc,
        _host_ptr(chunk_bytes), _ptr(dev_status), cs, xs, cb, None))


def kvc_deserialize(desc: Desc, inp, cdf, max1, stream_len, slab_off, dev_status=None, stream=None,
                    in_bytes=None):
    nb = inp.numel() * inp.element_size() if in_bytes is None else in_bytes
    _check("kvc_deserialize", _load().kvc_deserialize(desc.ref, _ptr(inp), nb, _ptr(cdf), _ptr(max1),
                                                      _ptr(stream_len), _ptr(slab_off),
                                                      _ptr(dev_status), _stream(stream)))


def kvc_int8_quantize(desc: Desc, group: int, kv, q, scale, zero_point, dev_status=None,
                      stream=None):
    _check("kvc_int8_quantize", _load().kvc_int8_quantize(desc.ref, group, _ptr(kv), _ptr(q),
                                                          _ptr(scale), _ptr(zero_point),
                                                          _ptr(dev_status), _stream(stream)))


def kvc_int8_dequantize(desc: Desc, group: int, q, scale, zero_point, out, out_dtype=KVC_F16, stream=None):
    _check("kvc_int8_dequantize", _load().kvc_int8_dequantize(desc.ref, group, _ptr(q), _ptr(scale),
                                                              _ptr(zero_point), _ptr(out), out_dtype,
                                                              _stream(stream)))


def kvc_delta_forward(desc: Desc, anchor_tokens: int, kv, delta, dev_status=None, stream=None):
    _check("kvc_delta_forward", _load().kvc_delta_forward(desc.ref, anchor_tokens, _ptr(kv), _ptr(delta),
                                                          _ptr(dev_status), _stream(stream)))


def kvc_delta_inverse(desc: Desc, anchor_tokens: int, y, stream=None):
    _check("kvc_delta_inverse", _load().kvc_delta_inverse(desc.ref, anchor_tokens, _ptr(y), _stream(stream)))


# --------------------------------------------------------------- convenience

@dataclass
class Buffers:
    """Preallocated device buffers for one problem shape."""
    desc: Desc
    sym: "object"
    max1: "object"
    cdf: "object"
    scratch: "object"
    stream_len: "object"
    slab_off: "object"
    payload: "object"
    dev_status: "object"
    out: "object"
    dec_sym: "object"


def alloc(desc: Desc, device="cuda", out_dtype=KVC_F16, with_dec_sym=False) -> Buffers:
    import torch
    L, C, T = desc.n_layers, desc.n_channels, desc.n_tokens
    u8, u16, i64 = torch.uint8, torch.int16, torch.int64

    def z(n, dt):
        return torch.empty(max(n, 1), dtype=dt, device=device)

    odt = torch.float16 if out_dtype == KVC_F16 else torch.float32
    n_el = L * 2 * T * C
    return Buffers(
        desc=desc,
        sym=z(n_el, u8), max1=z(L * 2 * T, u16),
        cdf=z(desc.cdf_bytes // 2, u16),
        scratch=z((desc.scratch_bytes + 15) // 16 * 16, u8),
        stream_len=z(desc.n_streams, u16),
        slab_off=z(desc.n_slabs + 1, i64),
        payload=z((desc.max_payload_bytes + 15) // 16 * 16, u8),
        dev_status=torch.zeros(1, dtype=torch.int32, device=device),
        out=z(n_el, odt),
        dec_sym=z(n_el, u8) if with_dec_sym else None,
    )


def encode(buf: Buffers, kv, fused_cdf: bool = True, stream=None):
    """quantize (+ CDF) then range-code and pack, all on `stream`."""
    d = buf.desc
    kvc_quantize(d, kv, buf.sym, buf.max1, buf.cdf if fused_cdf else None, buf.dev_status, stream)
    if not fused_cdf:
        kvc_cdf(d, buf.sym, buf.cdf, buf.dev_status, stream)
    kvc_encode(d, buf.sym, buf.cdf, buf.scratch, buf.stream_len, buf.slab_off, buf.payload,
               buf.dev_status, stream)


def decode(buf: Buffers, out_dtype=KVC_F16, stream=None, payload=None, payload_bytes=None):
    """decode + fused dequantize into buf.out (and buf.dec_sym if allocated)."""
    d = buf.desc
    kvc_decode(d, buf.payload if payload is None else payload, buf.slab_off, buf.stream_len, buf.cdf,
               buf.max1, buf.dec_sym, buf.out, out_dtype, buf.dev_status, stream,
               payload_bytes=payload_bytes)
