"""ctypes wrapper of the plain C oracle (kvc_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by
bench.py's CPU-baseline leg, never by the product library.  See kvc_oracle.c
for the page passages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvc_oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "kvc_container.c"), os.path.join(_HERE, "kvc_int8.c"),
         os.path.join(_HERE, "kvc_delta.c")]
# KVC_SANITIZE=1 builds and loads a copy compiled with AddressSanitizer and
# UndefinedBehaviorSanitizer (clang, whose runtime the process must preload).
SANITIZE = os.environ.get("KVC_SANITIZE") == "1"
SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
             "-g", "-shared-libsan"]
_LIB_PATH = os.path.join(_HERE, "liborc_san.so" if SANITIZE else "liborc.so")

ORC_OK, ORC_ERR_ARG, ORC_ERR_NONFINITE, ORC_ERR_CAPACITY, ORC_ERR_CORRUPT = 0, -1, -2, -3, -4

_lib = None


def build(force: bool = False) -> str:
    """Compile liborc.so: gcc, -O2, no FP contraction, no fast-math."""
    hdr = os.path.join(_HERE, "kvc_oracle.h")
    newest = max([os.path.getmtime(f) for f in _SRCS] + [os.path.getmtime(hdr)])
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cc = ["/opt/rocm/llvm/bin/clang", *SAN_FLAGS] if SANITIZE else ["gcc"]
        subprocess.check_call([*cc, "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, *_SRCS, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        lib.orc_half_to_float.restype = ctypes.c_float
        lib.orc_half_to_float.argtypes = [ctypes.c_uint16]
        lib.orc_float_to_half.restype = ctypes.c_uint16
        lib.orc_float_to_half.argtypes = [ctypes.c_float]
        lib.orc_quantize.restype = ctypes.c_int
        lib.orc_quantize.argtypes = [I32, I32, I64, P, P, P, P]
        lib.orc_cdf.restype = ctypes.c_int
        lib.orc_cdf.argtypes = [I32, I32, I64, I32, I32, I32, P, P]
        lib.orc_encode_stream.restype = I64
        lib.orc_encode_stream.argtypes = [P, I32, I32, P, P, I64]
        lib.orc_decode_stream.restype = ctypes.c_int
        lib.orc_decode_stream.argtypes = [P, I64, I32, I32, P, P]
        lib.orc_encode.restype = I64
        lib.orc_encode.argtypes = [I32, I32, I64, I32, I32, I32, P, P, P, P, P, I64]
        lib.orc_decode.restype = ctypes.c_int
        lib.orc_decode.argtypes = [I32, I32, I64, I32, I32, I32, P, P, P, P, P]
        lib.orc_dequantize.restype = ctypes.c_int
        lib.orc_dequantize.argtypes = [I32, I32, I64, P, P, P, P, I32]
        lib.orc_delta_forward.restype = ctypes.c_int
        lib.orc_delta_forward.argtypes = [I32, I32, I64, I32, I32, P, P, P]
        lib.orc_delta_inverse.restype = ctypes.c_int
        lib.orc_delta_inverse.argtypes = [I32, I32, I64, I32, I32, P]
        lib.orc_container_bytes.restype = I64
        lib.orc_container_bytes.argtypes = [I32, I32, I64, I32, I32, P, I64]
        lib.orc_container_payload_offset.restype = I64
        lib.orc_container_payload_offset.argtypes = [I32, I32, I64, I32, I32, P]
        lib.orc_serialize.restype = I64
        lib.orc_serialize.argtypes = [I32, I32, I64, I32, I32, P, P, P, P, P, I64, P, I64]
        lib.orc_deserialize.restype = ctypes.c_int
        lib.orc_deserialize.argtypes = [I32, I32, I64, I32, I32, P, P, I64, P, P, P, P, P]
        lib.orc_int8_quantize.restype = ctypes.c_int
        lib.orc_int8_quantize.argtypes = [I32, I32, I64, I32, P, P, P, P]
        lib.orc_int8_dequantize.restype = ctypes.c_int
        lib.orc_int8_dequantize.argtypes = [I32, I32, I64, I32, P, P, P, P, I32]
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    if not a.flags.c_contiguous:
        raise ValueError("array must be C-contiguous")
    return a.ctypes.data


class OracleError(RuntimeError):
    def __init__(self, fn, code):
        super().__init__(f"{fn} returned {code}")
        self.code = code


# ----------------------------------------------------------------- scalars

def half_to_float(h: int) -> float:
    return float(_load().orc_half_to_float(int(h) & 0xFFFF))


def float_to_half(f: float) -> int:
    return int(_load().orc_float_to_half(float(np.float32(f))))


# ----------------------------------------------------------------- sizes

def n_chunks(T: int, Tc: int) -> int:
    return (T + Tc - 1) // Tc


def chunk_tokens(T: int, Tc: int, j: int) -> int:
    return min(Tc, T - j * Tc)


def tables_of(T: int, Tc: int, tab_chunks: int = 1) -> tuple[int, int]:
    """(chunks per CDF table as stored, number of tables per (layer, K|V)):
    tab_chunks taken as at most NC (1 when there are no chunks)."""
    NC = n_chunks(T, Tc)
    S = min(tab_chunks, NC) if NC else 1
    return S, -(-NC // S)


# ----------------------------------------------------------------- steps

def quantize(kv: np.ndarray, bins: np.ndarray):
    """kv: uint16 fp16 bits [L][2][T][C]; bins int32 [L][2] -> (sym u8, max1 u16 [L][2][T])."""
    L, two, T, C = kv.shape
    assert two == 2
    bins = np.ascontiguousarray(bins, dtype=np.int32)
    kv = np.ascontiguousarray(kv, dtype=np.uint16)
    sym = np.empty(kv.shape, dtype=np.uint8)
    max1 = np.empty((L, 2, T), dtype=np.uint16)
    rc = _load().orc_quantize(L, C, T, _ptr(bins), _ptr(kv), _ptr(sym), _ptr(max1))
    if rc != ORC_OK:
        raise OracleError("orc_quantize", rc)
    return sym, max1


def cdf(sym: np.ndarray, Tc: int, A: int, tab_chunks: int = 1) -> np.ndarray:
    """sym u8 [L][2][T][C] -> cdf u16 [NG][L][2][C][A], one table per
    tab_chunks chunks (1: per chunk)."""
    L, _, T, C = sym.shape
    sym = np.ascontiguousarray(sym, dtype=np.uint8)
    out = np.empty((tables_of(T, Tc, tab_chunks)[1], L, 2, C, A), dtype=np.uint16)
    rc = _load().orc_cdf(L, C, T, Tc, tab_chunks, A, _ptr(sym), _ptr(out))
    if rc != ORC_OK:
        raise OracleError("orc_cdf", rc)
    return out


def encode_stream(q: np.ndarray, cdf_rows: np.ndarray) -> bytes:
    """q u8 [C]; cdf_rows u16 [C][A] -> stream bytes."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    cdf_rows = np.ascontiguousarray(cdf_rows, dtype=np.uint16)
    C, A = cdf_rows.shape
    assert q.shape == (C,)
    cap = 2 * C + 8
    buf = np.empty(cap, dtype=np.uint8)
    n = _load().orc_encode_stream(_ptr(q), C, A, _ptr(cdf_rows), _ptr(buf), cap)
    if n < 0:
        raise OracleError("orc_encode_stream", n)
    return buf[:n].tobytes()


def decode_stream(data: bytes, cdf_rows: np.ndarray):
    """-> (symbols u8 [C], corrupt flag)."""
    cdf_rows = np.ascontiguousarray(cdf_rows, dtype=np.uint16)
    C, A = cdf_rows.shape
    src = np.frombuffer(bytes(data) + b"\0", dtype=np.uint8)  # +1: never a zero-size buffer
    q = np.empty(C, dtype=np.uint8)
    bad = _load().orc_decode_stream(_ptr(src), len(data), C, A, _ptr(cdf_rows), _ptr(q))
    return q, bool(bad)


def encode(sym: np.ndarray, cdf_tab: np.ndarray, Tc: int, A: int, payload_cap: int | None = None,
           tab_chunks: int = 1):
    """-> (stream_len u16 [n_streams], slab_off u64 [n_slabs+1], payload u8)."""
    L, _, T, C = sym.shape
    NC = n_chunks(T, Tc)
    n_streams = 2 * L * T
    n_slabs = NC * L * 2
    if payload_cap is None:
        payload_cap = n_streams * (2 * C + 1)
    stream_len = np.zeros(n_streams, dtype=np.uint16)
    slab_off = np.zeros(n_slabs + 1, dtype=np.uint64)
    payload = np.zeros(max(payload_cap, 1), dtype=np.uint8)
    n = _load().orc_encode(L, C, T, Tc, tab_chunks, A, _ptr(np.ascontiguousarray(sym)),
                           _ptr(np.ascontiguousarray(cdf_tab)), _ptr(stream_len), _ptr(slab_off),
                           _ptr(payload), payload_cap)
    if n < 0:
        raise OracleError("orc_encode", n)
    return stream_len, slab_off, payload[:n].copy()


def decode(payload: np.ndarray, slab_off: np.ndarray, stream_len: np.ndarray, cdf_tab: np.ndarray,
           L: int, C: int, T: int, Tc: int, A: int, tab_chunks: int = 1):
    """-> (sym u8 [L][2][T][C], corrupt flag)."""
    sym = np.empty((L, 2, T, C), dtype=np.uint8)
    pay = np.concatenate([np.ascontiguousarray(payload, dtype=np.uint8), np.zeros(1, np.uint8)])
    rc = _load().orc_decode(L, C, T, Tc, tab_chunks, A, _ptr(pay), _ptr(np.ascontiguousarray(slab_off)),
                            _ptr(np.ascontiguousarray(stream_len)),
                            _ptr(np.ascontiguousarray(cdf_tab)), _ptr(sym))
    if rc not in (ORC_OK, ORC_ERR_CORRUPT):
        raise OracleError("orc_decode", rc)
    return sym, rc == ORC_ERR_CORRUPT


def dequantize(sym: np.ndarray, max1: np.ndarray, bins: np.ndarray, fp32: bool = True) -> np.ndarray:
    """-> float32 [L][2][T][C] or uint16 fp16 bits."""
    L, _, T, C = sym.shape
    out = np.empty(sym.shape, dtype=np.float32 if fp32 else np.uint16)
    rc = _load().orc_dequantize(L, C, T, _ptr(np.ascontiguousarray(bins, dtype=np.int32)),
                                _ptr(np.ascontiguousarray(sym)), _ptr(np.ascontiguousarray(max1)),
                                _ptr(out), 1 if fp32 else 0)
    if rc != ORC_OK:
        raise OracleError("orc_dequantize", rc)
    return out


def _bins32(bins) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(bins, dtype=np.int32).reshape(-1))


def container_bytes(L: int, C: int, T: int, Tc: int, bins, payload_bytes: int, tab_chunks: int = 1) -> int:
    n = _load().orc_container_bytes(L, C, T, Tc, tab_chunks, _ptr(_bins32(bins)), payload_bytes)
    if n < 0:
        raise OracleError("orc_container_bytes", n)
    return int(n)


def container_payload_offset(L: int, C: int, T: int, Tc: int, bins, tab_chunks: int = 1) -> int:
    n = _load().orc_container_payload_offset(L, C, T, Tc, tab_chunks, _ptr(_bins32(bins)))
    if n < 0:
        raise OracleError("orc_container_payload_offset", n)
    return int(n)


def serialize(cdf_tab: np.ndarray, max1: np.ndarray, stream_len: np.ndarray, payload: np.ndarray,
              bins, Tc: int, tab_chunks: int = 1) -> np.ndarray:
    """-> the container bytes (u8)."""
    L, _, T = max1.shape
    C = cdf_tab.shape[3]
    pb = int(payload.size)
    n = container_bytes(L, C, T, Tc, bins, pb, tab_chunks)
    out = np.empty(n, dtype=np.uint8)
    pay = np.ascontiguousarray(payload, dtype=np.uint8) if pb else np.zeros(1, np.uint8)
    rc = _load().orc_serialize(L, C, T, Tc, tab_chunks, _ptr(_bins32(bins)), _ptr(np.ascontiguousarray(cdf_tab)),
                               _ptr(np.ascontiguousarray(max1)), _ptr(np.ascontiguousarray(stream_len)),
                               _ptr(pay), pb, _ptr(out), n)
    if rc < 0:
        raise OracleError("orc_serialize", rc)
    return out


def deserialize(data: np.ndarray, L: int, C: int, T: int, Tc: int, bins, tab_chunks: int = 1):
    """-> dict(cdf, max1, stream_len, slab_off, payload_bytes, payload_offset)."""
    A = int(np.max(bins))
    NC = n_chunks(T, Tc)
    cdf_tab = np.empty((tables_of(T, Tc, tab_chunks)[1], L, 2, C, A), dtype=np.uint16)
    max1 = np.empty((L, 2, T), dtype=np.uint16)
    stream_len = np.empty(2 * L * T, dtype=np.uint16)
    slab_off = np.empty(NC * L * 2 + 1, dtype=np.uint64)
    pb = ctypes.c_int64(0)
    data = np.ascontiguousarray(data, dtype=np.uint8)
    rc = _load().orc_deserialize(L, C, T, Tc, tab_chunks, _ptr(_bins32(bins)), _ptr(data), data.size,
                                 _ptr(cdf_tab), _ptr(max1), _ptr(stream_len), _ptr(slab_off),
                                 ctypes.addressof(pb))
    if rc != ORC_OK:
        raise OracleError("orc_deserialize", rc)
    return dict(cdf=cdf_tab, max1=max1, stream_len=stream_len, slab_off=slab_off,
                payload_bytes=int(pb.value),
                payload_offset=container_payload_offset(L, C, T, Tc, bins, tab_chunks))


def delta_forward(kv: np.ndarray, bins: np.ndarray, Tc: int, G: int) -> np.ndarray:
    """Token-delta transform (anchors every G chunk-relative tokens): fp16 bits [L][2][T][C]."""
    L, _, T, C = kv.shape
    out = np.empty(kv.shape, dtype=np.uint16)
    rc = _load().orc_delta_forward(L, C, T, Tc, G, _ptr(np.ascontiguousarray(bins, dtype=np.int32)),
                                   _ptr(np.ascontiguousarray(kv, dtype=np.uint16)), _ptr(out))
    if rc != ORC_OK:
        raise OracleError("orc_delta_forward", rc)
    return out


def delta_inverse(y: np.ndarray, Tc: int, G: int) -> np.ndarray:
    """Inverse of delta_forward on a decoded fp16 tensor (a new array)."""
    L, _, T, C = y.shape
    out = np.array(y, dtype=np.uint16, copy=True, order="C")
    rc = _load().orc_delta_inverse(L, C, T, Tc, G, _ptr(out))
    if rc != ORC_OK:
        raise OracleError("orc_delta_inverse", rc)
    return out


def int8_quantize(kv: np.ndarray, g: int):
    """-> (q u8 [L][2][T][C], scale f32 [L][2][T][C/g], zero_point u8 [L][2][T][C/g])."""
    L, _, T, C = kv.shape
    q = np.empty(kv.shape, dtype=np.uint8)
    scale = np.empty((L, 2, T, C // g), dtype=np.float32)
    zp = np.empty((L, 2, T, C // g), dtype=np.uint8)
    rc = _load().orc_int8_quantize(L, C, T, g, _ptr(np.ascontiguousarray(kv, dtype=np.uint16)),
                                   _ptr(q), _ptr(scale), _ptr(zp))
    if rc != ORC_OK:
        raise OracleError("orc_int8_quantize", rc)
    return q, scale, zp


def int8_dequantize(q: np.ndarray, scale: np.ndarray, zp: np.ndarray, g: int, fp32: bool = False) -> np.ndarray:
    """-> fp16 bits (u16) [L][2][T][C], or float32 when fp32."""
    L, _, T, C = q.shape
    out = np.empty(q.shape, dtype=np.float32 if fp32 else np.uint16)
    rc = _load().orc_int8_dequantize(L, C, T, g, _ptr(np.ascontiguousarray(q)),
                                     _ptr(np.ascontiguousarray(scale, dtype=np.float32)),
                                     _ptr(np.ascontiguousarray(zp)), _ptr(out), 1 if fp32 else 0)
    if rc != ORC_OK:
        raise OracleError("orc_int8_dequantize", rc)
    return out


def chunk_of(r: dict, j: int, T: int, Tc: int, tab_chunks: int = 1):
    """Chunk j of an encoded tensor as a tensor of its own (T = N_j tokens):
    the CDF tables it was coded with (its own, or its group's when tables are
    shared), its max1 rows, its stream lengths and its payload bytes, cut out
    of codec()'s outputs ([CG] 2.3 step 3: chunks stream on their own)."""
    L = r["max1"].shape[0]
    nj = chunk_tokens(T, Tc, j)
    g = j // tables_of(T, Tc, tab_chunks)[0]
    s0, s1 = j * 2 * L, (j + 1) * 2 * L
    lo, hi = int(r["slab_off"][s0]), int(r["slab_off"][s1])
    return dict(cdf=np.ascontiguousarray(r["cdf"][g:g + 1]),
                max1=np.ascontiguousarray(r["max1"][:, :, j * Tc:j * Tc + nj]),
                stream_len=np.ascontiguousarray(r["stream_len"][j * 2 * L * Tc:j * 2 * L * Tc + 2 * L * nj]),
                payload=np.ascontiguousarray(r["payload"][lo:hi]), n_tokens=nj)


def serialize_chunk(r: dict, j: int, bins, T: int, Tc: int, tab_chunks: int = 1) -> np.ndarray:
    """The container of chunk j alone (a tensor of N_j tokens, one table)."""
    c = chunk_of(r, j, T, Tc, tab_chunks)
    return serialize(c["cdf"], c["max1"], c["stream_len"], c["payload"], bins, Tc)


def codec(kv: np.ndarray, bins: np.ndarray, Tc: int, tab_chunks: int = 1):
    """The whole hot path on the CPU: dict of every intermediate and output."""
    A = int(np.max(bins))
    sym, max1 = quantize(kv, bins)
    cdf_tab = cdf(sym, Tc, A, tab_chunks)
    stream_len, slab_off, payload = encode(sym, cdf_tab, Tc, A, tab_chunks=tab_chunks)
    L, _, T, C = kv.shape
    dsym, bad = decode(payload, slab_off, stream_len, cdf_tab, L, C, T, Tc, A, tab_chunks)
    out16 = dequantize(dsym, max1, bins, fp32=False)
    return dict(A=A, sym=sym, max1=max1, cdf=cdf_tab, stream_len=stream_len, slab_off=slab_off,
                payload=payload, dec_sym=dsym, corrupt=bad, out_f16=out16)
