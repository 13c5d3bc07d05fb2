"""Seeded synthetic fp16 KV-cache inputs shared by the oracle, the HIP path,
the tests and the bench.

This module draws numbers and nothing else: it holds none of the codec's
arithmetic.  Shapes follow the pages' models: the (32, 2, 256, 8, 128) fp16
kv_shape of the CacheGen/LMCache write-up ("3.2 Validation and testing"),
Llama-3.1-8B with the 7B/8B layer-wise bins ("2.2 CacheGenConfig",
"2.3 Encoder pipeline"), the 34B model at 80K tokens ("1.2 Core challenges"),
and a 70B-class GQA model.  Real KV caches of those models are not available;
these seeded AR(1) series stand in for them.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import List, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVC_SANITIZE=1: a copy built with AddressSanitizer and UndefinedBehaviorSanitizer (clang).
SANITIZE = os.environ.get("KVC_SANITIZE") == "1"
_LIB_PATH = os.path.join(_HERE, "libkvgen_san.so" if SANITIZE else "libkvgen.so")


@dataclass(frozen=True)
class KVConfig:
    name: str
    workload: str
    n_layers: int
    n_channels: int
    n_tokens: int
    chunk_tokens: int
    layer_bins: Tuple[Tuple[int, int, int], ...]  # (start_layer, end_layer, bins), half-open, K = V
    rho: float
    innov: str  # "normal" | "t3"
    scale_lo: float
    scale_hi: float
    outlier_frac: float = 0.0
    outlier_mul: float = 1.0
    seed: int = 0

    def bins(self) -> np.ndarray:
        """int32 [L][2] bins table (K, V) from the half-open layer ranges."""
        b = np.zeros((self.n_layers, 2), dtype=np.int32)
        for lo, hi, nb in self.layer_bins:
            b[lo:hi, :] = nb
        if (b == 0).any():
            raise ValueError(f"{self.name}: layer ranges do not cover all layers")
        return b

    @property
    def n_elements(self) -> int:
        return self.n_layers * 2 * self.n_tokens * self.n_channels

    @property
    def input_bytes(self) -> int:
        return 2 * self.n_elements

    def scaled(self, **kw) -> "KVConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return KVConfig(**d)


CONFIGS = {
    "c1": KVConfig(
        name="c1", workload="tiny_L2_C16_T64",
        n_layers=2, n_channels=16, n_tokens=64, chunk_tokens=256,
        layer_bins=((0, 1, 32), (1, 2, 16)),
        rho=0.9, innov="normal", scale_lo=0.1, scale_hi=4.0),
    "c2": KVConfig(
        name="c2", workload="mistral7b_chunk_L32_C1024_T256",
        n_layers=32, n_channels=1024, n_tokens=256, chunk_tokens=256,
        layer_bins=((0, 10, 32), (10, 32, 16)),
        rho=0.95, innov="normal", scale_lo=0.05, scale_hi=8.0),
    "c3": KVConfig(
        name="c3", workload="llama31_8b_8k_L32_C1024_T8192",
        n_layers=32, n_channels=1024, n_tokens=8192, chunk_tokens=256,
        layer_bins=((0, 10, 32), (10, 32, 16)),
        rho=0.95, innov="normal", scale_lo=0.05, scale_hi=8.0),
    "c4": KVConfig(
        name="c4", workload="34b_80k_L48_C1024_T80000",
        n_layers=48, n_channels=1024, n_tokens=80000, chunk_tokens=256,
        layer_bins=((0, 16, 32), (16, 48, 16)),
        rho=0.97, innov="normal", scale_lo=0.05, scale_hi=8.0,
        outlier_frac=0.02, outlier_mul=20.0),
    "c5": KVConfig(
        name="c5", workload="70b_gqa_32k_L80_C1024_T32768",
        n_layers=80, n_channels=1024, n_tokens=32768, chunk_tokens=256,
        layer_bins=((0, 10, 64), (10, 40, 32), (40, 80, 16)),
        rho=0.9, innov="t3", scale_lo=0.05, scale_hi=8.0,
        outlier_frac=0.05, outlier_mul=50.0),
}


class _Params(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int32), ("C", ctypes.c_int32), ("T", ctypes.c_int64),
        ("rho", ctypes.c_double), ("innov", ctypes.c_int32),
        ("scale_lo", ctypes.c_double), ("scale_hi", ctypes.c_double),
        ("outlier_frac", ctypes.c_double), ("outlier_mul", ctypes.c_double),
        ("seed", ctypes.c_uint64),
    ]


_lib = None


def build(force: bool = False) -> str:
    """Compile libkvgen.so with gcc (plain C, pthreads)."""
    import subprocess
    src = os.path.join(_HERE, "kvgen.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cc = ["gcc"]
        if SANITIZE:
            cc = ["/opt/rocm/llvm/bin/clang", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                  "-fno-omit-frame-pointer", "-g", "-shared-libsan"]
        subprocess.check_call([*cc, "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-ffp-contract=off", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.kvgen_generate.restype = ctypes.c_int64
        lib.kvgen_generate.argtypes = [ctypes.POINTER(_Params), ctypes.c_void_p, ctypes.c_int]
        lib.kvgen_fnv1a64.restype = ctypes.c_uint64
        lib.kvgen_fnv1a64.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        _lib = lib
    return _lib


def default_threads() -> int:
    n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        n = min(n, int(env))
    return max(1, min(n, 16))


def generate(cfg: KVConfig, out: np.ndarray | None = None, threads: int | None = None):
    """Return (kv, n_saturated): kv is uint16 [L][2][T][C] holding fp16 bits."""
    shape = (cfg.n_layers, 2, cfg.n_tokens, cfg.n_channels)
    if out is None:
        out = np.empty(shape, dtype=np.uint16)
    if out.shape != shape or out.dtype != np.uint16 or not out.flags.c_contiguous:
        raise ValueError("out must be C-contiguous uint16 of shape %r" % (shape,))
    p = _Params(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.rho,
                1 if cfg.innov == "t3" else 0, cfg.scale_lo, cfg.scale_hi,
                cfg.outlier_frac, cfg.outlier_mul, cfg.seed)
    sat = _load().kvgen_generate(ctypes.byref(p), out.ctypes.data, threads or default_threads())
    if sat < 0:
        raise ValueError("kvgen_generate rejected the parameters")
    return out, int(sat)


def checksum(buf: np.ndarray) -> int:
    """FNV-1a 64 of the buffer's bytes."""
    b = np.ascontiguousarray(buf)
    return int(_load().kvgen_fnv1a64(b.ctypes.data, b.nbytes))

