"""Checks against numbers the pages print (tests/golden/page_numbers.json)."""
import json
import math
import os

import numpy as np

import kvgen
import oracle

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_numbers.json")))


def test_kv_size_formula():
    g = GOLD["kv_size_formula_example"]
    cfg = kvgen.CONFIGS["c2"].scaled(n_tokens=g["seq_len"])
    assert cfg.n_layers == g["layers"] and cfg.n_channels == g["kv_heads"] * g["head_dim"]
    nbytes = cfg.n_layers * 2 * cfg.n_tokens * cfg.n_channels * g["dtype_bytes"]
    assert nbytes == cfg.input_bytes == 67108864
    assert round(nbytes / 1e6) == g["stated_megabytes"]


def test_validation_shape_is_the_mistral_chunk_config():
    g = GOLD["validation_kv_shape"]
    L, two, T, H, D = g["shape"]
    cfg = kvgen.CONFIGS["c2"]
    assert (cfg.n_layers, cfg.n_tokens, cfg.n_channels) == (L, T, H * D) and two == 2
    assert cfg.input_bytes == 33554432 == math.prod(g["shape"]) * 2
    assert cfg.chunk_tokens == GOLD["chunk_tokens"]["value"]


def test_preset_bins_and_alphabet_size():
    g = GOLD["preset_7b_8b"]
    for name in ("c2", "c3"):
        b = kvgen.CONFIGS[name].bins()
        assert b.shape == (g["nlayers"], 2)
        for lo, hi, nb in g["specs"]:
            assert (b[lo:hi] == nb).all()
    # a row that reaches both ends of the range uses 2*MAX + 1 = bins - 1 symbols:
    # 31 symbols ~ 5 bits for 32 bins, 15 symbols ~ 4 bits for 16 bins
    for nb, bits in g["approx_bits"].items():
        nb = int(nb)
        x = np.linspace(-1, 1, 4001, dtype=np.float32).astype(np.float16).view(np.uint16)
        kv = np.ascontiguousarray(np.broadcast_to(x[None, None, None], (1, 2, 1, x.size)))
        sym, _ = oracle.quantize(kv, np.array([[nb, nb]], np.int32))
        distinct = np.unique(sym).size
        assert distinct == nb - 1 and round(math.log2(distinct)) == bits
