"""GPU 8-bit comparator quantizer (kvc_int8_quantize / kvc_int8_dequantize)
bit for bit against the oracle: both kernel paths (a wave per row with
shuffle-reduced groups; a thread per group), edge values, and the non-finite
flag."""
import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


def _cfg(L, C, T, seed, innov="normal"):
    return kvgen.CONFIGS["c1"].scaled(n_layers=L, n_channels=C, n_tokens=T, seed=seed, innov=innov,
                                      layer_bins=((0, L, 16),), outlier_frac=0.05, outlier_mul=30.0)


CASES = [  # (name, cfg, group)
    ("C1024_g128_rows", kvgen.CONFIGS["c2"].scaled(n_tokens=48), 128),
    ("C64_g8_rows", _cfg(2, 64, 33, 1), 8),
    ("C96_g32_rows", _cfg(3, 96, 17, 2, "t3"), 32),
    ("C512_g512_rows", _cfg(1, 512, 9, 3), 512),
    ("C1024_g1024_groups", _cfg(1, 1024, 5, 4), 1024),
    ("C24_g12_groups", _cfg(2, 24, 40, 5), 12),
    ("C7_g7_groups", _cfg(1, 7, 50, 6, "t3"), 7),
]


def _run(kv_np, g):
    import torch
    L, _, T, C = kv_np.shape
    d = kvc.Desc(L, C, T, np.full((L, 2), 16, np.int32))
    kv = torch.from_numpy(kv_np.view(np.int16)).cuda()
    n_el, n_g = L * 2 * T * C, L * 2 * T * (C // g)
    q = torch.empty(max(n_el, 1), dtype=torch.uint8, device="cuda")
    sc = torch.empty(max(n_g, 1), dtype=torch.float32, device="cuda")
    zp = torch.empty(max(n_g, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty(max(n_el, 1), dtype=torch.int16, device="cuda")
    out32 = torch.empty(max(n_el, 1), dtype=torch.float32, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_int8_quantize(d, g, kv, q, sc, zp, st)
    kvc.kvc_int8_dequantize(d, g, q, sc, zp, out)
    kvc.kvc_int8_dequantize(d, g, q, sc, zp, out32, kvc.KVC_F32)
    torch.cuda.synchronize()
    return (q[:n_el].cpu().numpy().reshape(L, 2, T, C), sc[:n_g].cpu().numpy().reshape(L, 2, T, C // g),
            zp[:n_g].cpu().numpy().reshape(L, 2, T, C // g),
            out[:n_el].cpu().numpy().view(np.uint16).reshape(L, 2, T, C), int(st.item()),
            out32[:n_el].cpu().numpy().reshape(L, 2, T, C))


@pytest.mark.parametrize("name,cfg,g", CASES, ids=[c[0] for c in CASES])
def test_int8_bit_exact(name, cfg, g):
    say(f"[gpu] int8 {name}")
    kv_np, _ = kvgen.generate(cfg)
    q, sc, zp, out, st, out32 = _run(kv_np, g)
    oq, osc, ozp = oracle.int8_quantize(kv_np, g)
    assert st == 0
    assert np.array_equal(q, oq)
    assert np.array_equal(sc.view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(zp, ozp)
    assert np.array_equal(out, oracle.int8_dequantize(oq, osc, ozp, g))
    assert np.array_equal(out32.view(np.uint32), oracle.int8_dequantize(oq, osc, ozp, g, fp32=True).view(np.uint32))


@pytest.mark.parametrize("g", [16, 12])
def test_int8_edge_values(g):
    rng = np.random.default_rng(11)
    C = 48
    vals = np.array([0.0, -0.0, 65504.0, -65504.0, 6e-8, -6e-8, 1e-5, 2.5, -2.5, 1.0], np.float16)
    kv = rng.choice(vals, size=(2, 2, 30, C)).astype(np.float16)
    kv[0, 0, 0] = 2.5            # constant rows: every group constant
    kv[0, 1, 3] = 0.0            # zero row
    kv[1, 0, 5, :g] = -0.0       # one negative-zero group
    kv[1, 1, 7, :g] = [65504.0, -65504.0] * (g // 2)
    kv_np = kv.view(np.uint16)
    q, sc, zp, out, st, out32 = _run(kv_np, g)
    oq, osc, ozp = oracle.int8_quantize(kv_np, g)
    assert st == 0
    assert np.array_equal(q, oq) and np.array_equal(zp, ozp)
    assert np.array_equal(sc.view(np.uint32), osc.view(np.uint32))
    assert np.array_equal(out, oracle.int8_dequantize(oq, osc, ozp, g))
    want32 = oracle.int8_dequantize(oq, osc, ozp, g, fp32=True)
    assert np.array_equal(out32.view(np.uint32), want32.view(np.uint32))
    assert np.isfinite(out32).all()  # the +-65504 group: finite in fp32


def test_int8_nonfinite_flagged():
    kv = np.zeros((1, 2, 4, 64), np.uint16)
    kv[0, 1, 2, 17] = 0x7E00  # NaN
    for g in (16, 64):
        *_, st, _ = _run(kv, g)
        assert st & kvc.KVC_DEV_NONFINITE
