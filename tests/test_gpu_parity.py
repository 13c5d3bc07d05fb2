"""GPU parity: the HIP path through the C ABI against the oracle.

Bit-exact for everything integer (symbols, max1, CDFs, stream lengths, slab
offsets, payload bytes, decoded symbols) and for fp16 output; fp32 output is
compared bit for bit too, which is stricter than the 1e-6 relative bound the
codec promises (asserted as well).  Small and ragged shapes, and all five
workload sizes, are compared in full; the three large workloads chunk by
chunk, with the oracle fanned out over the host's cores.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "the GPU tests need a GPU"
    assert os.path.exists(kvc.LIB_PATH), "libkvc.so is not built"
    kvc.lib()
    say(f"device: {torch.cuda.get_device_name(0)}")


def cfg_of(L, C, T, Tc, specs, seed=0, rho=0.9, innov="normal", lo=0.1, hi=4.0, of=0.0, om=1.0):
    return kvgen.KVConfig(name="t", workload="t", n_layers=L, n_channels=C, n_tokens=T,
                          chunk_tokens=Tc, layer_bins=specs, rho=rho, innov=innov, scale_lo=lo,
                          scale_hi=hi, outlier_frac=of, outlier_mul=om, seed=seed)


SMALL = {
    "c1": kvgen.CONFIGS["c1"],
    "ragged_L3_C40_T300_Tc128": cfg_of(3, 40, 300, 128, ((0, 1, 32), (1, 3, 16)), seed=3),
    "C24_T100": cfg_of(2, 24, 100, 256, ((0, 2, 32),), seed=4),
    "C7_T70_Tc32": cfg_of(1, 7, 70, 32, ((0, 1, 16),), seed=5),
    "A256_and_A4": cfg_of(2, 64, 64, 256, ((0, 1, 256), (1, 2, 4)), seed=6, innov="t3", of=0.1, om=30),
    "Tc300_T700": cfg_of(1, 32, 700, 300, ((0, 1, 64),), seed=7),
    "A4_T257": cfg_of(1, 128, 257, 256, ((0, 1, 4),), seed=8),
    "mistral_L32_C1024_T64": kvgen.CONFIGS["c2"].scaled(n_tokens=64),
    "bins6_odd_MAX": cfg_of(2, 48, 90, 256, ((0, 2, 6),), seed=9),
    # alphabets whose 1024 / A is not a power of two (encoder tile widths)
    "A24_C96": cfg_of(1, 96, 80, 256, ((0, 1, 24),), seed=10),
    "A40_and_A24_C64": cfg_of(2, 64, 120, 256, ((0, 1, 40), (1, 2, 24)), seed=11),
    # 256 slabs or more: the fused quantize + CDF pass (ragged last chunk)
    "fused_L2_C64_T16421_Tc128": cfg_of(2, 64, 16421, 128, ((0, 1, 32), (1, 2, 16)), seed=12),
    # fused pass at A = 64: a 128 KB LDS histogram
    "fused_70b_shape_T300": kvgen.CONFIGS["c5"].scaled(n_tokens=300),
    # a quad of lanes per stream in the encoder (k_encode_split: at most 16384
    # streams, C a multiple of 4 CDF tiles): padded rows, 64-entry rows, a
    # ragged chunk
    "split_A24_C512_T200_Tc128": cfg_of(2, 512, 200, 128, ((0, 1, 24), (1, 2, 16)), seed=15),
    "split_A64_C256_T300": cfg_of(2, 256, 300, 256, ((0, 1, 64), (1, 2, 32)), seed=16),
    # more than 16384 streams: one lane per stream (the launches above with
    # few streams decode with a group of lanes per stream), rows of 8 and 16
    "one_lane_A8_C16_T9000": cfg_of(1, 16, 9000, 256, ((0, 1, 8),), seed=13),
    "one_lane_A16_C24_T9000": cfg_of(1, 24, 9000, 512, ((0, 1, 16),), seed=14),
    # the mode-first decoder's tiles: 64-entry rows (16-channel tiles), padded
    # 64-entry rows, 32-entry rows with a last tile of 8 channels (no 16-byte
    # path), and near-constant channels that take its fast path
    "one_lane_A64_C80_T9000": cfg_of(1, 80, 9000, 256, ((0, 1, 64),), seed=17, innov="t3", of=0.05, om=50),
    "one_lane_A40_C96_T9000": cfg_of(1, 96, 9000, 256, ((0, 1, 40),), seed=18),
    "one_lane_A32_C200_T9000": cfg_of(1, 200, 9000, 256, ((0, 1, 32),), seed=19, lo=0.05, hi=8.0, of=0.02, om=20),
    # layers with fewer bins than the table's rows: the mode-first decoder
    # takes a run of them with at least 4096 slabs in a launch of its own that
    # searches only the first 16 entries of each row (16-token chunks give
    # 2048 slabs per layer and K|V); shorter runs search whole rows
    "one_lane_A32_A16_C16_T32768_Tc16": cfg_of(2, 16, 32768, 16, ((0, 1, 32), (1, 2, 16)), seed=20),
    "one_lane_A32_A16_C64_T9000": cfg_of(2, 64, 9000, 256, ((0, 1, 32), (1, 2, 16)), seed=23),
    "one_lane_A64_A32_A16_C48_T6000": cfg_of(3, 48, 6000, 256, ((0, 1, 64), (1, 2, 32), (2, 3, 16)), seed=21,
                                             innov="t3", of=0.05, om=50),
}


def compare_full(name, kv, bins, Tc, fused=True, out_dtype=kvc.KVC_F16, exact_payload=False):
    say(f"[gpu] {name}: shape={kv.shape} Tc={Tc} fused={fused} out={out_dtype} exact={exact_payload}")
    g = run_gpu(kv, bins, Tc, fused=fused, out_dtype=out_dtype, exact_payload=exact_payload)
    r = oracle.codec(kv, bins, Tc)
    assert g["enc_status"] == 0 and g["dec_status"] == 0
    for key in ("sym", "max1", "cdf", "stream_len", "slab_off", "payload", "dec_sym"):
        a, b = g[key], r[key]
        assert a.shape == b.shape, (key, a.shape, b.shape)
        bad = np.argwhere(a != b)
        assert bad.size == 0, (key, bad[:3].tolist())
    if out_dtype == kvc.KVC_F16:
        assert np.array_equal(g["out"], r["out_f16"])
    else:
        ref = oracle.dequantize(r["dec_sym"], r["max1"], bins, fp32=True)
        assert np.array_equal(g["out"].view(np.uint32), ref.view(np.uint32))
        rel = np.abs(g["out"] - ref) / np.maximum(np.abs(ref), np.finfo(np.float32).tiny)
        assert rel.max(initial=0.0) <= 1e-6
    return g, r


@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes_bit_exact(name):
    cfg = SMALL[name]
    kv, _ = kvgen.generate(cfg)
    compare_full(name, kv, cfg.bins(), cfg.chunk_tokens)


@pytest.mark.parametrize("name", ["c1", "ragged_L3_C40_T300_Tc128", "C7_T70_Tc32", "Tc300_T700"])
def test_separate_cdf_fp32_out_exact_payload(name):
    cfg = SMALL[name]
    kv, _ = kvgen.generate(cfg)
    compare_full(name, kv, cfg.bins(), cfg.chunk_tokens, fused=False, out_dtype=kvc.KVC_F32,
                 exact_payload=True)


def test_edge_values():
    """Zero rows, +-65504, subnormals, -0.0, a row whose max is a subnormal."""
    rng = np.random.default_rng(12)
    L, T, C = 2, 40, 32
    x = (rng.standard_normal((L, 2, T, C)) * 3).astype(np.float32)
    x[0, 0, 0] = 0.0
    x[0, 1, 1] = -0.0
    x[1, 0, 2, :4] = [65504, -65504, 1e-7, -6e-8]
    x[1, 1, 3] = rng.standard_normal(C) * 1e-6  # all subnormal in fp16
    x[0, 0, 5, :] = 2.0**-24
    kv = x.astype(np.float16).view(np.uint16)
    bins = np.array([[32, 16], [256, 4]], np.int32)
    for odt in (kvc.KVC_F16, kvc.KVC_F32):
        compare_full("edge_values", kv, bins, 16, out_dtype=odt)


def test_one_lane_runs_of_kv_bins():
    """K and V of a layer with different bins (32 | 16, then 16 | 32): the
    mode-first decoder's launches split where the search depth changes (the
    16-entry run of 4096 slabs between two whole-row ones)."""
    cfg = cfg_of(2, 16, 32768, 16, ((0, 2, 32),), seed=22)
    kv, _ = kvgen.generate(cfg)
    compare_full("one_lane_kv_bins", kv, np.array([[32, 16], [16, 32]], np.int32), cfg.chunk_tokens)


def test_one_lane_runs_without_status():
    """kvc_decode with no status word cannot tell a guard launch about a
    stream that left the staged rows, so it searches whole rows in one
    launch: the same symbols and values as the oracle, as with a status word
    (runs per search depth and the guard)."""
    import torch
    cfg = SMALL["one_lane_A32_A16_C16_T32768_Tc16"]
    say("[gpu] one-lane runs, decode without a status word")
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, _, T, C = kv.shape
    d = kvc.Desc(L, C, T, bins, Tc)
    buf = kvc.alloc(d, out_dtype=kvc.KVC_F16, with_dec_sym=True)
    kvc.encode(buf, torch.from_numpy(kv.view(np.int16)).cuda())
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) == 0
    r = oracle.codec(kv, bins, Tc)
    n = kv.size
    for status in (None, buf.dev_status):
        buf.dec_sym.fill_(0xAB)
        buf.out.fill_(0)
        kvc.kvc_decode(d, buf.payload, buf.slab_off, buf.stream_len, buf.cdf, buf.max1, buf.dec_sym, buf.out,
                       kvc.KVC_F16, status)
        torch.cuda.synchronize()
        assert int(buf.dev_status.item()) == 0
        assert np.array_equal(buf.dec_sym[:n].cpu().numpy().reshape(kv.shape), r["sym"])
        got16 = buf.out[:n].cpu().view(torch.int16).numpy().view(np.uint16).reshape(kv.shape)
        assert np.array_equal(got16, r["out_f16"])


def test_empty_input():
    say("[gpu] empty input")
    import torch
    d = kvc.Desc(2, 16, 0, [[32, 16], [32, 16]])
    buf = kvc.alloc(d)
    buf.slab_off.fill_(123)
    kv = torch.empty(1, dtype=torch.int16, device="cuda")
    kvc.encode(buf, kv)
    kvc.decode(buf)
    torch.cuda.synchronize()
    assert int(buf.slab_off[0].item()) == 0 and int(buf.dev_status.item()) == 0


def test_nonfinite_flagged():
    say("[gpu] non-finite input")
    import torch
    cfg = SMALL["c1"]
    kv, _ = kvgen.generate(cfg)
    kv = kv.copy()
    kv[0, 1, 7, 3] = np.float16(np.inf).view(np.uint16)
    kv[1, 0, 9, 0] = np.uint16(0x7E00)  # NaN
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.bins())
    buf = kvc.alloc(d)
    kvc.kvc_quantize(d, torch.from_numpy(kv.view(np.int16)).cuda(), buf.sym, buf.max1, buf.cdf, buf.dev_status)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) & kvc.KVC_DEV_NONFINITE


@pytest.mark.parametrize("name", ["ragged_L3_C40_T300_Tc128", "one_lane_A32_C200_T9000",
                                  "one_lane_A32_A16_C16_T32768_Tc16"])
def test_corrupt_payload_flagged_and_bounded(name):
    """Group decoder, then the one-lane mode-first decoder (a wave-wide flag
    mask), then the latter on layers whose launches search only the first 16
    entries of each row: a code past them flags the stream, and the guard
    launch decodes every stream again over whole rows."""
    say(f"[gpu] corrupt payload {name}")
    import torch
    cfg = SMALL[name]
    kv, _ = kvgen.generate(cfg)
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.bins(), cfg.chunk_tokens)
    buf = kvc.alloc(d, with_dec_sym=True)
    kvc.encode(buf, torch.from_numpy(kv.view(np.int16)).cuda())
    torch.cuda.synchronize()
    total = int(buf.slab_off[d.n_slabs].item())
    bad = torch.full(((total + 3) // 4 * 4,), 0xFF, dtype=torch.uint8, device="cuda")
    buf.dev_status.zero_()
    kvc.decode(buf, payload=bad)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) & kvc.KVC_DEV_CORRUPT
    # the oracle agrees on the symbols it decodes from the same bytes
    r = oracle.codec(kv, cfg.bins(), cfg.chunk_tokens)
    want, flagged = oracle.decode(np.full(total, 0xFF, np.uint8), r["slab_off"], r["stream_len"], r["cdf"],
                                  cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.chunk_tokens, r["A"])
    assert flagged
    got = buf.dec_sym[: kv.size].cpu().numpy().reshape(kv.shape)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("name", ["ragged_L3_C40_T300_Tc128", "split_A24_C512_T200_Tc128"])
def test_payload_overflow_flagged_and_cap_respected(name):
    """One-lane and split encoders (the latter takes its slab offsets from the pack)."""
    say(f"[gpu] payload capacity {name}")
    import torch
    cfg = SMALL[name]
    kv, _ = kvgen.generate(cfg)
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.bins(), cfg.chunk_tokens)
    buf = kvc.alloc(d)
    kvt = torch.from_numpy(kv.view(np.int16)).cuda()
    kvc.encode(buf, kvt)
    torch.cuda.synchronize()
    total = int(buf.slab_off[d.n_slabs].item())
    cap = total // 2
    guard = torch.full((cap + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    buf.dev_status.zero_()
    kvc.kvc_encode(d, buf.sym, buf.cdf, buf.scratch, buf.stream_len, buf.slab_off, guard,
                   buf.dev_status, payload_cap=cap)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) & kvc.KVC_DEV_PAYLOAD_OVERFLOW
    g = guard.cpu().numpy()
    assert (g[cap:] == 0x5A).all()
    assert np.array_equal(g[:cap], buf.payload[:cap].cpu().numpy())


@pytest.mark.parametrize("name", ["C24_T100", "ragged_L3_C40_T300_Tc128", "split_A24_C512_T200_Tc128",
                                  "mistral_L32_C1024_T64", "one_lane_A8_C16_T9000", "one_lane_A64_C80_T9000",
                                  "one_lane_A40_C96_T9000"])
def test_bad_symbol_flagged(name):
    """A symbol >= A (no CDF interval) sets KVC_DEV_BAD_SYMBOL in kvc_cdf and in
    kvc_encode (one-lane, split and scalar-staging encoders; the one-lane
    encoder's staged symbols both as pair offsets, A a power of two, and
    clamped, A = 40; narrow and wide CDF kernels); the same symbols at A - 1
    (valid for the row, whatever the layer's bins) set nothing, and kvc_cdf's
    rows then equal the oracle's."""
    import torch
    cfg = SMALL[name]
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, bins, Tc)
    A = d.alphabet
    sym, _ = oracle.quantize(kv, bins)
    L, _, T, C = sym.shape
    for bad_value, want_flag in ((A - 1, 0), (A, kvc.KVC_DEV_BAD_SYMBOL), (255, kvc.KVC_DEV_BAD_SYMBOL)):
        say(f"[gpu] bad symbol {name}: value {bad_value} (A={A})")
        s2 = sym.copy()
        s2[L - 1, 1, T - 1, C - 1] = bad_value  # the last symbol of the last stream
        s2[0, 0, T // 2, C // 2] = bad_value
        buf = kvc.alloc(d)
        st = torch.from_numpy(s2).cuda()
        kvc.kvc_cdf(d, st, buf.cdf, buf.dev_status)
        torch.cuda.synchronize()
        assert int(buf.dev_status.item()) == want_flag
        if not want_flag:
            got = buf.cdf[: d.cdf_bytes // 2].cpu().numpy().view(np.uint16)
            assert np.array_equal(got, oracle.cdf(s2, Tc, A).ravel())
        good_cdf = torch.from_numpy(oracle.cdf(sym, Tc, A).ravel().view(np.int16)).cuda()
        buf.dev_status.zero_()
        kvc.kvc_encode(d, st, good_cdf, buf.scratch, buf.stream_len, buf.slab_off, buf.payload,
                       buf.dev_status)
        torch.cuda.synchronize()
        assert int(buf.dev_status.item()) & kvc.KVC_DEV_BAD_SYMBOL == want_flag


def test_one_lane_encoder_runs_redo():
    """Layers with fewer bins than the table's rows are encoded with only the
    first 2^n entries of each row staged.  A symbol of such a layer past them
    but below A (legal in its table, though no quantizer of its bins makes
    it) sends the call to its guard launch over whole rows: payload bit for
    bit as the oracle's, and no status bit left; a symbol >= A ends with
    exactly KVC_DEV_BAD_SYMBOL."""
    import torch
    cfg = SMALL["one_lane_A32_A16_C16_T32768_Tc16"]
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, bins, Tc)
    A = d.alphabet
    sym, _ = oracle.quantize(kv, bins)
    L, _, T, C = sym.shape
    for value, want in ((20, 0), (A + 8, kvc.KVC_DEV_BAD_SYMBOL)):
        say(f"[gpu] encoder runs: layer {L - 1} symbol {value} (A={A})")
        s2 = sym.copy()
        s2[L - 1, 0, T // 3, 5] = value   # layer of 16 bins: staged rows of 16 entries
        s2[L - 1, 1, T - 1, C - 1] = value
        tab = oracle.cdf(np.minimum(s2, A - 1), Tc, A)
        buf = kvc.alloc(d)
        buf.dev_status.zero_()
        kvc.kvc_encode(d, torch.from_numpy(s2).cuda(), torch.from_numpy(tab.ravel().view(np.int16)).cuda(),
                       buf.scratch, buf.stream_len, buf.slab_off, buf.payload, buf.dev_status)
        torch.cuda.synchronize()
        assert int(buf.dev_status.item()) == want
        if not want:
            wl, wo, wp = oracle.encode(s2, tab, Tc, A)
            assert np.array_equal(buf.stream_len[: d.n_streams].cpu().numpy().view(np.uint16), wl)
            assert np.array_equal(buf.slab_off[: d.n_slabs + 1].cpu().numpy().view(np.uint64), wo)
            n = int(wo[-1])
            assert np.array_equal(buf.payload[:n].cpu().numpy(), wp[:n])


def test_deterministic():
    cfg = SMALL["mistral_L32_C1024_T64"]
    kv, _ = kvgen.generate(cfg)
    say("[gpu] determinism")
    a = run_gpu(kv, cfg.bins(), 256)
    b = run_gpu(kv, cfg.bins(), 256)
    for k in ("cdf", "payload", "out"):
        assert np.array_equal(a[k], b[k])


def test_standalone_dequantize_matches_oracle():
    import torch
    cfg = SMALL["A256_and_A4"]
    kv, _ = kvgen.generate(cfg)
    sym, max1 = oracle.quantize(kv, cfg.bins())
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.bins())
    for odt, fp32 in ((kvc.KVC_F16, False), (kvc.KVC_F32, True)):
        say(f"[gpu] dequantize out={odt}")
        out = torch.empty(kv.size, dtype=torch.float32 if fp32 else torch.float16, device="cuda")
        kvc.kvc_dequantize(d, torch.from_numpy(sym).cuda(), torch.from_numpy(max1.view(np.int16)).cuda(),
                           out, odt)
        torch.cuda.synchronize()
        want = oracle.dequantize(sym, max1, cfg.bins(), fp32=fp32)
        got = out.cpu().numpy() if fp32 else out.cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got.reshape(want.shape).view(np.uint32 if fp32 else np.uint16),
                              want.view(np.uint32 if fp32 else np.uint16))


# ------------------------------------------------------------ workload sizes

def test_workload_tiny_and_mistral_chunk_full():
    for name in ("c1", "c2"):
        cfg = kvgen.CONFIGS[name]
        kv, _ = kvgen.generate(cfg)
        compare_full(name, kv, cfg.bins(), cfg.chunk_tokens)


def _host_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))  # a GPU machine's CPU share is 16 cores


@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_workload_full_size_bit_exact(name):
    """Every output of the three large workloads against the oracle, in the
    launch configuration bench.py times: symbols, max1, CDF rows, stream
    lengths, slab offsets, payload bytes, decoded symbols and fp16 output,
    chunk by chunk over the whole tensor.  Chunks are independent (their own
    CDFs, streams and slab offsets from the chunk's first byte), so the oracle
    runs on each chunk alone, fanned out over the host's cores, while the GPU
    outputs come back one chunk at a time.  The reconstruction bound is
    checked on the GPU over the whole tensor as well."""
    from concurrent.futures import ThreadPoolExecutor

    import torch
    cfg = kvgen.CONFIGS[name]
    say(f"[gpu] {name}: generating {cfg.input_bytes / 1e9:.1f} GB input")
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, T, C = cfg.n_layers, cfg.n_tokens, cfg.n_channels
    d = kvc.Desc(L, C, T, bins, Tc)
    A, NC, twoL = d.alphabet, d.n_chunks, 2 * L
    buf = kvc.alloc(d, with_dec_sym=True)
    kvt = torch.from_numpy(kv.view(np.int16)).cuda()
    say(f"[gpu] {name}: encode + decode (the launches bench.py times)")
    kvc.encode(buf, kvt, fused_cdf=True)
    kvc.decode(buf, out_dtype=kvc.KVC_F16)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) == 0
    n_el = kv.size
    lens = buf.stream_len[: d.n_streams].cpu().numpy().view(np.uint16)
    offs = buf.slab_off[: d.n_slabs + 1].cpu().numpy().view(np.uint64).astype(np.int64)
    assert offs[0] == 0 and (np.diff(offs) >= 0).all() and offs[-1] == lens.astype(np.int64).sum()
    # reconstruction bound |y - x| <= m/(2 MAX) + 8 m 2^-24 + half an fp16 ulp of y, everywhere
    MAX = torch.from_numpy((bins // 2 - 1).astype(np.float32)).cuda()
    y_all = buf.out[:n_el].view(L, 2, T, C)
    m_all = buf.max1[: L * 2 * T].view(torch.float16).view(L, 2, T)
    for l in range(L):
        x = kvt.view(torch.float16).view(L, 2, T, C)[l].float()
        y = y_all[l].float()
        m = m_all[l].float()[..., None]
        ulp = torch.abs(y_all[l]).float() * 2.0**-11 + 2.0**-25
        bound = m / (2 * MAX[l][:, None, None]) + 8 * m * 2.0**-24 + ulp
        assert bool((torch.abs(y - x) <= bound).all()), l
    del kvt
    sym_v = buf.sym[:n_el].view(L, 2, T, C)
    dec_v = buf.dec_sym[:n_el].view(L, 2, T, C)
    max_v = buf.max1[: L * 2 * T].view(L, 2, T)
    cdf_v = buf.cdf[: d.cdf_bytes // 2].view(NC, L, 2, C, A)

    def check(j, g):
        t0, nj = j * Tc, min(Tc, T - j * Tc)
        r = oracle.codec(np.ascontiguousarray(kv[:, :, t0:t0 + nj]), bins, Tc)
        s0 = j * twoL * Tc
        base = offs[j * twoL]
        want = {"sym": r["sym"], "dec_sym": r["sym"], "max1": r["max1"], "cdf": r["cdf"][0],
                "stream_len": r["stream_len"], "slab_off": r["slab_off"].astype(np.int64),
                "payload": r["payload"], "out": r["out_f16"]}
        got = dict(g, stream_len=lens[s0:s0 + twoL * nj],
                   slab_off=offs[j * twoL:(j + 1) * twoL + 1] - base)
        for k, w in want.items():
            a = got[k]
            assert a.shape == w.shape and np.array_equal(a, w), (name, j, k)
        assert not r["corrupt"]
        return j

    threads = _host_threads()
    say(f"[gpu] {name}: {NC} chunks against the oracle on {threads} host threads "
        f"({os.cpu_count()} CPUs visible)")
    done = 0
    with ThreadPoolExecutor(max_workers=threads) as ex:
        pending = []
        for j in range(NC):
            t0, nj = j * Tc, min(Tc, T - j * Tc)
            g = {"sym": sym_v[:, :, t0:t0 + nj].cpu().numpy(),
                 "dec_sym": dec_v[:, :, t0:t0 + nj].cpu().numpy(),
                 "max1": max_v[:, :, t0:t0 + nj].cpu().numpy().view(np.uint16),
                 "cdf": cdf_v[j].cpu().numpy().view(np.uint16),
                 "payload": buf.payload[int(offs[j * twoL]):int(offs[(j + 1) * twoL])].cpu().numpy(),
                 "out": y_all[:, :, t0:t0 + nj].cpu().view(torch.int16).numpy().view(np.uint16)}
            pending.append(ex.submit(check, j, g))
            while len(pending) >= 2 * threads:  # bounds the chunks held on the host
                pending.pop(0).result()
                done += 1
                if done % 64 == 0:
                    say(f"[gpu] {name}: {done}/{NC} chunks bit-exact")
        for f in pending:
            f.result()
    say(f"[gpu] {name}: all {NC} chunks bit-exact")
    del buf
    torch.cuda.empty_cache()
