"""GPU token-delta coding (kvc_delta_forward / kvc_delta_inverse) bit for bit
against the oracle: both kernel paths (a wave per anchor group with 16-byte
rows; a one-wave block per group with the anchor in LDS, and a thread per
element for the inverse), in place and not, anchor spacings from 1 to past
the chunk, ragged chunks; the whole chain forward -> codec -> inverse; the
overflow flag; and sampled chunks of the Llama-3.1-8B-shaped 8K workload."""
import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import run_gpu, say

pytestmark = pytest.mark.gpu


def _cfg(L, C, T, Tc, seed, specs=None):
    return kvgen.CONFIGS["c1"].scaled(n_layers=L, n_channels=C, n_tokens=T, chunk_tokens=Tc, seed=seed,
                                      rho=0.95, layer_bins=specs or ((0, L, 16),))


CASES = [  # (name, cfg, G)
    ("vec_C64_G4_ragged", _cfg(2, 64, 300, 128, 1, ((0, 1, 32), (1, 2, 16))), 4),
    ("vec_C1024_G3", kvgen.CONFIGS["c2"].scaled(n_tokens=40, n_layers=3), 3),
    ("vec_C512_G1", _cfg(1, 512, 33, 16, 2), 1),
    ("vec_C96_G300_past_chunk", _cfg(2, 96, 257, 256, 3), 300),
    ("any_C24_G5", _cfg(2, 24, 130, 64, 4), 5),
    ("any_C7_G2", _cfg(1, 7, 50, 16, 5), 2),
    ("any_C2048_G8", _cfg(1, 2048, 20, 16, 6), 8),
]


def _dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()


@pytest.mark.parametrize("name,cfg,G", CASES, ids=[c[0] for c in CASES])
def test_forward_inverse_bit_exact(name, cfg, G):
    import torch
    say(f"[gpu] delta {name}")
    kv, _ = kvgen.generate(cfg)
    L, _, T, C = kv.shape
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    d = kvc.Desc(L, C, T, bins, Tc)
    want = oracle.delta_forward(kv, bins, Tc, G)
    x = _dev(kv)
    out = torch.empty_like(x)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_delta_forward(d, G, x, out, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)
    # in place
    kvc.kvc_delta_forward(d, G, x, x, st)
    torch.cuda.synchronize()
    assert np.array_equal(x.cpu().numpy().view(np.uint16), want)
    # inverse of a decoded tensor (the oracle's codec output on the deltas), in place
    dec = oracle.codec(want, bins, Tc)["out_f16"]
    y = _dev(dec)
    kvc.kvc_delta_inverse(d, G, y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint16), oracle.delta_inverse(dec, Tc, G))


def test_whole_chain_through_the_codec():
    import torch
    cfg = _cfg(2, 128, 600, 256, 7, ((0, 1, 32), (1, 2, 16)))
    kv, _ = kvgen.generate(cfg)
    L, _, T, C = kv.shape
    bins, Tc, G = cfg.bins(), cfg.chunk_tokens, 4
    d = kvc.Desc(L, C, T, bins, Tc)
    x = _dev(kv)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_delta_forward(d, G, x, x, st)
    torch.cuda.synchronize()
    g = run_gpu(x.cpu().numpy().view(np.uint16), bins, Tc)
    assert g["enc_status"] == 0 and g["dec_status"] == 0
    y = _dev(g["out"])
    kvc.kvc_delta_inverse(d, G, y)
    torch.cuda.synchronize()
    want = oracle.delta_inverse(oracle.codec(oracle.delta_forward(kv, bins, Tc, G), bins, Tc)["out_f16"], Tc, G)
    assert np.array_equal(y.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("C", [8, 12])
def test_saturation_and_nonfinite(C):
    """Deltas past the fp16 range saturate (bit-exact against the oracle, status
    clear), on both kernel paths (C = 8: 16-byte rows; C = 12: a thread per
    element); the inverse saturates its sums; Inf in a delta row is flagged."""
    import torch
    from test_oracle_delta import saturation_example
    say(f"[gpu] delta saturation C={C}")
    base, bins = saturation_example()
    kv = np.zeros((1, 2, 2, C), np.uint16)
    kv[..., :4] = base
    kv[..., 4:8] = base[..., ::-1]
    d = kvc.Desc(1, C, 2, bins, 2)
    want = oracle.delta_forward(kv, bins, 2, 2)
    x = _dev(kv)
    out = torch.empty_like(x)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_delta_forward(d, 2, x, out, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(out.cpu().numpy().view(np.uint16), want)
    z = np.zeros((1, 2, 2, C), np.uint16)
    z[0, :, 0, :4] = np.array([65504.0, -65504.0, 65504.0, 1.0], np.float16).view(np.uint16)
    z[0, :, 1, :4] = np.array([32.0, -32.0, -1.0, 1.0], np.float16).view(np.uint16)
    y = _dev(z)
    kvc.kvc_delta_inverse(d, 2, y)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().view(np.uint16), oracle.delta_inverse(z, 2, 2))
    kv[0, 1, 1, C - 1] = np.float16(np.inf).view(np.uint16)
    kvc.kvc_delta_forward(d, 2, _dev(kv), out, st)
    torch.cuda.synchronize()
    assert int(st.item()) & kvc.KVC_DEV_NONFINITE


def test_llama_8k_sampled_chunks():
    import torch
    cfg = kvgen.CONFIGS["c3"]
    say("[gpu] delta: Llama-3.1-8B 8K forward, codec, inverse")
    kv, _ = kvgen.generate(cfg)
    L, _, T, C = kv.shape
    bins, Tc, G = cfg.bins(), cfg.chunk_tokens, 4
    d = kvc.Desc(L, C, T, bins, Tc)
    x = _dev(kv)
    out = torch.empty_like(x)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_delta_forward(d, G, x, out, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    got = out.view(L, 2, T, C)
    rng = np.random.default_rng(1)
    for l, j in [(0, 0), (31, 31)] + [(int(rng.integers(L)), int(rng.integers(T // Tc))) for _ in range(3)]:
        part = np.ascontiguousarray(kv[l:l + 1, :, j * Tc:(j + 1) * Tc])
        want = oracle.delta_forward(part, bins[l:l + 1], Tc, G)
        assert np.array_equal(got[l:l + 1, :, j * Tc:(j + 1) * Tc].cpu().numpy().view(np.uint16), want), (l, j)
    # the whole chain at this size: deltas in place, the codec, the inverse on the decoded
    # fp16; each chunk of a (layer, K|V) is independent, so the oracle runs chunk by chunk
    kvc.kvc_delta_forward(d, G, x, x, st)
    buf = kvc.alloc(d)
    kvc.encode(buf, x)
    kvc.decode(buf)
    kvc.kvc_delta_inverse(d, G, buf.out)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(buf.dev_status.item()) == 0
    y = buf.out[: kv.size].view(L, 2, T, C)
    for l, j in [(0, 1), (int(rng.integers(L)), int(rng.integers(T // Tc)))]:
        part = np.ascontiguousarray(kv[l:l + 1, :, j * Tc:(j + 1) * Tc])
        b = bins[l:l + 1]
        want = oracle.delta_inverse(oracle.codec(oracle.delta_forward(part, b, Tc, G), b, Tc)["out_f16"], Tc, G)
        assert np.array_equal(y[l:l + 1, :, j * Tc:(j + 1) * Tc].cpu().numpy().view(np.uint16), want), (l, j)
