"""GPU quality levels and chunk containers (kvc_quantize_levels,
kvc_serialize_chunk) against the oracle: each level equals an independent
quantization with its own bins (one-pass kernel and level-by-level path),
each chunk container is byte-identical to the oracle's, and a stream that
mixes levels chunk by chunk decodes to each chunk's level."""
import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


def _cfg(L, C, T, Tc, seed):
    return kvgen.CONFIGS["c1"].scaled(n_layers=L, n_channels=C, n_tokens=T, chunk_tokens=Tc,
                                      layer_bins=((0, L, 16),), seed=seed, rho=0.95)


def _levels(L, tables):
    """bins [L][2] per level from (first half, second half) pairs."""
    out = []
    for a, b in tables:
        t = np.full((L, 2), b, np.int32)
        t[: max(1, L // 2)] = a
        out.append(t)
    return out


CASES = {
    # 516 slabs: the one-pass kernel (3 histograms, 14 KB of LDS at C = 64)
    "onepass_L2_C64_T16421_Tc128": (_cfg(2, 64, 16421, 128, 21), [(32, 16), (16, 8), (8, 4)]),
    # few slabs: level by level
    "bylevel_L3_C40_T300_Tc128": (_cfg(3, 40, 300, 128, 22), [(32, 16), (64, 6)]),
    # >= 256 slabs, but 256-bin histograms of 512 channels exceed a block's LDS: level by level
    "bylevel_C512_A256_Tc8": (_cfg(1, 512, 1030, 8, 23), [(256, 256), (64, 64)]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_levels_equal_independent_quantizations(name):
    import torch
    cfg, tables = CASES[name]
    say(f"[gpu] levels {name}")
    kv_np, _ = kvgen.generate(cfg)
    L, _, T, C = kv_np.shape
    Tc = cfg.chunk_tokens
    binss = _levels(L, tables)
    descs = [kvc.Desc(L, C, T, b, Tc) for b in binss]
    kv = torch.from_numpy(kv_np.view(np.int16)).cuda()
    n_el = L * 2 * T * C
    syms = [torch.empty(n_el, dtype=torch.uint8, device="cuda") for _ in descs]
    cdfs = [torch.empty(d.cdf_bytes // 2, dtype=torch.int16, device="cuda") for d in descs]
    max1 = torch.empty(L * 2 * T, dtype=torch.int16, device="cuda")
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvc.kvc_quantize_levels(descs, kv, syms, max1, cdfs, st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for d, b, sy, cd in zip(descs, binss, syms, cdfs):
        osym, omax1 = oracle.quantize(kv_np, b)
        ocdf = oracle.cdf(osym, Tc, int(b.max()))
        assert np.array_equal(sy.cpu().numpy().reshape(L, 2, T, C), osym)
        assert np.array_equal(max1.cpu().numpy().view(np.uint16).reshape(L, 2, T), omax1)
        assert np.array_equal(cd.cpu().numpy().view(np.uint16), ocdf.reshape(-1))


def test_chunk_containers_and_a_mixed_level_stream():
    import torch
    cfg = _cfg(3, 64, 300, 128, 24)
    tables = [(32, 16), (8, 4)]
    kv_np, _ = kvgen.generate(cfg)
    L, _, T, C = kv_np.shape
    Tc = cfg.chunk_tokens
    NC = oracle.n_chunks(T, Tc)
    kv = torch.from_numpy(kv_np.view(np.int16)).cuda()
    levels = []
    for b in _levels(L, tables):
        d = kvc.Desc(L, C, T, b, Tc)
        buf = kvc.alloc(d)
        kvc.encode(buf, kv)
        torch.cuda.synchronize()
        assert int(buf.dev_status.item()) == 0
        levels.append((b, d, buf, oracle.codec(kv_np, b, Tc)))
    choice = [j % 2 for j in range(NC)]  # chunk j sent at level j % 2
    for j in range(NC):
        b, d, buf, r = levels[choice[j]]
        nj = oracle.chunk_tokens(T, Tc, j)
        want = oracle.serialize_chunk(r, j, b, T, Tc)
        dc = kvc.Desc(L, C, nj, b, Tc)
        assert dc.container_bytes(int(want[32:40].view(np.uint64)[0])) == want.size
        out = torch.full(((d.container_bytes(d.max_payload_bytes) + 15) // 16 * 16,), 0xA5,
                         dtype=torch.uint8, device="cuda")
        kvc.kvc_serialize_chunk(d, j, buf.cdf, buf.max1, buf.stream_len, buf.slab_off, buf.payload,
                                out, buf.dev_status)
        torch.cuda.synchronize()
        assert int(buf.dev_status.item()) == 0
        got = out[: want.size].cpu().numpy()
        assert np.array_equal(got, want), (j, np.argwhere(got != want)[:4].tolist())
        # the receiver: the chunk as a tensor of its own
        rb = kvc.alloc(dc, out_dtype=kvc.KVC_F16)
        inp = out[: want.size].clone()
        kvc.kvc_deserialize(dc, inp, rb.cdf, rb.max1, rb.stream_len, rb.slab_off, rb.dev_status)
        po = dc.container_payload_offset
        kvc.kvc_decode(dc, inp.data_ptr() + po, rb.slab_off, rb.stream_len, rb.cdf, rb.max1, None,
                       rb.out, kvc.KVC_F16, rb.dev_status, payload_bytes=want.size - po)
        torch.cuda.synchronize()
        assert int(rb.dev_status.item()) == 0
        y = rb.out[: L * 2 * nj * C].cpu().view(torch.int16).numpy().view(np.uint16).reshape(L, 2, nj, C)
        assert np.array_equal(y, r["out_f16"][:, :, j * Tc:j * Tc + nj])
