"""GPU byte container (kvc_serialize / kvc_deserialize) against the oracle:
byte-identical containers, round trips, decoding straight from the
container's payload section, and the device flags of its error paths."""
import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


def _cfg_of(L, C, T, Tc, layer_bins, seed):
    return kvgen.CONFIGS["c1"].scaled(n_layers=L, n_channels=C, n_tokens=T, chunk_tokens=Tc,
                                      layer_bins=layer_bins, seed=seed)


CASES = {
    "c1": kvgen.CONFIGS["c1"],
    "ragged_L3_C40_T300_Tc128": _cfg_of(3, 40, 300, 128, ((0, 1, 32), (1, 3, 16)), 3),
    "A256_A6_C24_T70": _cfg_of(2, 24, 70, 256, ((0, 1, 256), (1, 2, 6)), 6),
    "mistral_L32_C1024_T64": kvgen.CONFIGS["c2"].scaled(n_tokens=64),
    "fused_L2_C64_T16421_Tc128": _cfg_of(2, 64, 16421, 128, ((0, 1, 32), (1, 2, 16)), 12),
}


def _encode(cfg):
    import torch
    kv_np, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, _, T, C = kv_np.shape
    d = kvc.Desc(L, C, T, bins, Tc)
    buf = kvc.alloc(d, out_dtype=kvc.KVC_F16)
    kv = torch.from_numpy(kv_np.view(np.int16)).cuda()
    kvc.encode(buf, kv)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) == 0
    return kv_np, d, buf


def _container(d, buf, cap=None):
    import torch
    cap = d.container_bytes(d.max_payload_bytes) if cap is None else cap
    out = torch.full(((cap + 15) // 16 * 16 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    kvc.kvc_serialize(d, buf.cdf, buf.max1, buf.stream_len, buf.slab_off, buf.payload, out,
                      buf.dev_status, out_cap=cap)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", list(CASES))
def test_container_is_byte_identical_and_round_trips(name):
    import torch
    cfg = CASES[name]
    say(f"[gpu] container {name}")
    kv_np, d, buf = _encode(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, _, T, C = kv_np.shape
    r = oracle.codec(kv_np, bins, Tc)
    want = oracle.serialize(r["cdf"], r["max1"], r["stream_len"], r["payload"], bins, Tc)
    out = _container(d, buf)
    assert int(buf.dev_status.item()) == 0
    got = out[: want.size].cpu().numpy()
    assert np.array_equal(got, want), np.argwhere(got != want)[:5].tolist()
    assert int(out[want.size]) == 0xA5  # nothing past the container

    # back into fresh buffers, then decode straight from the container
    n = want.size
    inp = out[:n].clone()
    fresh = kvc.alloc(d, out_dtype=kvc.KVC_F16, with_dec_sym=True)
    for t in (fresh.cdf, fresh.max1, fresh.stream_len, fresh.slab_off):
        t.fill_(-1)
    kvc.kvc_deserialize(d, inp, fresh.cdf, fresh.max1, fresh.stream_len, fresh.slab_off,
                        fresh.dev_status)
    torch.cuda.synchronize()
    assert int(fresh.dev_status.item()) == 0
    ncdf = d.cdf_bytes // 2
    assert torch.equal(fresh.cdf[:ncdf], buf.cdf[:ncdf])
    assert torch.equal(fresh.max1[: L * 2 * T], buf.max1[: L * 2 * T])
    assert torch.equal(fresh.stream_len[: d.n_streams], buf.stream_len[: d.n_streams])
    assert torch.equal(fresh.slab_off[: d.n_slabs + 1], buf.slab_off[: d.n_slabs + 1])
    po = d.container_payload_offset
    kvc.kvc_decode(d, inp.data_ptr() + po, fresh.slab_off, fresh.stream_len, fresh.cdf, fresh.max1,
                   fresh.dec_sym, fresh.out, kvc.KVC_F16, fresh.dev_status, payload_bytes=n - po)
    torch.cuda.synchronize()
    assert int(fresh.dev_status.item()) == 0
    n_el = L * 2 * T * C
    assert np.array_equal(fresh.dec_sym[:n_el].cpu().numpy().reshape(L, 2, T, C), r["sym"])
    got16 = fresh.out[:n_el].cpu().view(torch.int16).numpy().view(np.uint16).reshape(L, 2, T, C)
    assert np.array_equal(got16, r["out_f16"])


def test_oracle_container_deserializes_on_the_gpu():
    import torch
    cfg = CASES["ragged_L3_C40_T300_Tc128"]
    kv_np, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    L, _, T, C = kv_np.shape
    r = oracle.codec(kv_np, bins, Tc)
    data = oracle.serialize(r["cdf"], r["max1"], r["stream_len"], r["payload"], bins, Tc)
    d = kvc.Desc(L, C, T, bins, Tc)
    buf = kvc.alloc(d)
    inp = torch.from_numpy(data).cuda()
    kvc.kvc_deserialize(d, inp, buf.cdf, buf.max1, buf.stream_len, buf.slab_off, buf.dev_status)
    torch.cuda.synchronize()
    assert int(buf.dev_status.item()) == 0
    assert np.array_equal(buf.cdf[: d.cdf_bytes // 2].cpu().numpy().view(np.uint16),
                          r["cdf"].reshape(-1))
    assert np.array_equal(buf.slab_off[: d.n_slabs + 1].cpu().numpy().view(np.uint64), r["slab_off"])


def test_error_flags():
    import torch
    cfg = CASES["c1"]
    kv_np, d, buf = _encode(cfg)
    n = d.container_bytes(int(buf.slab_off[d.n_slabs].item()))

    # too small for the payload: flagged, and nothing written at or past the cap
    cap = d.container_payload_offset + 16
    assert cap < n
    out = _container(d, buf, cap=cap)
    assert int(buf.dev_status.item()) & kvc.KVC_DEV_PAYLOAD_OVERFLOW
    assert bool((out[cap:] == 0xA5).all())
    buf.dev_status.zero_()

    # a CDF row whose implied entries do not hold
    saved = buf.cdf.clone()
    buf.cdf[d.alphabet - 1] = 7  # slab 0, channel 0, last entry
    _container(d, buf)
    assert int(buf.dev_status.item()) & kvc.KVC_DEV_BAD_CDF
    buf.cdf.copy_(saved)
    buf.dev_status.zero_()

    # header or lengths that do not match the descriptor
    good = _container(d, buf)[:n].clone()
    assert int(buf.dev_status.item()) == 0
    fresh = kvc.alloc(d)
    for pos, val in ((0, 0), (12, 17), (64, 8)):  # magic, C, first bins byte
        bad = good.clone()
        bad[pos] = val
        fresh.dev_status.zero_()
        kvc.kvc_deserialize(d, bad, fresh.cdf, fresh.max1, fresh.stream_len, fresh.slab_off,
                            fresh.dev_status)
        torch.cuda.synchronize()
        assert int(fresh.dev_status.item()) & kvc.KVC_DEV_BAD_CONTAINER, pos
    bad = good.clone()
    bad[d.container_payload_offset - 16] ^= 1  # a stream length: no longer sums to the payload
    fresh.dev_status.zero_()
    kvc.kvc_deserialize(d, bad, fresh.cdf, fresh.max1, fresh.stream_len, fresh.slab_off,
                        fresh.dev_status)
    torch.cuda.synchronize()
    assert int(fresh.dev_status.item()) & kvc.KVC_DEV_BAD_CONTAINER


def test_full_size_round_trip_llama_8k():
    """At the full 8K-token shape: the container's size follows the format, and
    decoding from it gives what decoding the encoder's buffers gives."""
    import torch
    cfg = kvgen.CONFIGS["c3"]
    say("[gpu] container c3 full size")
    kv_np, d, buf = _encode(cfg)
    pb = int(buf.slab_off[d.n_slabs].item())
    out = _container(d, buf)
    n = d.container_bytes(pb)
    assert int(buf.dev_status.item()) == 0
    assert int(out[40:48].cpu().numpy().view(np.uint64)[0]) == n
    fresh = kvc.alloc(d, out_dtype=kvc.KVC_F16)
    kvc.kvc_deserialize(d, out[:n], fresh.cdf, fresh.max1, fresh.stream_len, fresh.slab_off,
                        fresh.dev_status)
    kvc.decode(buf)
    po = d.container_payload_offset
    kvc.kvc_decode(d, out.data_ptr() + po, fresh.slab_off, fresh.stream_len, fresh.cdf, fresh.max1,
                   None, fresh.out, kvc.KVC_F16, fresh.dev_status, payload_bytes=n - po)
    torch.cuda.synchronize()
    assert int(fresh.dev_status.item()) == 0 and int(buf.dev_status.item()) == 0
    assert torch.equal(fresh.out, buf.out)
    bits = 8 * n / (cfg.n_elements)
    say(f"[gpu] c3 container {n} bytes, {bits:.4f} bits/elem")
