"""kvc_encode_noalloc (the encoder with the library's own per-GPU workspace,
for callers that cannot allocate) against kvc_encode with a caller
workspace: stream lengths, slab offsets, payload bytes and status bit for
bit, on two calls in a row, the second with a smaller input (the shared
workspace then holds the first call's bytes), then a decode of the second
call's output back to its symbols.  A shape whose workspace exceeds the
array is refused before any launch."""
from __future__ import annotations

import numpy as np
import pytest

import entropy_coding_02_amd as kvc
import kvgen
import oracle
from gpu_util import say

pytestmark = pytest.mark.gpu


def _encode_both(cfg):
    import torch
    kv, _ = kvgen.generate(cfg)
    bins, Tc = cfg.bins(), cfg.chunk_tokens
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, bins, Tc)
    assert d.scratch_bytes <= kvc.KVC_NOALLOC_SCRATCH_BYTES
    a = kvc.alloc(d, with_dec_sym=True)
    kvt = torch.from_numpy(kv.view(np.int16)).cuda()
    kvc.kvc_quantize(d, kvt, a.sym, a.max1, a.cdf, a.dev_status)
    kvc.kvc_encode(d, a.sym, a.cdf, a.scratch, a.stream_len, a.slab_off, a.payload, a.dev_status)
    n = d.n_streams
    len2 = torch.full_like(a.stream_len, 0x7777)
    off2 = torch.full_like(a.slab_off, -1)
    pay2 = torch.full_like(a.payload, 0xA5)
    st2 = torch.zeros_like(a.dev_status)
    kvc.kvc_encode_noalloc(d, a.sym, a.cdf, len2, off2, pay2, st2)
    torch.cuda.synchronize()
    assert int(a.dev_status.item()) == 0 and int(st2.item()) == 0
    total = int(a.slab_off[d.n_slabs].item())
    assert torch.equal(len2[:n], a.stream_len[:n])
    assert torch.equal(off2[: d.n_slabs + 1], a.slab_off[: d.n_slabs + 1])
    assert torch.equal(pay2[:total], a.payload[:total])
    return d, a, kv, total


def test_encode_noalloc_matches_encode_twice_then_smaller():
    big = kvgen.CONFIGS["c2"]                                   # 16384 streams: the split encoder
    small = kvgen.CONFIGS["c2"].scaled(n_layers=3, n_tokens=200, chunk_tokens=64,
                                       layer_bins=((0, 1, 32), (1, 3, 16)))  # ragged chunks
    for cfg in (big, small):
        say(f"[gpu] noalloc encode: L={cfg.n_layers} C={cfg.n_channels} T={cfg.n_tokens} Tc={cfg.chunk_tokens}")
        d, a, kv, total = _encode_both(cfg)
    # the second (smaller) call's bytes decode back to its symbols and match the oracle
    import torch
    kvc.kvc_decode(d, a.payload, a.slab_off, a.stream_len, a.cdf, a.max1, a.dec_sym, a.out, kvc.KVC_F16,
                   a.dev_status)
    torch.cuda.synchronize()
    assert int(a.dev_status.item()) == 0
    n_el = kv.size
    assert torch.equal(a.dec_sym[:n_el], a.sym[:n_el])
    r = oracle.codec(kv, cfg.bins(), cfg.chunk_tokens)
    assert np.array_equal(a.payload[:total].cpu().numpy(), r["payload"])


def test_encode_noalloc_refuses_oversized_shape():
    cfg = kvgen.CONFIGS["c3"]                                  # 8K tokens: a 1 GB workspace
    d = kvc.Desc(cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.bins(), cfg.chunk_tokens)
    assert d.scratch_bytes > kvc.KVC_NOALLOC_SCRATCH_BYTES
    rc = kvc.lib().kvc_encode_noalloc(d.ref, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                      None, None)
    assert rc == kvc.KVC_ERR_CAPACITY
