"""Helpers for the GPU tests: run the whole HIP path through the C ABI and
bring every intermediate back to the host."""
from __future__ import annotations

import sys

import numpy as np

import entropy_coding_02_amd as kvc


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(kv_np: np.ndarray, bins: np.ndarray, Tc: int, fused: bool = True,
            out_dtype: int = kvc.KVC_F16, exact_payload: bool = False, keep_device=False,
            cdf_chunks: int = 0):
    """kv_np: uint16 fp16 bits [L][2][T][C].  Returns a dict of numpy arrays."""
    import torch
    L, _, T, C = kv_np.shape
    d = kvc.Desc(L, C, T, bins, Tc, cdf_chunks=cdf_chunks)
    buf = kvc.alloc(d, out_dtype=out_dtype, with_dec_sym=True)
    kv = torch.from_numpy(kv_np.view(np.int16)).cuda() if kv_np.size else torch.empty(1, dtype=torch.int16, device="cuda")
    kvc.encode(buf, kv, fused_cdf=fused)
    torch.cuda.synchronize()
    enc_status = int(buf.dev_status.item())
    n_slabs = d.n_slabs
    slab_off = buf.slab_off[: n_slabs + 1].cpu().numpy().view(np.uint64)
    total = int(slab_off[-1])
    buf.dev_status.zero_()
    if exact_payload:
        # the smallest buffer the decoder accepts: the packed size rounded up to whole dwords
        # (at least 16 bytes), the padding filled with junk it must not use
        nb = max(16, (total + 3) // 4 * 4)
        pay = torch.full((nb,), 0xA5, dtype=torch.uint8, device="cuda")
        pay[:total] = buf.payload[:total]
        kvc.decode(buf, out_dtype=out_dtype, payload=pay, payload_bytes=nb)
    else:
        kvc.decode(buf, out_dtype=out_dtype)
    torch.cuda.synchronize()
    dec_status = int(buf.dev_status.item())
    n_el = L * 2 * T * C
    res = dict(
        desc=d, A=d.alphabet, enc_status=enc_status, dec_status=dec_status,
        sym=buf.sym[:n_el].cpu().numpy().reshape(L, 2, T, C),
        max1=buf.max1[: L * 2 * T].cpu().numpy().view(np.uint16).reshape(L, 2, T),
        cdf=buf.cdf[: d.cdf_bytes // 2].cpu().numpy().view(np.uint16).reshape(-1, L, 2, C, d.alphabet),
        stream_len=buf.stream_len[: d.n_streams].cpu().numpy().view(np.uint16),
        slab_off=slab_off,
        payload=buf.payload[:total].cpu().numpy(),
        dec_sym=buf.dec_sym[:n_el].cpu().numpy().reshape(L, 2, T, C),
    )
    out = buf.out[:n_el].cpu()
    res["out"] = (out.view(torch.int16).numpy().view(np.uint16) if out_dtype == kvc.KVC_F16
                  else out.numpy()).reshape(L, 2, T, C)
    if keep_device:
        res["buf"] = buf
    return res
