#!/usr/bin/env python3
"""Throughput of the KV codec hot path on one MI355X.

One step = the whole hot path over one batch of synthetic fp16 KV already in
HBM: quantize + CDF (kvc_quantize), range coding + packing (kvc_encode), and
decode with fused dequantization to fp16 (kvc_decode).  Every step first
writes a 512 MiB buffer, which evicts the L2 caches and the 256 MB MALL, so
no stage reads what the previous step left in a cache.  `value` is fp16 input
bytes per second of whole steps (GB/s), the eviction write included.
Per-stage times (median and p90 over the steps) come from HIP events recorded
on the stream the kernels run on, around the stages only.  The roofline
object is for the decode kernel (one launch per kvc_decode call).  The CPU
baseline is the plain oracle on a bounded sample of the same workload, on one
core and fanned out over chunks on the host's cores.

The default workload is the 34B-class model at 80K tokens (48 layers, 8 x 128
KV channels, 313 chunks, the last of 128 tokens), the largest configuration.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "KV codec encode/decode GB/s (fp16 in) + bits/elem + % HBM roofline, 1 GPU"
HBM_PEAK_GBPS = 8000.0
DEFAULT_CONFIG = "c4"
FLUSH_BYTES = 512 << 20  # written before every step: more than the MALL and all L2s hold


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the container, 8-bit, quality-level and token-delta legs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also launch one elementwise kernel that reads and writes 256 MiB "
                         "(the reference for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("READ_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files of a --calibrate-copy "
                         "run (READ_COUNTERS, then WRITE_COUNTERS) into profiles/traffic.json")
    return ap.parse_args()


CSRC = "entropy_coding_02_amd/csrc/"
COMMON = [CSRC + "kvc_common.h"]
# the sources each kernel is built from (a traffic record is used only while they are unchanged)
KERNEL_SOURCES = {
    "k_decode": [CSRC + "kvc_decode.hip", CSRC + "lane_coder.h", CSRC + "pair_tile.h"] + COMMON,
    "k_decode_group": [CSRC + "kvc_decode.hip", CSRC + "lane_coder.h", CSRC + "pair_tile.h"] + COMMON,
    "k_decode_mode": [CSRC + "kvc_decode.hip", CSRC + "lane_coder.h", CSRC + "pair_tile.h"] + COMMON,
    "k_quant_cdf_levels": [CSRC + "kvc_quantize.hip"] + COMMON,
    "k_quantize_rows": [CSRC + "kvc_quantize.hip"] + COMMON,
    "k_cdf_wide": [CSRC + "kvc_cdf.hip"] + COMMON,
    "k_slab_sum": [CSRC + "kvc_encode.hip"] + COMMON,
    "k_scan": [CSRC + "kvc_encode.hip"] + COMMON,
    "k_encode": [CSRC + "kvc_encode.hip", CSRC + "lane_coder.h", CSRC + "pair_tile.h"] + COMMON,
    "k_encode_split": [CSRC + "kvc_encode.hip", CSRC + "lane_coder.h", CSRC + "pair_tile.h"] + COMMON,
    "k_pack": [CSRC + "kvc_encode.hip"] + COMMON,
    "k_pack_flat": [CSRC + "kvc_encode.hip"] + COMMON,
    "k_quant_cdf": [CSRC + "kvc_quantize.hip"] + COMMON,
}
COPY_BYTES = 256 << 20


def sources_sha256(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()


def kernel_key(name: str):
    low = name.lower()
    if "elementwise" in low and "add<unsigned char>" in low:
        return "copy"  # the --calibrate-copy kernel (a uint8 add; the other legs add floats)
    base = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0].split("<")[0]
    return base.strip() if base.strip() in KERNEL_SOURCES else None


READ_COUNTERS = ["TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum",
                 "TCC_EA0_RDREQ_128B_sum"]
WRITE_COUNTERS = ["TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_RDREQ_DRAM_sum",
                  "TCC_EA0_WRREQ_DRAM_sum"]


def summarize_pmc(read_csv: str, write_csv: str, workload: str):
    """HBM bytes per dispatch of each hot kernel from two rocprofv3 --pmc runs
    of the L2-to-memory request counters (READ_COUNTERS, then WRITE_COUNTERS):
    reads weighted by request size (32 / 64 / 128 bytes), writes as 32- and
    64-byte requests, and the share of requests that went to DRAM.  The
    --calibrate-copy kernel (COPY_BYTES read and written) gives the scale that
    turns the weighted counts into bytes (it should be about 1).  A call is a
    run of consecutive dispatches of one kernel (kvc_decode launches the
    mode-first decoder once per run of layers with equal search depth, then
    a guard launch): their counts are summed.  Medians over calls, into
    profiles/traffic.json."""
    import csv

    def per_kernel(path, names):
        disp = {}  # dispatch id -> (kernel key, {counter: value})
        for r in csv.DictReader(open(path)):
            if r.get("Counter_Name") not in names:
                continue
            did = int(r["Dispatch_Id"])
            key, d = disp.setdefault(did, (kernel_key(r["Kernel_Name"]), {}))
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        vals, prev, call = {}, None, None
        for did in sorted(disp):
            key, d = disp[did]
            if key is None:
                prev = None
                continue
            if key != prev:
                call = vals.setdefault(key, {}).setdefault(did, {})
            for c, v in d.items():
                call[c] = call.get(c, 0.0) + v
            prev = key
        return vals

    def med(xs):
        xs = sorted(xs)
        return xs[len(xs) // 2]

    rd, wr = per_kernel(read_csv, READ_COUNTERS), per_kernel(write_csv, WRITE_COUNTERS)

    def read_bytes(c):
        return 32 * c["TCC_EA0_RDREQ_32B_sum"] + 64 * c["TCC_EA0_RDREQ_64B_sum"] + 128 * c["TCC_EA0_RDREQ_128B_sum"]

    def write_bytes(c):
        n64 = c["TCC_EA0_WRREQ_64B_sum"]
        return 32 * (c["TCC_EA0_WRREQ_sum"] - n64) + 64 * n64

    rf = COPY_BYTES / med([read_bytes(c) for c in rd["copy"].values()])
    rw = COPY_BYTES / med([write_bytes(c) for c in wr["copy"].values()])
    path = os.path.join(ROOT, "profiles", "traffic.json")
    db = json.load(open(path)) if os.path.exists(path) else {}
    for k in sorted(set(rd) & set(wr) - {"copy"}):
        r_b = med([read_bytes(c) for c in rd[k].values()])
        w_b = med([write_bytes(c) for c in wr[k].values()])
        req = med([c["TCC_EA0_RDREQ_sum"] for c in rd[k].values()])
        unsized = req - med([c["TCC_EA0_RDREQ_32B_sum"] + c["TCC_EA0_RDREQ_64B_sum"] + c["TCC_EA0_RDREQ_128B_sum"]
                             for c in rd[k].values()])
        dram = med([c["TCC_EA0_RDREQ_DRAM_sum"] for c in wr[k].values()])
        wdram = med([c["TCC_EA0_WRREQ_DRAM_sum"] for c in wr[k].values()])
        wreq = med([c["TCC_EA0_WRREQ_sum"] for c in wr[k].values()])
        db[f"{k}/{workload}"] = {
            "bytes_per_launch": round(r_b * rf + w_b * rw),
            "read_bytes": round(r_b * rf), "write_bytes": round(w_b * rw),
            "read_requests": req, "read_requests_of_no_size_counter": unsized,
            "read_dram_share": round(dram / req, 4) if req else None,
            "write_dram_share": round(wdram / wreq, 4) if wreq else None,
            "copy_scale_read": rf, "copy_scale_write": rw,
            "counters": READ_COUNTERS + WRITE_COUNTERS,
            "sources": KERNEL_SOURCES[k], "source_sha256": sources_sha256(KERNEL_SOURCES[k]),
        }
        print(k, json.dumps(db[f"{k}/{workload}"]))
    json.dump(db, open(path, "w"), indent=1, sort_keys=True)


def traffic_for(kernel: str, workload: str):
    """HBM bytes per launch from committed counter runs, if they were taken on
    the current kernel source (profiles/traffic.json records its hash)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{kernel}/{workload}")
    except Exception:
        return None
    if not rec:
        return None
    ok = sources_sha256(rec.get("sources", [])) == rec.get("source_sha256")
    return rec.get("bytes_per_launch") if ok else None


def container_leg(kvc, d, buf, cfg, stream, steps):
    """The byte container (kvc_serialize / kvc_deserialize) of the last step's
    output: its size in bits per element and each call's time (HIP events on
    the launch stream, median of `steps` calls), outside the timed step."""
    import torch
    pb = int(buf.slab_off[d.n_slabs].item())
    n = d.container_bytes(pb)
    out = torch.empty((n + 15) // 16 * 16, dtype=torch.uint8, device="cuda")
    cdf2 = torch.empty_like(buf.cdf)
    max2 = torch.empty_like(buf.max1)
    len2 = torch.empty_like(buf.stream_len)
    off2 = torch.empty_like(buf.slab_off)
    ser, des = [], []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        kvc.kvc_serialize(d, buf.cdf, buf.max1, buf.stream_len, buf.slab_off, buf.payload, out,
                          buf.dev_status, stream, out_cap=n)
        e[1].record(stream)
        kvc.kvc_deserialize(d, out, cdf2, max2, len2, off2, buf.dev_status, stream, in_bytes=n)
        e[2].record(stream)
        torch.cuda.synchronize()
        ser.append(e[0].elapsed_time(e[1]))
        des.append(e[1].elapsed_time(e[2]))
    assert int(buf.dev_status.item()) == 0, "device status flags set by the container calls"
    assert torch.equal(cdf2, buf.cdf) and torch.equal(off2[: d.n_slabs + 1], buf.slab_off[: d.n_slabs + 1])
    n_el = cfg.n_elements
    full = pb + d.cdf_bytes + 2 * (2 * d.n_layers * d.n_tokens) + 2 * d.n_streams
    return {"bytes": n, "bits_per_elem": round(8 * n / n_el, 4),
            "bits_per_elem_full_tables": round(8 * full / n_el, 4),
            "serialize_ms": round(statistics.median(ser), 4),
            "deserialize_ms": round(statistics.median(des), 4)}


def rel_rmse_f16(y, x, piece=1 << 26):
    """sqrt(mean((y - x)^2)) / sqrt(mean(x^2)) of two flat tensors (x fp16,
    y fp16 or fp32), accumulated in fp64 a slice at a time (no full-size temporaries)."""
    import torch
    se = sx = 0.0
    for i in range(0, x.numel(), piece):
        xs = x[i:i + piece].double()
        ds = y[i:i + piece].double() - xs
        se += float(torch.dot(ds, ds))
        sx += float(torch.dot(xs, xs))
    return (se / sx) ** 0.5 if sx > 0 else 0.0


def int8_leg(kvc, d, kvt, buf, cfg, stream, steps, container_bits):
    """The 8-bit comparator on the same input: its size next to the codec's
    container, and both reconstructions' relative RMS error against the fp16
    input (the codec's from the last step's decode), outside the timed step."""
    import torch
    C = cfg.n_channels
    g = 128 if C % 128 == 0 else C  # head_dim of the workloads' 8 x 128 heads
    n_el, n_g = cfg.n_elements, cfg.n_elements // g
    q = torch.empty(n_el, dtype=torch.uint8, device="cuda")
    sc = torch.empty(n_g, dtype=torch.float32, device="cuda")
    zp = torch.empty(n_g, dtype=torch.uint8, device="cuda")
    y8 = torch.empty(n_el, dtype=torch.float32, device="cuda")  # the page's dequantizer returns fp32
    qt, dt = [], []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        kvc.kvc_int8_quantize(d, g, kvt, q, sc, zp, buf.dev_status, stream)
        e[1].record(stream)
        kvc.kvc_int8_dequantize(d, g, q, sc, zp, y8, kvc.KVC_F32, stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        qt.append(e[0].elapsed_time(e[1]))
        dt.append(e[1].elapsed_time(e[2]))
    if int(buf.dev_status.item()):
        raise RuntimeError(f"8-bit comparator leg: device status {int(buf.dev_status.item()):#x}")
    x = kvt.view(torch.float16).reshape(-1)

    def rel_rmse(y):
        return rel_rmse_f16(y.reshape(-1)[:n_el], x)

    bits8 = 8 + 8 * 5 / g  # u8 code per element, fp32 scale and u8 zero point per group
    return {"group": g, "bits_per_elem": round(bits8, 4),
            "size_ratio_vs_codec_container": round(bits8 / container_bits, 3),
            "rel_rmse_int8": round(rel_rmse(y8), 6),
            "rel_rmse_codec": round(rel_rmse(buf.out.view(torch.float16)), 6), "int8_output": "fp32",
            "quantize_ms": round(statistics.median(qt), 4),
            "dequantize_ms": round(statistics.median(dt), 4)}


def levels_leg(kvc, cfg, kvt, stream, steps):
    """Three quality levels of the same input (the workload's bins, then
    halved twice, at least 4): one kvc_quantize_levels call against one
    kvc_quantize per level, and each level's container size and relative RMS
    error after encode, serialize and decode, outside the timed step."""
    import numpy as np
    import torch
    L, C, T, Tc = cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.chunk_tokens
    b0 = cfg.bins()
    tables = [b0, np.maximum(b0 // 2, 4), np.maximum(b0 // 4, 4)]
    tables = [t + (t % 2) for t in tables]
    descs = [kvc.Desc(L, C, T, t, Tc) for t in tables]
    # symbols and CDFs per level; one set of coder buffers, decoded output
    # included, serves every level in turn (the largest level sizes it)
    shared = kvc.alloc(descs[0], out_dtype=kvc.KVC_F16)
    for d in descs[1:]:
        assert d.scratch_bytes <= descs[0].scratch_bytes and d.max_payload_bytes <= descs[0].max_payload_bytes
    bufs = [shared] + [dataclasses.replace(shared, desc=d, sym=torch.empty_like(shared.sym),
                                           cdf=torch.empty(d.cdf_bytes // 2, dtype=torch.int16, device="cuda"))
                       for d in descs[1:]]
    one, sep = [], []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        kvc.kvc_quantize_levels(descs, kvt, [b.sym for b in bufs], bufs[0].max1, [b.cdf for b in bufs],
                                bufs[0].dev_status, stream)
        e[1].record(stream)
        for d, b in zip(descs, bufs):
            kvc.kvc_quantize(d, kvt, b.sym, b.max1, b.cdf, b.dev_status, stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        one.append(e[0].elapsed_time(e[1]))
        sep.append(e[1].elapsed_time(e[2]))
    x = kvt.view(torch.float16).reshape(-1)
    out, level_bytes = [], []
    for t, d, b in zip(tables, descs, bufs):
        kvc.kvc_encode(d, b.sym, b.cdf, b.scratch, b.stream_len, b.slab_off, b.payload, b.dev_status,
                       stream)
        kvc.decode(b, stream=stream)
        torch.cuda.synchronize()
        assert int(b.dev_status.item()) == 0, "device status flags set in the levels leg"
        n = d.container_bytes(int(b.slab_off[d.n_slabs].item()))
        level_bytes.append(n)
        out.append({"bins": sorted({int(v) for v in t.reshape(-1)}, reverse=True),
                    "container_bits_per_elem": round(8 * n / cfg.n_elements, 4),
                    "rel_rmse": round(rel_rmse_f16(b.out[: cfg.n_elements], x), 6)})
    res = {"levels": out, "one_pass_ms": round(statistics.median(one), 4),
           "level_by_level_ms": round(statistics.median(sep), 4)}
    res["streaming"] = streaming_leg(kvc, cfg, descs, bufs, max(level_bytes), steps)
    return res


def streaming_leg(kvc, cfg, descs, bufs, max_level_bytes, steps):
    """kvc_stream_encode over the quality levels: chunk j at the level of a
    fixed schedule (runs of 16 chunks cycling 0, 1, 2, 1), each chunk's
    container copied to page-locked host memory at its exact size.  Wall
    time of the whole call with the copies on a second stream (overlapped)
    and on the compute stream (serial), next to one plain device-to-host
    copy of the same number of bytes.  Outside the timed step."""
    import numpy as np
    import torch
    nc = descs[0].n_chunks
    cycle = [0, 1, 2, 1]
    sched = np.array([cycle[(j // 16) % 4] for j in range(nc)], np.int32)
    work = torch.empty(kvc.kvc_stream_work_bytes(descs, 0), dtype=torch.uint8, device="cuda")
    host = torch.empty(int(max_level_bytes * 1.05) + nc * 4096, dtype=torch.uint8).pin_memory()
    sizes = torch.zeros(nc, dtype=torch.int64).pin_memory()
    st = bufs[0].dev_status
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    syms, cdfs, max1 = [b.sym for b in bufs], [b.cdf for b in bufs], bufs[0].max1

    def run(two):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        kvc.kvc_stream_encode(descs, sched, syms, cdfs, max1, work, host, sizes, st, cs, xs if two else cs)
        return (time.perf_counter() - t0) * 1e3

    run(True)  # warm-up
    if int(st.item()):
        raise RuntimeError(f"streaming leg: device status {int(st.item()):#x}")
    reps = max(1, min(steps, 3))
    ov = statistics.median([run(True) for _ in range(reps)])
    se = statistics.median([run(False) for _ in range(reps)])
    total = int(sizes.sum().item())
    dev = torch.empty(total, dtype=torch.uint8, device="cuda")
    cp = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        host[:total].copy_(dev, non_blocking=True)
        torch.cuda.synchronize()
        cp.append((time.perf_counter() - t0) * 1e3)
    d2h = statistics.median(cp)
    in_bytes = 2 * cfg.n_elements
    del work, dev
    return {"chunks": nc, "schedule": "runs of 16 chunks at levels 0, 1, 2, 1, ...",
            "chunks_per_level": [int((sched == i).sum()) for i in range(len(descs))],
            "container_bytes": total, "bits_per_elem": round(8 * total / cfg.n_elements, 4),
            "overlapped_ms": round(ov, 3), "serial_ms": round(se, 3),
            "overlap_speedup": round(se / ov, 3), "d2h_only_ms": round(d2h, 3),
            "d2h_GBps": round(total / (d2h * 1e-3) / 1e9, 2),
            "overlapped_input_GBps": round(in_bytes / (ov * 1e-3) / 1e9, 2),
            "timing": "wall clock of kvc_stream_encode (it returns with every container in host memory)"}


def entropy_bound_bits(sym, L, T, C, A, span):
    """Sum over CDF tables (spans of `span` tokens) and channels of N_g * H,
    H the empirical entropy of the channel's symbols over the table's tokens:
    the least payload a coder with one static model per table can reach, in
    bits.  GPU bincount per (layer, K|V) row block."""
    import math
    import torch
    ng = -(-T // span)
    rows = sym[: 2 * L * T * C].view(2 * L, T, C)
    grp = torch.arange(T, device=sym.device) // span
    base = (grp[:, None] * C + torch.arange(C, device=sym.device)[None, :]) * A
    nlogn = 0.0
    for lk in range(2 * L):
        cnt = torch.bincount((base + rows[lk].long()).view(-1), minlength=ng * C * A).double()
        nz = cnt[cnt > 0]
        nlogn += float((nz * torch.log2(nz)).sum())
    sizes = [min(span, T - g * span) for g in range(ng)]
    return 2 * L * C * sum(n * math.log2(n) for n in sizes) - nlogn


def cdf_sharing_leg(kvc, cfg, kvt, buf, stream):
    """CDF tables shared by N consecutive chunks (N = 1: the page's per-chunk
    tables; 4; all: one table per (layer, K|V, channel)): container, payload
    and table bits per element, the payload against the entropy bound of the
    same tables, and the stage times of one run each (HIP events).  Outside
    the timed step; reuses the step's buffers (N = 1 has the most tables)."""
    import torch
    L, C, T, Tc = cfg.n_layers, cfg.n_channels, cfg.n_tokens, cfg.chunk_tokens
    bins = cfg.bins()
    n = cfg.n_elements
    per_table = 2 * C * int((bins - 2).sum())  # compact bytes of one table of every (layer, K|V)
    out = []
    for label, N in (("1", 1), ("4", 4), ("all", 1 << 30)):
        d = kvc.Desc(L, C, T, bins, Tc, cdf_chunks=N)
        b = dataclasses.replace(buf, desc=d)
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record(stream)
        kvc.kvc_quantize(d, kvt, b.sym, b.max1, b.cdf, b.dev_status, stream)
        e[1].record(stream)
        kvc.kvc_encode(d, b.sym, b.cdf, b.scratch, b.stream_len, b.slab_off, b.payload, b.dev_status, stream)
        e[2].record(stream)
        kvc.decode(b, stream=stream)
        e[3].record(stream)
        torch.cuda.synchronize()
        if int(b.dev_status.item()):
            raise RuntimeError(f"CDF sharing leg: device status {int(b.dev_status.item()):#x} at N = {label}")
        pay = int(b.slab_off[d.n_slabs].item())
        s_eff = min(N, d.n_chunks) if d.n_chunks else 1  # chunks per table as stored
        ng = -(-d.n_chunks // s_eff)
        assert d.cdf_bytes == ng * 2 * L * C * d.alphabet * 2
        bound = entropy_bound_bits(b.sym, L, T, C, d.alphabet, max(min(s_eff * Tc, T), 1))
        out.append({"chunks_per_table": label, "tables_per_layer_kv": ng,
                    "container_bits_per_elem": round(8 * d.container_bytes(pay) / n, 4),
                    "payload_bits_per_elem": round(8 * pay / n, 4),
                    "table_bits_per_elem": round(8 * ng * per_table / n, 4),
                    "entropy_bound_bits_per_elem": round(bound / n, 4),
                    "payload_over_bound": round(8 * pay / bound, 4) if bound > 0 else None,
                    "quantize_cdf_ms": round(e[0].elapsed_time(e[1]), 4),
                    "encode_ms": round(e[1].elapsed_time(e[2]), 4),
                    "decode_ms": round(e[2].elapsed_time(e[3]), 4)})
    return {"tables": out, "timing": "one run each, HIP events; quantize_cdf includes the tables"}


def delta_leg(kvc, d, buf, cfg, kvt, stream, steps):
    """Token-delta coding (anchors every G chunk-relative tokens) in front of
    the codec: container size and relative RMS error after forward, encode,
    decode and inverse, for a few anchor spacings at the workload's bins and
    one at halved bins, next to the plain codec; forward and inverse times
    (HIP events, median of `steps`).  Outside the timed step; reuses the
    step's buffers."""
    import numpy as np
    import torch
    n = cfg.n_elements
    x = kvt.view(torch.float16).reshape(-1)
    dlt = torch.empty_like(kvt)
    st = torch.zeros(1, dtype=torch.int32, device="cuda")

    def run(desc, G):
        b = dataclasses.replace(buf, desc=desc)
        if G:
            kvc.kvc_delta_forward(desc, G, kvt, dlt, st, stream)
        kvc.encode(b, dlt if G else kvt, stream=stream)
        kvc.decode(b, stream=stream)
        if G:
            kvc.kvc_delta_inverse(desc, G, b.out, stream)
        torch.cuda.synchronize()
        flags = int(st.item()) | int(b.dev_status.item())
        if flags:
            raise RuntimeError(f"token-delta leg: device status {flags:#x} at anchor spacing {G}")
        nb = desc.container_bytes(int(b.slab_off[desc.n_slabs].item()))
        r = {"container_bits_per_elem": round(8 * nb / n, 4),
             "rel_rmse": round(rel_rmse_f16(b.out[:n].view(torch.float16), x), 6)}
        if G:  # deltas clamped to +-65504 (counted in rel_rmse; an upper bound: inputs may sit there)
            r["saturated_elems"] = int((dlt.view(torch.float16).abs() == 65504.0).sum().item())
        return r

    L = cfg.n_layers
    b0 = cfg.bins()
    half = np.maximum(b0 // 2, 4)
    half = half + (half % 2)
    d_half = kvc.Desc(L, cfg.n_channels, cfg.n_tokens, half, cfg.chunk_tokens)
    out = {"plain": run(d, 0), "anchors": []}
    for G, desc, tag in ((2, d, b0), (4, d, b0), (8, d, b0), (4, d_half, half)):
        r = run(desc, G)
        r.update(anchor_tokens=G, bins=sorted({int(v) for v in tag.reshape(-1)}, reverse=True))
        out["anchors"].append(r)
    fw, iv = [], []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        kvc.kvc_delta_forward(d, 4, kvt, dlt, st, stream)
        e[1].record(stream)
        kvc.kvc_delta_inverse(d, 4, dlt, stream)
        e[2].record(stream)
        torch.cuda.synchronize()
        fw.append(e[0].elapsed_time(e[1]))
        iv.append(e[1].elapsed_time(e[2]))
    out["forward_ms"] = round(statistics.median(fw), 4)
    out["inverse_ms"] = round(statistics.median(iv), 4)
    out["forward_GBps"] = round(4 * n / (out["forward_ms"] * 1e-3) / 1e9, 1)  # 2 B in + 2 B out
    del dlt
    return out


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, kv_np, budget_s=8.0):
    """The oracle, as it stands, over a bounded sample of the workload: whole
    chunks (all layers, K and V, 256 tokens), the whole hot path on each
    (quantize, CDF, encode, pack, decode, dequantize).  First on one core
    (one chunk again and again for about budget_s), then fanned out over
    chunks on the host's cores (one chunk per thread at a time, for about
    budget_s; the oracle releases the GIL, so the threads run in parallel).
    The reported value is the all-core rate."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    L, T, C, Tc = cfg.n_layers, cfg.n_tokens, cfg.n_channels, cfg.chunk_tokens
    bins = cfg.bins()
    NC = (T + Tc - 1) // Tc

    def chunk(j):
        t0 = j * Tc
        return np.ascontiguousarray(kv_np[:, :, t0:min(T, t0 + Tc)])

    def run(sub):
        r = oracle.codec(sub, bins, Tc)
        assert not r["corrupt"]
        return sub.size

    # one core
    sub0 = chunk(0)
    n1, t1, p1 = 0, 0.0, 0
    while t1 < budget_s:
        t0 = time.perf_counter()
        n1 += run(sub0)
        t1 += time.perf_counter() - t0
        p1 += 1
    one = 2 * n1 / t1 / 1e9
    # all cores: distinct chunks, one per thread at a time
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(avail, 16))  # the GPU machine's CPU share is 16 cores
    chunks = [chunk(j % NC) for j in range(threads)]
    na, rounds = 0, 0
    ta0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=threads) as ex:
        while time.perf_counter() - ta0 < budget_s or rounds == 0:
            na += sum(ex.map(run, chunks))
            rounds += 1
    ta = time.perf_counter() - ta0
    allc = 2 * na / ta / 1e9
    sample = (f"one core: {p1} pass(es) of the whole hot path over chunk 0 (all {L} layers, K and V, "
              f"{sub0.shape[2]} tokens, {sub0.size} elements) in {t1:.1f} s; all cores: {rounds} "
              f"round(s) of {threads} distinct chunks in parallel threads in {ta:.1f} s")
    return {"value": round(allc, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample, "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "affinity_cores": avail, "one_core_GBps": round(one, 4), "all_core_GBps": round(allc, 4)}


def main():
    args = parse()
    if args.summarize_pmc:
        import kvgen
        summarize_pmc(*args.summarize_pmc, kvgen.CONFIGS[args.config].workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this codec is measured on one GPU; --gpus must be 1 "
                                   "(the path is not sharded across GPUs)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import entropy_coding_02_amd as kvc
    import kvgen

    cfg = kvgen.CONFIGS[args.config]
    L, T, C, Tc = cfg.n_layers, cfg.n_tokens, cfg.n_channels, cfg.chunk_tokens
    kv_np, _ = kvgen.generate(cfg)
    torch.cuda.set_device(0)
    kvt = torch.from_numpy(kv_np.view(np.int16)).cuda()
    d = kvc.Desc(L, C, T, cfg.bins(), Tc)
    buf = kvc.alloc(d, out_dtype=kvc.KVC_F16)
    stream = torch.cuda.current_stream()

    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")

    def step(ev=None):
        flush.fill_(1)  # evict L2 and MALL (outside the stage events)
        if ev:
            ev[0].record(stream)
        kvc.kvc_quantize(d, kvt, buf.sym, buf.max1, buf.cdf, buf.dev_status, stream)
        if ev:
            ev[1].record(stream)
        kvc.kvc_encode(d, buf.sym, buf.cdf, buf.scratch, buf.stream_len, buf.slab_off, buf.payload,
                       buf.dev_status, stream)
        if ev:
            ev[2].record(stream)
        kvc.kvc_decode(d, buf.payload, buf.slab_off, buf.stream_len, buf.cdf, buf.max1, None, buf.out,
                       kvc.KVC_F16, buf.dev_status, stream)
        if ev:
            ev[3].record(stream)

    if args.calibrate_copy:
        # one kernel that reads COPY_BYTES and writes COPY_BYTES
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.add(src, 1, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert int(buf.dev_status.item()) == 0, "device status flags set"

    ms_step = (t1 - t0) * 1e3 / args.steps

    def p90(v):
        v = sorted(v)
        return v[min(len(v) - 1, int(0.9 * len(v)))]

    t_q = [e[0].elapsed_time(e[1]) for e in evs]
    t_e = [e[1].elapsed_time(e[2]) for e in evs]
    t_d = [e[2].elapsed_time(e[3]) for e in evs]
    t_s = [e[0].elapsed_time(e[3]) for e in evs]
    q_ms, e_ms, d_ms = statistics.median(t_q), statistics.median(t_e), statistics.median(t_d)
    d_avg = sum(t_d) / args.steps
    in_bytes = cfg.input_bytes
    n_el = cfg.n_elements
    A = d.alphabet
    payload = int(buf.slab_off[d.n_slabs].item())
    cdf_b, max1_b, len_b, off_b = d.cdf_bytes, 2 * (L * 2 * T), 2 * d.n_streams, 8 * (d.n_slabs + 1)
    side = cdf_b + max1_b + len_b + off_b
    # algorithmic bytes per call of each stage (what it must read and write at least)
    alg = {
        # fp16 in; symbols, max1 and CDFs out
        "quantize_cdf": 2 * n_el + n_el + max1_b + cdf_b,
        # symbols and CDFs in; payload, stream lengths and slab offsets out
        "encode_pack": n_el + cdf_b + payload + len_b + off_b,
        # payload, CDFs, max1, stream lengths, slab offsets in; fp16 out
        "decode_dequant": payload + side + 2 * n_el,
    }
    ms = {"quantize_cdf": q_ms, "encode_pack": e_ms, "decode_dequant": d_ms}
    stages = {k: {"ms": round(ms[k], 4), "algorithmic_bytes": alg[k],
                  "GBps": round(alg[k] / (ms[k] * 1e-3) / 1e9, 1),
                  "frac_hbm": round(alg[k] / (ms[k] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)} for k in alg}
    # the decode stage is one kvc_decode call: its duration is the stage's
    dec_bytes = alg["decode_dequant"]
    # the kernel kvc_decode launches: several lanes per stream on small launches, else one lane
    # per stream with the mode-first search for rows of 5 to 64 entries (once per run of layers
    # with equal search depth, then a guard launch), binary lifting otherwise
    dec_kernel = ("k_decode_group" if d.decode_lanes > 1 else
                  "k_decode_mode" if 4 < d.alphabet <= 64 else "k_decode")
    achieved = dec_bytes / (d_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(in_bytes / (ms_step * 1e-3) / 1e9, 3),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32+u32",
        "data": "synthetic",
        "config": {"workload": cfg.workload, "layers": L, "channels": C, "tokens": T,
                   "chunk_tokens": Tc, "bins": [list(s) for s in cfg.layer_bins], "alphabet": A,
                   "input": "fp16 [L][2][T][C]", "output": "fp16"},
        "encode_GBps": round(in_bytes / ((q_ms + e_ms) * 1e-3) / 1e9, 3),
        "decode_GBps": round(in_bytes / (d_ms * 1e-3) / 1e9, 3),
        "stage_ms": {k: round(v, 4) for k, v in ms.items()},
        "stage_ms_p90": {"quantize_cdf": round(p90(t_q), 4), "encode_pack": round(p90(t_e), 4),
                         "decode_dequant": round(p90(t_d), 4)},
        "hot_path_ms": {"median": round(statistics.median(t_s), 4), "p90": round(p90(t_s), 4)},
        "timing": (f"each step writes {FLUSH_BYTES >> 20} MiB first (evicting L2 and MALL); value and "
                   "ms_per_step are wall-clock over the K steps including that write; stage times are "
                   "HIP events around the stages on their stream"),
        "stages": stages,
        "payload_bits_per_elem": round(8 * payload / n_el, 4),
        "total_bits_per_elem": round(8 * (payload + side) / n_el, 4),
        "roofline": {"kernel": dec_kernel, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(dec_kernel, cfg.workload),
                     "algorithmic_bytes_per_launch": dec_bytes},
    }
    del flush
    if not args.no_legs:
        res["container"] = container_leg(kvc, d, buf, cfg, stream, args.steps)
        res["int8_comparator"] = int8_leg(kvc, d, kvt, buf, cfg, stream, args.steps,
                                          res["container"]["bits_per_elem"])
        res["quality_levels"] = levels_leg(kvc, cfg, kvt, stream, args.steps)
        res["streaming"] = res["quality_levels"].pop("streaming")
        res["token_delta"] = delta_leg(kvc, d, buf, cfg, kvt, stream, args.steps)
        res["cdf_sharing"] = cdf_sharing_leg(kvc, cfg, kvt, buf, stream)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, kv_np)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
