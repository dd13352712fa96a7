"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the path over one batch: the store of the step's new
tokens and the attention, by default in one pa_decode_append launch
(``--separate-store``: pa_store_kv, then pa_decode).  The default workload is one Qwen3-8B
attention layer in decode: 32 sequences with contexts uniform in
[512, 4096], 32 query / 8 KV heads, head_dim 128, bf16, block size 16.  To
keep the 256 MB last-level cache from serving the KV, each step uses the
next of ``--layers`` independent layer caches (as a model's decode step
walks its layers), each laid out with the same sequence lengths.

Printed: one JSON line with the step throughput (algorithmic KV GB/s of the
decode reads), the decode kernel's roofline against 8 TB/s, secondary
measurements, and the oracle's CPU throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import copy
import json
import math
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0       # published dense bf16 matrix peak


# HBM bytes per decode_kernel launch on this workload (the launch that also
# stores the step's tokens, pa_decode_append), from rocprofv3 FETCH_SIZE
# and WRITE_SIZE passes scaled by the same counters on a plain 1 GiB copy
# (bench.py --copy-probe 1024), and the hash of the kernel sources they were
# taken on: once those sources change the figure no longer applies.
DECODE_TRAFFIC = {"sources_sha256": "7a6cfb9a9c8ffe173c27e6db2e6d68aeed638fa89e1d733295b7f798ae77942d",
                  "bytes_per_launch": 305882633}
DECODE_SOURCES = ("decode_kernel.h", "store_row.h", "pa_device.h", "pa_internal.h", "decode_bf16.hip")


def decode_sources_sha256():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_attention_26_amd", "csrc")
    for name in DECODE_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def decode_traffic():
    ok = DECODE_TRAFFIC["sources_sha256"] == decode_sources_sha256()
    return DECODE_TRAFFIC["bytes_per_launch"] if ok else None


def kv_bytes(lens, hkv, d, es):
    return int(np.sum(lens)) * 2 * hkv * d * es


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""), "compute_units": p.multi_processor_count,
            "memory_gib": round(p.total_memory / 2**30, 1)}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--layers", type=int, default=8, help="distinct layer caches cycled through")
    ap.add_argument("--partition", type=int, default=64, help="split-K partition tokens (0 = no split)")
    ap.add_argument("--separate-store", action="store_true",
                    help="store the new tokens with pa_store_kv before pa_decode instead of in the decode launch")
    ap.add_argument("--stamp-every", type=int, default=4,
                    help="time every N-th decode launch of the timed region with kernel-stamped events")
    ap.add_argument("--no-extras", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only-extra", choices=EXTRA_GROUPS, default=None,
                    help="run only this group of secondary measurements and print them (for profiling)")
    ap.add_argument("--hbm-probe", action="store_true",
                    help="only measure the HBM reference kernels (streaming read, copy, random 4 KB tiles)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 4 times (calibrates HBM byte counters)")
    ap.add_argument("--decode-trace", action="store_true",
                    help="only record per-wave phase times of the headline decode kernel (libpa_trace.so)")
    ap.add_argument("--decode-trace-out", default=None, metavar="NPY",
                    help="with --decode-trace: also save the raw records [launch][wave][16] (uint32) there")
    ap.add_argument("--decode-trace-workload", default="layer", choices=("layer", "long16", "long32"),
                    help="with --decode-trace: the Qwen3-8B layer (default) or the long-context batch at block "
                         "16 / 32 (512-token partitions, a cache flush before each launch)")
    return ap.parse_args()


_FLUSH = []


def flush_caches():
    """Read a 1 GiB device buffer (a sum over it): evicts a timed call's data
    from the L2s and the 256 MB last-level cache and leaves only clean lines
    behind.  (A fill would leave up to 256 MB of dirty lines, written back
    while the next timed call runs.)"""
    import torch
    if not _FLUSH:
        _FLUSH.append(torch.zeros(1 << 28, dtype=torch.float32, device="cuda"))
    _FLUSH[0].sum()


def timed_calls(fn, reps=50, warm=5, flush=True):
    """Median / p10 / p90 ms of fn() measured with events on the current
    stream, each rep preceded (outside its events) by a 1 GiB read that
    flushes the caches unless flush is False."""
    import torch
    for _ in range(warm):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        if flush:
            flush_caches()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


EXTRA_GROUPS = ("long_context", "mixed", "fork", "verify", "handoff", "hbm_probe")


def hbm_probe(torch):
    """Practical HBM ceilings on this GPU from the reference kernels of
    libpa_probe.so: a streaming read of 4 GiB, a copy of 2 GiB (read + write
    counted), and whole 4 KB tiles of a 4 GiB buffer read once each in a
    seeded random order (decode's access pattern), each with the default
    cache policy and with the non-temporal hint on the loads ("_nt").
    Median of 20 calls, each after a cache flush."""
    import ctypes as C
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_attention_26_amd", "libpa_probe.so")
    lib = C.CDLL(path)
    lib.pa_probe_read.argtypes = [C.c_void_p, C.c_size_t, C.c_int, C.c_void_p, C.c_int, C.c_void_p]
    lib.pa_probe_copy.argtypes = [C.c_void_p, C.c_void_p, C.c_size_t, C.c_int, C.c_int, C.c_void_p]
    lib.pa_probe_tiles.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int, C.c_void_p, C.c_int, C.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid = cus * 8
    stream = lambda: C.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = torch.zeros(1 << 32, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(grid * 256, dtype=torch.int32, device="cuda")
    half = big.numel() // 2
    n_tiles = big.numel() // 4096
    order = torch.from_numpy(np.random.default_rng(11).permutation(n_tiles).astype(np.int32)).cuda()
    out = {}
    for nt, sfx in ((0, ""), (1, "_nt")):
        med, _, _ = timed_calls(lambda: lib.pa_probe_read(big.data_ptr(), big.numel(), grid, sink.data_ptr(), nt,
                                                          stream()), 20)
        out["stream_read_4GiB" + sfx] = dict(GBps=round(big.numel() / med / 1e6, 1), ms=round(med, 4))
        med, _, _ = timed_calls(lambda: lib.pa_probe_copy(big.data_ptr(), big.data_ptr() + half, half, grid, nt,
                                                          stream()), 20)
        out["copy_2GiB_read_plus_write" + sfx] = dict(GBps=round(2 * half / med / 1e6, 1), ms=round(med, 4))
        med, _, _ = timed_calls(lambda: lib.pa_probe_tiles(big.data_ptr(), order.data_ptr(), n_tiles, cus * 4,
                                                           sink.data_ptr(), nt, stream()), 20)
        out["random_4KB_tiles_read_4GiB" + sfx] = dict(GBps=round(big.numel() / med / 1e6, 1), ms=round(med, 4))
    del big, sink, order
    torch.cuda.empty_cache()
    return out


def decode_trace(args, torch):
    """Per-wave phase times of the headline decode kernel, from the
    measurement build libpa_trace.so (the same kernel with s_memrealtime
    stamps, 100 MHz).  Each of args.steps launches (after args.warmup) runs
    alone: the step's store (the layer) or a cache flush (long context), then
    pa_decode with a trace buffer armed, then a synchronisation.  Times are
    microseconds from the launch's first wave start; medians over the waves of
    a launch, then over the launches."""
    import ctypes as C
    from paged_kv_attention_26_amd import _lib
    _lib.LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "paged_kv_attention_26_amd",
                                 "libpa_trace.so")
    _lib._lib = None
    lib = _lib.lib()
    lib.pa_decode_trace_next.restype = C.c_int
    lib.pa_decode_trace_next.argtypes = [C.c_void_p]
    import workloads as W
    from paged_kv_attention_26_amd import binding as pa, runner
    long_ctx = args.decode_trace_workload != "layer"
    part = 512 if long_ctx else args.partition
    layers = []
    if long_ctx:
        g = runner.prepare(W.config3(16 if args.decode_trace_workload == "long16" else 32))
        runner.store_step(g)
        layers.append(g)
    else:
        for li in range(args.layers):
            b = W.config2()
            if li:
                b.free_order = np.random.default_rng(1000 + li).permutation(b.num_blocks)
            layers.append(runner.prepare(b))
    d0 = layers[0].dec
    ws = pa.decode_workspace(len(d0["idx"]), layers[0].batch.num_q_heads, layers[0].batch.head_dim, d0["max_len"],
                             part)
    out = torch.empty_like(d0["q"])
    buf = torch.zeros(4096 * 16, dtype=torch.int32, device="cuda")
    recs = []
    for i in range(args.warmup + args.steps):
        g = layers[i % len(layers)]
        if long_ctx:
            flush_caches()
        else:
            runner.store_step(g)
        buf.zero_()
        _lib.check(lib.pa_decode_trace_next(C.c_void_p(buf.data_ptr())), "pa_decode_trace_next")
        runner.decode_step(g, out=out, partition_tokens=part, workspace=ws)
        torch.cuda.synchronize()
        if i >= args.warmup:
            r = buf.view(-1, 16).cpu().numpy().astype(np.int64)
            recs.append(r[r[:, 0] != 0])
    med = lambda x: float(np.median(x))
    per = []
    for r in recs:
        t0 = r[:, 0].min()
        t = (r[:, :6] - t0) / 100.0                         # us
        ids_req, ids = (r[:, 14] - t0) / 100.0, (r[:, 15] - t0) / 100.0
        arrived = np.where(r[:, 13] != 0, (r[:, 13] - t0) / 100.0, np.nan)
        xcc = r[:, 7] & 15
        merged = r[:, 10] != 0
        end = t[:, 5]
        per.append(dict(
            waves=len(r), kernel_end=end.max(), start_last=t[:, 0].max(), start_med=med(t[:, 0]),
            prefix_med=med(t[:, 1]), ids_req_med=med(ids_req), ids_med=med(ids), ids_max=ids.max(),
            issue_med=med(t[:, 2]), issue_max=t[:, 2].max(), step1_med=med(t[:, 3]),
            range_end_med=med(t[:, 4]), range_end_max=t[:, 4].max(), end_med=med(end),
            step_us_med=med((t[:, 4] - t[:, 3]) / np.maximum(r[:, 9] - 1, 1)),
            merged_frac=float(merged.mean()), end_med_merging=med(end[merged]) if merged.any() else float("nan"),
            count_in_us_med=float(np.nanmedian(arrived - t[:, 4])),
            merge_us_med=float(np.nanmedian((end - arrived)[merged])) if merged.any() else float("nan"),
            end_med_not_merging=med(end[~merged]),
            two_seg_frac=float((r[:, 8] >= 2).mean()),
            xcd_range_end_med=[med(t[xcc == x, 4]) if (xcc == x).any() else float("nan") for x in range(8)],
            xcd_is_block_mod_8=bool(np.all(xcc == (r[:, 6] & 7))),
            steps=(int(r[:, 9].min()), med(r[:, 9]), int(r[:, 9].max()))))
    if args.decode_trace_out:
        n = max(len(r) for r in recs)
        raw = np.zeros((len(recs), n, 16), np.uint32)
        for i, r in enumerate(recs):
            raw[i, :len(r)] = r
        np.save(args.decode_trace_out, raw)
    keys = [k for k in per[0] if k not in ("xcd_range_end_med", "steps", "waves", "xcd_is_block_mod_8")]
    summ = {k: round(med([p[k] for p in per]), 2) for k in keys}
    summ["xcd_range_end_med"] = [round(med([p["xcd_range_end_med"][x] for p in per]), 1) for x in range(8)]
    summ["waves"] = per[0]["waves"]
    summ["steps_min_med_max"] = per[0]["steps"]
    summ["xcd_is_block_mod_8"] = all(p["xcd_is_block_mod_8"] for p in per)
    summ["kernel_end_per_launch"] = [round(p["kernel_end"], 1) for p in per]
    return {"decode_trace": summ, "launches": len(per), "workload": args.decode_trace_workload}


def extras(pa, runner, W, torch, groups=EXTRA_GROUPS):
    """Secondary measurements: long-context decode at block 16 and 32 with
    the bulk store and a bulk block copy ("long_context"), the mixed chunked-prefill batch's store,
    decode and prefill ("mixed"), the fp8 fork decode ("fork"), speculative
    verification of 4 draft tokens on the Qwen3-8B layer ("verify")."""
    out = {}
    for B in ((16, 32) if "long_context" in groups else ()):
        b = W.config3(B)
        g = runner.prepare(b)
        runner.store_step(g)
        # the workload's own split: partitions of 512 tokens
        ws = pa.decode_workspace(len(g.dec["idx"]), b.num_q_heads, b.head_dim, g.dec["max_len"], 512)
        med, p10, p90 = timed_calls(lambda: runner.decode_step(g, partition_tokens=512, workspace=ws))
        byt = kv_bytes(g.dec["host_lens"], b.num_kv_heads, b.head_dim, 2)
        out[f"long_context_decode_b{B}"] = dict(GBps=round(byt / med / 1e6, 1), ms=round(med, 4),
                                                p10_ms=round(p10, 4), p90_ms=round(p90, 4),
                                                frac=round(byt / med / 1e6 / HBM_PEAK_GBS, 4),
                                                kv_bytes=byt, tokens=int(np.sum(g.dec["host_lens"])))
        if B == 16:
            T = g.prior_slots.numel()
            med, _, _ = timed_calls(lambda: runner.fill_prior(g), 10, warm=2)
            moved = T * b.num_kv_heads * b.head_dim * 2 * (2 + 2) + 4 * T
            out["bulk_store_b16"] = dict(GBps=round(moved / med / 1e6, 1), ms=round(med, 3), tokens=T,
                                         frac=round(moved / med / 1e6 / HBM_PEAK_GBS, 4))
            # bulk copy-on-write: every free block of the pool receives a copy of a used one
            used = sorted({blk for row in g.tables for blk in row})
            free = sorted(set(range(b.num_blocks)) - set(used))
            n = min(len(used), len(free))
            pairs = torch.tensor(np.stack([np.array(used[:n]), np.array(free[:n])], 1), dtype=torch.int32,
                                 device="cuda")
            med, _, _ = timed_calls(lambda: pa.copy_blocks(g.cache, pairs), 20, warm=2)
            moved = n * 2 * 2 * b.num_kv_heads * B * b.head_dim * 2
            out["bulk_copy_b16"] = dict(GBps=round(moved / med / 1e6, 1), ms=round(med, 3), pairs=n,
                                        frac=round(moved / med / 1e6 / HBM_PEAK_GBS, 4))
        del g
        torch.cuda.empty_cache()
    if "mixed" in groups:
        mixed_batch(pa, runner, W, out)
    if "verify" in groups:
        b = W.verify_batch()
        g = runner.prepare(b)
        runner.store_step(g)
        med, p10, p90 = timed_calls(lambda: runner.chunk_step(g))
        tl, ql = g.chunk["host_prefix"] + g.chunk["host_q"], g.chunk["host_q"]
        byt = kv_bytes(tl, b.num_kv_heads, b.head_dim, 2)
        fl = sum(4 * b.head_dim * b.num_q_heads * (int(n) * int(P) + int(n) * (int(n) + 1) // 2)
                 for P, n in zip(g.chunk["host_prefix"], ql))
        out["verify_k4"] = dict(GBps=round(byt / med / 1e6, 1), frac=round(byt / med / 1e6 / HBM_PEAK_GBS, 4),
                                TFLOPs=round(fl / med / 1e9, 1), ms=round(med, 4), p10_ms=round(p10, 4),
                                p90_ms=round(p90, 4), kv_bytes=byt, tokens=int(np.sum(tl)))
        del g
        torch.cuda.empty_cache()
        # the same verification over the long-context prefixes (contexts of
        # 128..32768 tokens: the launch cuts the batch into equal stretches)
        b = W.verify_long_batch()
        g = runner.prepare(b)
        runner.store_step(g)
        med, p10, p90 = timed_calls(lambda: runner.chunk_step(g), 20)
        tl = g.chunk["host_prefix"] + g.chunk["host_q"]
        byt = kv_bytes(tl, b.num_kv_heads, b.head_dim, 2)
        out["verify_long_context_k4"] = dict(GBps=round(byt / med / 1e6, 1), frac=round(byt / med / 1e6 / HBM_PEAK_GBS, 4),
                                             ms=round(med, 4), p10_ms=round(p10, 4), p90_ms=round(p90, 4),
                                             kv_bytes=byt, tokens=int(np.sum(tl)))
        del g
        torch.cuda.empty_cache()
    if "handoff" in groups:
        # prefill -> decode KV hand-off of the Qwen3-8B layer's 32 sequences:
        # pack out of the paged pools, store into another cache's own blocks
        b = W.config2()
        g = runner.prepare(b)
        runner.store_step(g)
        rows = int(np.sum(b.total_lens))
        k = torch.empty((rows, b.num_kv_heads, b.head_dim), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        pargs = runner.pack_args(g)                          # uploaded once: the timed call is pa_pack_kv alone
        med_p, _, _ = timed_calls(lambda: runner.pack_all(g, k_out=k, v_out=v, args=pargs))
        d = copy.copy(b)
        d.free_order = np.random.default_rng(2002).permutation(b.num_blocks)
        gd = runner.prepare(d, fill=False)
        slots = runner.all_slots(gd)
        med_u, _, _ = timed_calls(lambda: pa.store_kv(gd.cache, k, v, slots))
        byt = kv_bytes(b.total_lens, b.num_kv_heads, b.head_dim, 2)
        out["handoff_pack"] = dict(GBps=round(2 * byt / med_p / 1e6, 1), frac=round(2 * byt / med_p / 1e6 / HBM_PEAK_GBS, 4),
                                   ms=round(med_p, 4), kv_bytes=byt)
        out["handoff_unpack_store"] = dict(GBps=round((2 * byt + 4 * rows) / med_u / 1e6, 1),
                                           frac=round((2 * byt + 4 * rows) / med_u / 1e6 / HBM_PEAK_GBS, 4),
                                           ms=round(med_u, 4))
        del g, gd
    if "hbm_probe" in groups:
        out["hbm_probe"] = hbm_probe(torch)
    if "fork" in groups:
        fb = W.config5()
        gf = runner.run_fork(fb)
        # block tables, lengths and queries uploaded once: the timed call is pa_decode alone
        lens = [gf.bm.seq_len(x) for x in gf.beams]
        table = torch.from_numpy(gf.bm.block_tables(gf.beams, gf.pad)).cuda()
        lens_t = torch.tensor(lens, dtype=torch.int32, device="cuda")
        q = torch.from_numpy(np.ascontiguousarray(fb.q).view(np.int16)).view(torch.bfloat16).cuda()
        fout = torch.empty_like(q)
        ws = pa.decode_workspace(len(lens), fb.num_q_heads, fb.head_dim, max(lens), 0)
        med, _, _ = timed_calls(lambda: pa.decode(gf.cache, q, table, lens_t, max(lens), fb.scale, out=fout,
                                                  workspace=ws), flush=False)
        byt = kv_bytes(lens, fb.num_kv_heads, fb.head_dim, 1)
        out["fork_fp8_decode"] = dict(GBps_logical=round(byt / med / 1e6, 1), ms=round(med, 4),
                                      note="cache resident: 8 beams share the prompt blocks")
    return out


def mixed_batch(pa, runner, W, out):
    """Mixed chunked-prefill batch: the step's store, the decode of its 64
    sequences and the prefill of its 8 chunks of 512."""
    b = W.config4()
    g = runner.prepare(b)
    med, _, _ = timed_calls(lambda: runner.store_step(g))
    T = g.step_slots.numel()
    out["mixed_store"] = dict(GBps=round(T * b.num_kv_heads * b.head_dim * 8 / med / 1e6, 1), ms=round(med, 4))
    runner.store_step(g)
    ws = pa.decode_workspace(len(g.dec["idx"]), b.num_q_heads, b.head_dim, g.dec["max_len"], 0)
    med, p10, p90 = timed_calls(lambda: runner.decode_step(g, workspace=ws))
    byt = kv_bytes(g.dec["host_lens"], b.num_kv_heads, b.head_dim, 2)
    out["mixed_decode"] = dict(GBps=round(byt / med / 1e6, 1), ms=round(med, 4), p10_ms=round(p10, 4),
                               p90_ms=round(p90, 4), frac=round(byt / med / 1e6 / HBM_PEAK_GBS, 4))
    med, p10, p90 = timed_calls(lambda: runner.chunk_step(g))
    fl = 0
    for P, n in zip(g.chunk["host_prefix"], g.chunk["host_q"]):
        fl += 4 * b.head_dim * b.num_q_heads * (int(n) * int(P) + int(n) * (int(n) + 1) // 2)
    out["mixed_prefill_chunk"] = dict(TFLOPs=round(fl / med / 1e9, 1), ms=round(med, 4), p10_ms=round(p10, 4),
                                      p90_ms=round(p90, 4),
                                      frac=round(fl / med / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4), flops=fl)

    # The whole step: store the 4096 chunk rows and 64 decode tokens, then the
    # two attention calls, one after the other on one stream ...
    def step_one_stream():
        runner.store_step(g)
        runner.chunk_step(g)
        runner.decode_step(g, workspace=ws)
    med, _, _ = timed_calls(step_one_stream)
    out["mixed_step"] = dict(ms=round(med, 4), note="store + prefill + decode, one stream")
    # ... and with the decode on a second stream (default priority), which
    # waits for the store and runs beside the prefill.
    import torch
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()

    def step_two_streams():
        runner.store_step(g)
        side.wait_stream(main)
        runner.chunk_step(g)
        with torch.cuda.stream(side):
            runner.decode_step(g, workspace=ws)
        main.wait_stream(side)
    med, _, _ = timed_calls(step_two_streams)
    out["mixed_step_two_streams"] = dict(ms=round(med, 4), note="decode on a second stream beside the prefill")
    del g
    # the same chunks over an fp8 e4m3 cache (per-head scales; bf16 matrix cores)
    b8 = W.config4(kv_dtype="fp8")
    g8 = runner.prepare(b8)
    runner.store_step(g8)
    med, p10, p90 = timed_calls(lambda: runner.chunk_step(g8))
    out["mixed_prefill_chunk_fp8"] = dict(TFLOPs=round(fl / med / 1e9, 1), ms=round(med, 4), p10_ms=round(p10, 4),
                                          p90_ms=round(p90, 4),
                                          frac=round(fl / med / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4))


# ---------------------------------------------------------------- oracle on the host
# Oracle workloads timed on the host: name -> (unit of the rate, what a unit of
# work is).  Each worker process builds the workload's oracle state itself
# (outside the timed window), then runs its share of the units round-robin
# for the time budget.
CPU_WORKLOADS = {
    "decode_qwen3_8b_layer": "GB/s",      # the 32 sequences of the Qwen3-8B decode layer
    "decode_long_context": "GB/s",        # 24 sequences with the long-context lengths
    "prefill_mixed_chunks": "TFLOP/s",    # the mixed batch's 8 chunks of 512
    "store_bulk": "GB/s",                 # 16384 bf16 rows stored 512 at a time
}


def _cpu_state(name):
    """(list of units, amount of work per unit, function running one unit)."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import workloads as W
    from oracle import paged
    from tests import oracle_setup as OS
    if name in ("decode_qwen3_8b_layer", "decode_long_context"):
        b = W.config2() if name == "decode_qwen3_8b_layer" else W.config3_sample()
        st = OS.build(b)
        tables = OS.table_array(st.tables, st.pad_block)
        lens = b.total_lens

        def run(i):
            paged.decode_attention(st.kc, st.vc, "bf16", b.q_decode[i:i + 1], "bf16", tables[i:i + 1],
                                   lens[i:i + 1], b.scale)
        return list(range(len(lens))), [kv_bytes(lens[i:i + 1], b.num_kv_heads, b.head_dim, 2)
                                        for i in range(len(lens))], run
    if name == "prefill_mixed_chunks":
        b = W.config4()
        st = OS.build(b)
        ch = np.flatnonzero(b.is_chunk)
        cu = np.concatenate([[0], np.cumsum(b.new_lens[ch])])

        def run(j):
            i = ch[j]
            paged.prefill_chunk_attention(st.kc, st.vc, "bf16", b.q_chunk[cu[j]:cu[j + 1]], "bf16",
                                          [0, int(b.new_lens[i])], [int(b.total_lens[i])],
                                          OS.table_array([st.tables[i]], st.pad_block), b.scale)
        fl = [4 * b.head_dim * b.num_q_heads * (int(b.new_lens[i]) * int(b.prior_lens[i]) +
                                                int(b.new_lens[i]) * (int(b.new_lens[i]) + 1) // 2) / 1e3
              for i in ch]                                  # in kFLOP: rates come out in TFLOP/s via /1e9
        return list(range(len(ch))), fl, run
    if name == "store_bulk":
        b = W.store_sample()
        _, _, _, step, _ = OS.allocate(b)
        slots = np.concatenate(step).astype(np.int64)
        k, v = OS.rows_of(b, "step")
        kc, vc = paged.new_pools(b.num_blocks, b.num_kv_heads, b.block_size, b.head_dim, "bf16")
        n = 512

        def run(j):
            sl = slice(j * n, (j + 1) * n)
            paged.store_kv(kc, vc, "bf16", k[sl], v[sl], "bf16", slots[sl])
        units = list(range(len(slots) // n))
        return units, [n * b.num_kv_heads * b.head_dim * 2 * (2 + 2) + 4 * n] * len(units), run
    raise ValueError(name)


def _cpu_worker(rank, nproc, cpu, names, budget, barrier, results):
    """One pinned process: per workload, build the oracle state, wait for the
    other workers, then run units rank, rank + nproc, ... for budget seconds."""
    os.sched_setaffinity(0, {cpu})
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except ImportError:
        pass
    for name in names:
        units, amount, run = _cpu_state(name)
        mine = units[rank::nproc] or units[:1]
        barrier.wait(timeout=900)
        done, work, k = 0, 0.0, 0
        t0 = time.perf_counter()
        while True:
            u = mine[k % len(mine)]
            run(u)
            work += amount[u]
            done += 1
            k += 1
            if time.perf_counter() - t0 >= budget:
                break
        results.put((name, rank, work, time.perf_counter() - t0, done))
        del units, amount, run


def _cpu_mode(nproc, budget):
    """Run every CPU workload on nproc processes pinned to distinct CPUs
    (one BLAS thread each).  Returns {name: (rate, units done, seconds)}."""
    import multiprocessing as mp
    cpus = sorted(os.sched_getaffinity(0))[:nproc]
    env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in env:                      # read by numpy's BLAS when a spawned child imports it
        os.environ[k] = "1"
    ctx = mp.get_context("spawn")
    barrier, results = ctx.Barrier(len(cpus)), ctx.Queue()
    names = list(CPU_WORKLOADS)
    procs = [ctx.Process(target=_cpu_worker, args=(r, len(cpus), c, names, budget, barrier, results))
             for r, c in enumerate(cpus)]
    try:
        for p in procs:
            p.start()
        got = [results.get(timeout=1800) for _ in range(len(names) * len(cpus))]
        for p in procs:
            p.join(timeout=60)
    finally:
        for k, v in env.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
        for p in procs:
            if p.is_alive():
                p.terminate()
    out = {}
    for name in names:
        rows = [g for g in got if g[0] == name]
        secs = max(g[3] for g in rows)
        out[name] = (sum(g[2] for g in rows) / secs / 1e9, sum(g[4] for g in rows), secs)
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(budget_s=2.5, max_procs=16):
    """The oracle (plain fp64 numpy, as it stands) timed on the host in two
    modes: one process pinned to one CPU, and one pinned process per CPU of
    this process's affinity set (at most max_procs) sharing the units of each
    workload.  The headline is the all-core rate on the Qwen3-8B decode
    layer (the bench's own workload)."""
    n_all = min(len(os.sched_getaffinity(0)), max_procs)
    t0 = time.perf_counter()
    one = _cpu_mode(1, budget_s)
    every = _cpu_mode(n_all, budget_s)
    wall = time.perf_counter() - t0

    def fmt(mode, n):
        return {k: dict(value=round(r, 4), unit=CPU_WORKLOADS[k], units=u, seconds=round(sec, 2), processes=n)
                for k, (r, u, sec) in mode.items()}
    head = every["decode_qwen3_8b_layer"]
    return dict(value=round(head[0], 4), unit="GB/s", cores=n_all, kind="oracle",
                sample=f"fp64 numpy oracle decode of the Qwen3-8B layer's 32 sequences, {n_all} pinned processes "
                       f"sharing them round-robin for {budget_s} s ({head[1]} sequence decodes)",
                cpu_model=cpu_model(), single_core=fmt(one, 1), all_cores=fmt(every, n_all),
                wall_s=round(wall, 1))


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library runs on a single MI355X and has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        # A plain device-to-device copy of known size: each launch reads and
        # writes exactly MIB MiB, the yardstick for FETCH_SIZE / WRITE_SIZE.
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_per_launch": n, "launches": 4}), flush=True)
        return
    if args.hbm_probe:
        print(json.dumps({"hbm_probe": hbm_probe(torch)}), flush=True)
        return
    if args.decode_trace:
        print(json.dumps(decode_trace(args, torch)), flush=True)
        return
    import workloads as W
    from paged_kv_attention_26_amd import binding as pa, runner
    if args.only_extra:
        print(json.dumps({"extras": extras(pa, runner, W, torch, (args.only_extra,))}), flush=True)
        return

    base = W.config2()
    lens_all = base.total_lens
    layers = []
    for li in range(args.layers):
        b = W.config2()
        if li:
            b.free_order = np.random.default_rng(1000 + li).permutation(b.num_blocks)
        g = runner.prepare(b)
        layers.append(g)
    d0 = layers[0].dec
    ws = pa.decode_workspace(len(d0["idx"]), base.num_q_heads, base.head_dim, d0["max_len"], args.partition)
    out = torch.empty_like(d0["q"])
    step_bytes = kv_bytes(lens_all, base.num_kv_heads, base.head_dim, 2)
    fused = not args.separate_store
    # the decode launch's own algorithmic bytes: the KV it reads, and when it
    # also stores the step's tokens, their rows read once and written once
    new_rows = len(lens_all) * base.num_kv_heads * base.head_dim * 2 * 2
    launch_bytes = step_bytes + (2 * new_rows if fused else 0)

    def step(i, stamp=None):
        g = layers[i % len(layers)]
        if not fused:
            runner.store_step(g)
        if stamp is not None:
            pa.time_next_decode(*stamp)
        if fused:
            return runner.decode_step_append(g, out=out, partition_tokens=args.partition, workspace=ws)
        return runner.decode_step(g, out=out, partition_tokens=args.partition, workspace=ws)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Every stamp_every-th decode launch of the timed region stamps a pair of
    # events with the kernel's own start and end (pa_decode_time_next), so the
    # timed stream carries no marker packets; the events are created by one
    # record() each beforehand.  A stamped launch costs the step a few
    # microseconds, which is why not every launch carries them.
    every = max(1, args.stamp_every)
    stamped = [i for i in range(args.steps) if i % every == every - 1] or [args.steps - 1]
    evs = {i: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for i in stamped}
    for e0, e1 in evs.values():
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, evs.get(i))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs.values()])
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg = float(dec_ms.mean())
    achieved = launch_bytes / (dec_avg * 1e-3) / 1e9
    rec = {
        "metric": "paged decode KV GB/s (% HBM peak) + prefill-chunk TFLOP/s, Qwen3-8B layer",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3-8b decode layer: 32 seqs, ctx U[512,4096], Hq 32 / Hkv 8, d 128, "
                               "bf16 KV, block 16, 32 new tokens stored + paged decode"
                               + (" in one launch" if fused else " (separate store launch)"),
                   "global_batch": int(len(lens_all)), "seq_len": int(np.max(lens_all)),
                   "kv_tokens": int(np.sum(lens_all)), "layer_caches": args.layers,
                   "partition_tokens": args.partition, "parallelism": "single-gpu"},
        "device": device_info(torch),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": decode_traffic() if fused else None,
                     "kernel": "pa::decode_kernel<bf16, d128, B16, G4>",
                     "kernel_ms_avg": round(dec_avg, 5), "kernel_ms_median": round(float(np.median(dec_ms)), 5),
                     "kernel_ms_p10": round(float(np.percentile(dec_ms, 10)), 5),
                     "kernel_ms_p90": round(float(np.percentile(dec_ms, 90)), 5),
                     "kernel_launches_timed": int(len(dec_ms)),
                     "algorithmic_bytes_per_launch": launch_bytes},
    }
    if not args.no_extras:
        del layers
        torch.cuda.empty_cache()
        rec["extras"] = extras(pa, runner, W, torch)
    if not args.no_cpu:
        rec["cpu_baseline"] = cpu_baseline()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
