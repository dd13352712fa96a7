"""Benchmark of the paged-attention hot path on one MI355X.

A step is one pass of the path over one batch: pa_store_kv of the step's new
tokens, then the attention call(s).  The default workload is one Qwen3-8B
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


# HBM bytes per decode_kernel launch on this workload, from rocprofv3 FETCH_SIZE
# and WRITE_SIZE passes scaled by the same counters on a plain 1 GiB copy
# (bench.py --copy-probe 1024), and the hash of the kernel sources they were
# taken on: once those sources change the figure no longer applies.
DECODE_TRAFFIC = {"sources_sha256": "f862b40bf4b8b2a618349774811e6b8e2063a9ca36a134ad03b764a35402194d",
                  "bytes_per_launch": 305715764}
DECODE_SOURCES = ("decode_kernel.h", "pa_device.h", "pa_internal.h", "decode_bf16.hip")


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
    ap.add_argument("--partition", type=int, default=0, help="split-K partition tokens (0 = library default)")
    ap.add_argument("--stamp-every", type=int, default=4,
                    help="time every N-th decode launch of the timed region with kernel-stamped events")
    ap.add_argument("--no-extras", action="store_true", help="skip the secondary measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--only-extra", choices=EXTRA_GROUPS, default=None,
                    help="run only this group of secondary measurements and print them (for profiling)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 4 times (calibrates HBM byte counters)")
    return ap.parse_args()


def timed_calls(fn, reps, warm=3):
    """Median / p10 / p90 ms of fn() measured with events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return float(np.median(t)), float(np.percentile(t, 10)), float(np.percentile(t, 90))


EXTRA_GROUPS = ("long_context", "mixed", "fork", "verify", "handoff")


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
        med, p10, p90 = timed_calls(lambda: runner.decode_step(g, partition_tokens=512, workspace=ws), 20)
        byt = kv_bytes(g.dec["host_lens"], b.num_kv_heads, b.head_dim, 2)
        out[f"long_context_decode_b{B}"] = dict(GBps=round(byt / med / 1e6, 1), ms=round(med, 4),
                                                p10_ms=round(p10, 4), p90_ms=round(p90, 4),
                                                frac=round(byt / med / 1e6 / HBM_PEAK_GBS, 4),
                                                kv_bytes=byt, tokens=int(np.sum(g.dec["host_lens"])))
        if B == 16:
            T = g.prior_slots.numel()
            med, _, _ = timed_calls(lambda: runner.fill_prior(g), 5, warm=1)
            moved = T * b.num_kv_heads * b.head_dim * 2 * (2 + 2) + 4 * T
            out["bulk_store_b16"] = dict(GBps=round(moved / med / 1e6, 1), ms=round(med, 3), tokens=T,
                                         frac=round(moved / med / 1e6 / HBM_PEAK_GBS, 4))
            # bulk copy-on-write: every free block of the pool receives a copy of a used one
            used = sorted({blk for row in g.tables for blk in row})
            free = sorted(set(range(b.num_blocks)) - set(used))
            n = min(len(used), len(free))
            pairs = torch.tensor(np.stack([np.array(used[:n]), np.array(free[:n])], 1), dtype=torch.int32,
                                 device="cuda")
            med, _, _ = timed_calls(lambda: pa.copy_blocks(g.cache, pairs), 10, warm=2)
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
        med, p10, p90 = timed_calls(lambda: runner.chunk_step(g), 20)
        tl, ql = g.chunk["host_prefix"] + g.chunk["host_q"], g.chunk["host_q"]
        byt = kv_bytes(tl, b.num_kv_heads, b.head_dim, 2)
        fl = sum(4 * b.head_dim * b.num_q_heads * (int(n) * int(P) + int(n) * (int(n) + 1) // 2)
                 for P, n in zip(g.chunk["host_prefix"], ql))
        out["verify_k4"] = dict(GBps=round(byt / med / 1e6, 1), frac=round(byt / med / 1e6 / HBM_PEAK_GBS, 4),
                                TFLOPs=round(fl / med / 1e9, 1), ms=round(med, 4), p10_ms=round(p10, 4),
                                p90_ms=round(p90, 4), kv_bytes=byt, tokens=int(np.sum(tl)))
        del g
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
        med_p, _, _ = timed_calls(lambda: runner.pack_all(g, k_out=k, v_out=v, args=pargs), 20)
        d = copy.copy(b)
        d.free_order = np.random.default_rng(2002).permutation(b.num_blocks)
        gd = runner.prepare(d, fill=False)
        slots = runner.all_slots(gd)
        med_u, _, _ = timed_calls(lambda: pa.store_kv(gd.cache, k, v, slots), 20)
        byt = kv_bytes(b.total_lens, b.num_kv_heads, b.head_dim, 2)
        out["handoff_pack"] = dict(GBps=round(2 * byt / med_p / 1e6, 1), frac=round(2 * byt / med_p / 1e6 / HBM_PEAK_GBS, 4),
                                   ms=round(med_p, 4), kv_bytes=byt)
        out["handoff_unpack_store"] = dict(GBps=round((2 * byt + 4 * rows) / med_u / 1e6, 1),
                                           frac=round((2 * byt + 4 * rows) / med_u / 1e6 / HBM_PEAK_GBS, 4),
                                           ms=round(med_u, 4))
        del g, gd
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
                                                  workspace=ws), 20)
        byt = kv_bytes(lens, fb.num_kv_heads, fb.head_dim, 1)
        out["fork_fp8_decode"] = dict(GBps_logical=round(byt / med / 1e6, 1), ms=round(med, 4),
                                      note="cache resident: 8 beams share the prompt blocks")
    return out


def mixed_batch(pa, runner, W, out):
    """Mixed chunked-prefill batch: the step's store, the decode of its 64
    sequences and the prefill of its 8 chunks of 512."""
    b = W.config4()
    g = runner.prepare(b)
    med, _, _ = timed_calls(lambda: runner.store_step(g), 20)
    T = g.step_slots.numel()
    out["mixed_store"] = dict(GBps=round(T * b.num_kv_heads * b.head_dim * 8 / med / 1e6, 1), ms=round(med, 4))
    runner.store_step(g)
    ws = pa.decode_workspace(len(g.dec["idx"]), b.num_q_heads, b.head_dim, g.dec["max_len"], 0)
    med, _, _ = timed_calls(lambda: runner.decode_step(g, workspace=ws), 20)
    byt = kv_bytes(g.dec["host_lens"], b.num_kv_heads, b.head_dim, 2)
    out["mixed_decode"] = dict(GBps=round(byt / med / 1e6, 1), ms=round(med, 4))
    med, _, _ = timed_calls(lambda: runner.chunk_step(g), 20)
    fl = 0
    for P, n in zip(g.chunk["host_prefix"], g.chunk["host_q"]):
        fl += 4 * b.head_dim * b.num_q_heads * (int(n) * int(P) + int(n) * (int(n) + 1) // 2)
    out["mixed_prefill_chunk"] = dict(TFLOPs=round(fl / med / 1e9, 1), ms=round(med, 4),
                                      frac=round(fl / med / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4), flops=fl)

    # The whole step: store the 4096 chunk rows and 64 decode tokens, then the
    # two attention calls, one after the other on one stream ...
    def step_one_stream():
        runner.store_step(g)
        runner.chunk_step(g)
        runner.decode_step(g, workspace=ws)
    med, _, _ = timed_calls(step_one_stream, 20)
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
    med, _, _ = timed_calls(step_two_streams, 20)
    out["mixed_step_two_streams"] = dict(ms=round(med, 4), note="decode on a second stream beside the prefill")
    del g
    # the same chunks over an fp8 e4m3 cache (per-head scales; bf16 matrix cores)
    b8 = W.config4(kv_dtype="fp8")
    g8 = runner.prepare(b8)
    runner.store_step(g8)
    med, _, _ = timed_calls(lambda: runner.chunk_step(g8), 20)
    out["mixed_prefill_chunk_fp8"] = dict(TFLOPs=round(fl / med / 1e9, 1), ms=round(med, 4),
                                          frac=round(fl / med / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4))


def cpu_baseline(batch, budget_s=10.0):
    """The oracle (plain fp64 numpy) on a bounded sample of the workload: it
    decodes the batch's sequences one by one, pass after pass, for about
    budget_s seconds, and reports the KV bytes attended per second.  Measured
    twice: with every BLAS thread the host gives it, and on one thread.
    Returns (all threads, one thread)."""
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle import paged
    from tests import oracle_setup as OS
    st = OS.build(batch)
    dec = np.flatnonzero(~batch.is_chunk)
    tables = OS.table_array([st.tables[i] for i in dec], st.pad_block)
    lens = batch.total_lens[dec]

    def run():
        seqs, byt, tokens = 0, 0, 0
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < budget_s:
            s = seqs % len(dec)
            paged.decode_attention(st.kc, st.vc, batch.kv_dtype, batch.q_decode[s:s + 1], batch.io_dtype,
                                   tables[s:s + 1], lens[s:s + 1], batch.scale)
            byt += kv_bytes(lens[s:s + 1], batch.num_kv_heads, batch.head_dim, 2)
            tokens += int(lens[s])
            seqs += 1
        dt = time.perf_counter() - t0
        try:                               # threads the oracle's BLAS calls actually run on
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:
            threads = 1
        return dict(value=round(byt / dt / 1e9, 4), unit="GB/s", cores=int(threads), kind="oracle",
                    sample=f"fp64 numpy decode of the {len(dec)} sequences, {seqs / len(dec):.1f} passes "
                           f"({seqs} sequence decodes, {tokens} KV tokens x {batch.num_kv_heads} kv heads) "
                           f"in {dt:.1f} s")

    every = run()
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = run()
    except ImportError:
        one = None
    return every, one


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

    def step(i):
        g = layers[i % len(layers)]
        runner.store_step(g)
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
        g = layers[i % len(layers)]
        runner.store_step(g)
        if i in evs:
            pa.time_next_decode(evs[i][0], evs[i][1])
        runner.decode_step(g, out=out, partition_tokens=args.partition, workspace=ws)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs.values()])
    ms_per_step = wall * 1e3 / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    dec_avg = float(dec_ms.mean())
    achieved = step_bytes / (dec_avg * 1e-3) / 1e9
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
                               "bf16 KV, block 16, store 32 tokens + paged decode",
                   "global_batch": int(len(lens_all)), "seq_len": int(np.max(lens_all)),
                   "kv_tokens": int(np.sum(lens_all)), "layer_caches": args.layers,
                   "partition_tokens": args.partition or 64, "parallelism": "single-gpu"},
        "device": device_info(torch),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": decode_traffic(),
                     "kernel": "pa::decode_kernel<bf16, d128, B16, G4>",
                     "kernel_ms_avg": round(dec_avg, 5), "kernel_ms_median": round(float(np.median(dec_ms)), 5),
                     "kernel_launches_timed": int(len(dec_ms)),
                     "algorithmic_bytes_per_launch": step_bytes},
    }
    if not args.no_extras:
        del layers
        torch.cuda.empty_cache()
        rec["extras"] = extras(pa, runner, W, torch)
    if not args.no_cpu:
        rec["cpu_baseline"], one = cpu_baseline(W.config2())
        if one is not None:
            rec["cpu_baseline_single_thread"] = one
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
