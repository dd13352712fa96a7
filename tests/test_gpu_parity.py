"""GPU parity of libpa against the CPU oracle (needs an MI355X).

Store and copy are compared bit for bit over the whole pool (untouched slots
must keep their NaN poison); attention within max-abs 1e-4 (fp32 cache),
2e-2 (bf16) and 6e-2 (fp8) of the fp64 oracle.  Both sides make the same
allocation decisions (the native block manager equals the oracle's, checked
on the CPU), and every input comes from the seeded generators.
"""
import copy
import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import oracle_setup as OS

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_26_amd import _lib
    _lib.lib()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor, kv: str) -> np.ndarray:
    t = t.detach().cpu()
    if kv == "f32":
        return t.view(torch.int32).numpy().view(np.uint32)
    if kv == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def oracle_bits(a: np.ndarray, kv: str) -> np.ndarray:
    return a.view(np.uint32) if kv == "f32" else a


def out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def edge_batch(kv="bf16", B=16):
    rng = np.random.default_rng(77)
    lens = np.array([1, 2, 15, 16, 17, 63, 64, 65, 511, 512, 513, 1024, 1025, 0, 129, 4100])
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    io = "f32" if kv == "f32" else "bf16"
    Hq, Hkv, d = (8, 2, 64) if kv == "f32" else (32, 8, 128)
    return W.paged_batch(f"edge-{kv}-b{B}", 77, kv_dtype=kv, io_dtype=io, Hq=Hq, Hkv=Hkv, d=d, B=B,
                         prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)


def skew_batch():
    """One long sequence beside empty and one-token ones: far fewer work units
    than the host's upper bound, so the launch has more waves than units."""
    rng = np.random.default_rng(78)
    lens = np.array([6000] + [0] * 8 + [1] * 7)
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    return W.paged_batch("skew-bf16", 78, kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                         prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)


def many_batch():
    """600 short sequences (0 to 200 tokens): more sequences than threads in a
    workgroup, so the per-sequence prefixes built in LDS take several
    sequences per thread."""
    rng = np.random.default_rng(79)
    lens = rng.integers(0, 201, 600)
    lens[::97] = 0
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    return W.paged_batch("many-bf16", 79, kv_dtype="bf16", io_dtype="bf16", Hq=8, Hkv=2, d=128, B=16,
                         prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)


def max_seqs_batch():
    """8192 sequences, the most one call takes (the decode kernel's prefix
    over sequences lives in LDS), of 0 to 40 tokens."""
    rng = np.random.default_rng(80)
    lens = rng.integers(0, 41, 8192)
    lens[::61] = 0
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    return W.paged_batch("maxseq-bf16", 80, kv_dtype="bf16", io_dtype="bf16", Hq=8, Hkv=2, d=64, B=16,
                         prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)


SMALL = {
    "c1": lambda: W.config1(),
    "c2s": lambda: W.config2(small=True),
    "c3s16": lambda: W.config3(16, small=True),
    "c3s32": lambda: W.config3(32, small=True),
    "edge16": lambda: edge_batch("bf16", 16),
    "edge32": lambda: edge_batch("bf16", 32),
    "edge-f32": lambda: edge_batch("f32", 16),
    "skew": skew_batch,
    "many": many_batch,
}


@pytest.mark.parametrize("name", list(SMALL))
def test_store_is_bit_exact_over_the_whole_pool(name):
    from paged_kv_attention_26_amd import runner
    say(f"[gpu] store {name}")
    batch = SMALL[name]()
    g = runner.prepare(batch)
    runner.store_step(g)
    torch.cuda.synchronize()
    st = OS.build(batch)
    assert g.tables == st.tables
    assert np.array_equal(bits(g.cache.k_cache, batch.kv_dtype), oracle_bits(st.kc, batch.kv_dtype))
    assert np.array_equal(bits(g.cache.v_cache, batch.kv_dtype), oracle_bits(st.vc, batch.kv_dtype))


def slot_pattern(rng, num_blocks, B, T):
    """T distinct slots (or -1) mixing whole blocks, runs that start at odd
    offsets and cross block ends, short aligned runs, skipped tokens inside
    runs and lone tokens, over a random block order."""
    blocks = list(rng.permutation(num_blocks))
    out = []
    while len(out) < T and len(blocks) >= 2:
        kind = int(rng.integers(0, 5))
        b0, b1 = int(blocks.pop()), int(blocks.pop())
        if kind == 0:                                       # two whole blocks, in order
            run = list(range(b0 * B, b0 * B + B)) + list(range(b1 * B, b1 * B + B))
        elif kind == 1:                                     # odd start, crossing into the next block
            o = int(rng.integers(1, B))
            run = list(range(b0 * B + o, b0 * B + B)) + list(range(b1 * B, b1 * B + int(rng.integers(1, B))))
        elif kind == 2:                                     # aligned but short runs
            run = list(range(b0 * B, b0 * B + int(rng.integers(1, 8)))) + list(range(b1 * B + 8, b1 * B + 13))
        elif kind == 3:                                     # a whole block with skipped tokens
            run = [sl if rng.random() > 0.2 else -1 for sl in range(b0 * B, b0 * B + B)]
        else:                                               # lone tokens at random offsets
            run = [b0 * B + int(rng.integers(0, B)), b1 * B + int(rng.integers(0, B)), -1]
        out.extend(run)
    return np.asarray(out[:T], dtype=np.int32)


@pytest.mark.parametrize("T", [700, 1, 37, 128, 129])
@pytest.mark.parametrize("kv,B,D", [("bf16", 16, 128), ("bf16", 32, 64), ("f32", 16, 64), ("f32", 32, 128),
                                    ("fp8", 16, 128), ("fp8", 32, 128), ("fp8raw", 16, 128), ("fp8raw", 32, 64)])
def test_store_slot_patterns_bit_exact(kv, B, D, T):
    """pa_store_kv with arbitrary slot patterns (whole and partial blocks,
    misaligned and skipped tokens) against the oracle's scatter, bit for bit
    over the whole poisoned pool.  Batches of at most 128 tokens take the
    one-wave-per-row store, larger ones the 64-token tiles; fp8raw stores
    e4m3 codes as they are."""
    from oracle import paged
    from paged_kv_attention_26_amd import binding as pa
    rng = np.random.default_rng(4242 + B + D + T)
    NB, H = 96, 2
    slots = slot_pattern(rng, NB, B, T)
    T = len(slots)
    say(f"[gpu] store slot patterns {kv} B{B} d{D}: {T} tokens, {int((slots < 0).sum())} skipped")
    x = rng.standard_normal((2, T, H, D)).astype(np.float32)
    scale = (rng.random(H).astype(np.float32) * 0.5 + 0.25) if kv == "fp8" else None
    if kv == "fp8raw":
        kin, vin = (rng.integers(0, 256, (2, T, H, D)).astype(np.uint8))
        scale = np.ones(H, np.float32)                    # the cache's scales; a raw store ignores them
        kt = torch.from_numpy(kin).cuda()
        vt = torch.from_numpy(vin).cuda()
        kv = in_dt = "fp8"
    elif kv == "f32":
        kin, vin = x[0], x[1]
        kt, vt = torch.from_numpy(kin).cuda(), torch.from_numpy(vin).cuda()
        in_dt = "f32"
    else:
        kin, vin = W.to_bf16_bits(x[0]), W.to_bf16_bits(x[1])
        kt = torch.from_numpy(kin.view(np.int16)).view(torch.bfloat16).cuda()
        vt = torch.from_numpy(vin.view(np.int16)).view(torch.bfloat16).cuda()
        in_dt = "bf16"
    cache = pa.alloc_cache(NB, H, B, D, kv, k_scale=scale, v_scale=scale)
    pa.store_kv(cache, kt, vt, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    kc, vc = paged.new_pools(NB, H, B, D, kv)
    paged.store_kv(kc, vc, kv, kin, vin, in_dt, slots, k_scale=scale, v_scale=scale)
    assert np.array_equal(bits(cache.k_cache, kv), oracle_bits(kc, kv))
    assert np.array_equal(bits(cache.v_cache, kv), oracle_bits(vc, kv))


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("part", [0, 64, 128, 512, "B", "3B"])
def test_decode_matches_oracle(name, part):
    """Decode against the oracle at partitions of 64, 128 and 512 tokens,
    one and three blocks (steps of 64 tokens then span several partitions,
    and a wave's range can start inside a step) and 0 (no split)."""
    from paged_kv_attention_26_amd import runner
    batch = SMALL[name]()
    if isinstance(part, str):
        part = batch.block_size * (3 if part == "3B" else 1)
    say(f"[gpu] decode {name} partition {part}")
    g = runner.prepare(batch)
    runner.store_step(g)
    out = runner.decode_step(g, partition_tokens=part)
    torch.cuda.synchronize()
    ref = OS.decode_ref(batch, OS.build(batch))
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref))
    say(f"      max abs err {err:.3e}")
    assert err < TOL[batch.kv_dtype]


@pytest.mark.parametrize("part", [64, 1024, 0])
def test_decode_at_the_sequence_limit(part):
    """The largest batch one call takes (8192 sequences), at the default
    partition, at 64 blocks of 16 and with no split: store bit-exact over the
    whole pool, every output against the oracle, and the pack of every
    sequence bit-exact."""
    from oracle import paged
    from paged_kv_attention_26_amd import runner
    say(f"[gpu] decode at the sequence limit, partition {part}")
    batch = max_seqs_batch()
    g = runner.prepare(batch)
    runner.store_step(g)
    got = out_f64(runner.decode_step(g, partition_tokens=part))
    k, v = runner.pack_all(g)
    torch.cuda.synchronize()
    st = OS.build(batch)
    assert np.array_equal(bits(g.cache.k_cache, "bf16"), oracle_bits(st.kc, "bf16"))
    assert np.array_equal(bits(g.cache.v_cache, "bf16"), oracle_bits(st.vc, "bf16"))
    err = np.max(np.abs(got - OS.decode_ref(batch, st)))
    say(f"      max abs err {err:.3e}")
    assert err < TOL["bf16"]
    kr, vr = paged.pack_kv(st.kc, st.vc, st.tables, batch.total_lens)
    assert np.array_equal(bits(k, "bf16"), oracle_bits(kr, "bf16")) and np.array_equal(bits(v, "bf16"), oracle_bits(vr, "bf16"))


@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_f32_head_dim_128(G, B):
    """An fp32 cache at head_dim 128 (32-token steps from four heads per
    group up): ragged lengths across several steps and partitions, against
    the oracle within the fp32 tolerance, at the default partition and at
    128-token partitions."""
    from paged_kv_attention_26_amd import runner
    rng = np.random.default_rng(600 + 10 * G + B)
    lens = np.concatenate([[0, 1, 31, 32, 33, 64, 65, 700], rng.integers(1, 900, 9)])
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    batch = W.paged_batch(f"f32-d128-g{G}-b{B}", 600 + G, kv_dtype="f32", io_dtype="f32", Hq=2 * G, Hkv=2, d=128,
                          B=B, prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)
    say(f"[gpu] decode f32 d128 G{G} B{B}")
    g = runner.prepare(batch)
    runner.store_step(g)
    st = OS.build(batch)
    ref = OS.decode_ref(batch, st)
    for part in (0, 128):
        got = out_f64(runner.decode_step(g, partition_tokens=part))
        torch.cuda.synchronize()
        err = np.max(np.abs(got - ref))
        say(f"      partition {part}: max abs err {err:.3e}")
        assert err < TOL["f32"]


@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_decode_fp8_head_dim_64(G, B):
    """An fp8 cache at head_dim 64 (up to four waves per SIMD, so launches
    of up to 4096 waves): ragged lengths, per-head scales, against the oracle
    at the default and at 128-token partitions."""
    from paged_kv_attention_26_amd import runner
    rng = np.random.default_rng(700 + 10 * G + B)
    lens = np.concatenate([[0, 1, 63, 64, 65, 1100], rng.integers(1, 1500, 10)])
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    batch = W.paged_batch(f"fp8-d64-g{G}-b{B}", 700 + G, kv_dtype="fp8", io_dtype="bf16", Hq=4 * G, Hkv=4, d=64,
                          B=B, prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)
    say(f"[gpu] decode fp8 d64 G{G} B{B}")
    g = runner.prepare(batch)
    runner.store_step(g)
    st = OS.build(batch)
    assert np.array_equal(bits(g.cache.k_cache, "fp8"), st.kc) and np.array_equal(bits(g.cache.v_cache, "fp8"), st.vc)
    ref = OS.decode_ref(batch, st)
    for part in (0, 128):
        got = out_f64(runner.decode_step(g, partition_tokens=part))
        torch.cuda.synchronize()
        err = np.max(np.abs(got - ref))
        say(f"      partition {part}: max abs err {err:.3e}")
        assert err < TOL["fp8"]


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_every_compiled_decode_shape(kv, d, B, G):
    """Every (cache dtype, head_dim, block size, group) the decode compiles,
    on a small ragged batch: the store bit-exact over the whole pool, the
    decode against the oracle, the pack bit-exact."""
    from oracle import paged
    from paged_kv_attention_26_amd import runner
    rng = np.random.default_rng(800 + 97 * G + B + d)
    lens = np.concatenate([[0, 1, B - 1, B, B + 1, 200], rng.integers(1, 300, 4)])
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    io = "f32" if kv == "f32" else "bf16"
    batch = W.paged_batch(f"every-{kv}-d{d}-b{B}-g{G}", 800 + G, kv_dtype=kv, io_dtype=io, Hq=2 * G, Hkv=2, d=d,
                          B=B, prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)
    g = runner.prepare(batch)
    runner.store_step(g)
    got = out_f64(runner.decode_step(g))
    k, v = runner.pack_all(g)
    torch.cuda.synchronize()
    st = OS.build(batch)
    assert np.array_equal(bits(g.cache.k_cache, kv), oracle_bits(st.kc, kv))
    assert np.array_equal(bits(g.cache.v_cache, kv), oracle_bits(st.vc, kv))
    assert np.max(np.abs(got - OS.decode_ref(batch, st))) < TOL[kv]
    kr, vr = paged.pack_kv(st.kc, st.vc, st.tables, batch.total_lens)
    assert np.array_equal(bits(k, kv), oracle_bits(kr, kv)) and np.array_equal(bits(v, kv), oracle_bits(vr, kv))


def _append_vs_store_then_decode(batch, partitions=(64,)):
    """pa_decode_append against pa_store_kv followed by pa_decode on a second
    copy of the same cache: outputs and both pools bit for bit."""
    from paged_kv_attention_26_amd import runner
    for part in partitions:
        ga, gb = runner.prepare(batch), runner.prepare(batch)
        runner.store_step(ga)
        want = runner.decode_step(ga, partition_tokens=part)
        got = runner.decode_step_append(gb, partition_tokens=part)
        torch.cuda.synchronize()
        raw = lambda t: t.contiguous().view(torch.uint8)  # bytes: the pools' poison pattern is a NaN
        assert torch.equal(raw(want), raw(got))
        assert torch.equal(raw(ga.cache.k_cache), raw(gb.cache.k_cache))
        assert torch.equal(raw(ga.cache.v_cache), raw(gb.cache.v_cache))
        del ga, gb


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_append_every_compiled_shape(kv, d, B, G):
    """The store-and-decode launch (pa_decode_append) in every (cache dtype,
    head_dim, block size, group) the decode compiles, on a ragged batch with
    empty and one-token sequences, at 64-token partitions and without a
    split: the same outputs and pools, bit for bit, as the store followed by
    the decode."""
    rng = np.random.default_rng(900 + 97 * G + B + d)
    lens = np.concatenate([[0, 1, B - 1, B, B + 1, 200], rng.integers(1, 300, 4)])
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    io = "f32" if kv == "f32" else "bf16"
    batch = W.paged_batch(f"append-{kv}-d{d}-b{B}-g{G}", 900 + G, kv_dtype=kv, io_dtype=io, Hq=2 * G, Hkv=2, d=d,
                          B=B, prior_lens=prior, new_lens=new, is_chunk=np.zeros(len(lens), bool), rng=rng)
    say(f"[gpu] decode append {batch.name}")
    _append_vs_store_then_decode(batch, partitions=(64, 0))


@pytest.mark.parametrize("name", ["edge-fp8-b32", "skew", "many", "max-seqs", "qwen3-8b-layer"])
def test_decode_append_larger_batches(name):
    """pa_decode_append on the edge lengths (fp8, block 32, partitions of 64,
    512 and none), one long sequence among empty ones (64 and none), 600
    sequences (the LDS prefix; 64, 256 and none), 8192 sequences of 0 to 40
    tokens (the most one call takes; 16 and none) and the full Qwen3-8B
    layer as benchmarked: bit for bit the store followed by the decode."""
    batch = {"edge-fp8-b32": lambda: edge_batch("fp8", 32), "skew": skew_batch, "many": many_batch,
             "max-seqs": max_seqs_batch, "qwen3-8b-layer": W.config2}[name]()
    say(f"[gpu] decode append {name}")
    parts = {"edge-fp8-b32": (64, 512, 0), "skew": (64, 0), "many": (64, 256, 0), "max-seqs": (16, 0),
             "qwen3-8b-layer": (64,)}[name]
    _append_vs_store_then_decode(batch, partitions=parts)


@pytest.mark.parametrize("form", ["separate", "fused"])
def test_step_replays_in_a_hip_graph(form):
    """A decode step with a caller-owned workspace captured in a HIP graph,
    in both forms: the store of the step's tokens then pa_decode, or one
    pa_decode_append.  No call allocates or synchronises, so it captures,
    and every replay, with eager work and synchronisation between replays,
    gives the eager result bit for bit."""
    from paged_kv_attention_26_amd import binding as pa, runner
    say(f"[gpu] decode step in a HIP graph ({form})")
    batch = W.config2(small=True)
    g = runner.prepare(batch)
    ws = pa.decode_workspace(1, 1, batch.head_dim, 1, 0)
    out = torch.empty_like(g.dec["q"])

    def step():
        if form == "fused":
            runner.decode_step_append(g, out=out, workspace=ws)
            return
        runner.store_step(g)
        runner.decode_step(g, out=out, workspace=ws)
    step()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):                      # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), rep
        other = runner.decode_step(g, partition_tokens=128)          # eager work between replays
        torch.cuda.synchronize()
        assert int(torch.count_nonzero(ws[:4096 * 4])) == 0
        del other


def test_decode_repeated_calls_reuse_the_workspace():
    """Calls of different shapes and partition sizes, interleaved on one
    workspace, repeat bit-identically, and every call leaves the per-item
    arrival counters (the workspace's first 4096 int32) at zero."""
    from paged_kv_attention_26_amd import binding as pa, runner
    batches = [W.config3(16, small=True), W.config2(small=True), skew_batch()]
    gs = []
    for b in batches:
        g = runner.prepare(b)
        runner.store_step(g)
        gs.append(g)
    ws = pa.decode_workspace(1, 1, 128, 1, 0)
    first = {}
    for rep in range(3):
        for i, g in enumerate(gs):
            for part in (0, 128):
                o = runner.decode_step(g, partition_tokens=part, workspace=ws).clone()
                torch.cuda.synchronize()
                assert int(torch.count_nonzero(ws[:4096 * 4])) == 0, (i, part, rep)
                if (i, part) in first:
                    assert torch.equal(o.view(torch.int16), first[(i, part)].view(torch.int16)), (i, part, rep)
                else:
                    first[(i, part)] = o


def test_decode_timing_hook_stamps_one_kernel():
    """pa_decode_time_next: the armed call gives the same bits as an unarmed
    one and stamps its events with a positive kernel duration; the next,
    unarmed call leaves the events as they were."""
    from paged_kv_attention_26_amd import binding as pa, runner
    say("[gpu] decode timing hook")
    batch = SMALL["c2s"]()
    g = runner.prepare(batch)
    runner.store_step(g)
    ref = runner.decode_step(g).clone()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    e1.record()
    torch.cuda.synchronize()
    pa.time_next_decode(e0, e1)
    out = runner.decode_step(g).clone()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1)
    say(f"      kernel {t * 1e3:.1f} us")
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert 0.0 < t < 1000.0
    runner.decode_step(g)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == t


def test_block_permutation_leaves_output_bit_identical():
    from paged_kv_attention_26_amd import runner
    a = W.config2(small=True)
    b = W.config2(small=True)
    b.free_order = np.random.default_rng(99).permutation(b.num_blocks)
    ga, gb = runner.prepare(a), runner.prepare(b)
    runner.store_step(ga), runner.store_step(gb)
    assert ga.tables != gb.tables
    oa, ob = runner.decode_step(ga), runner.decode_step(gb)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


def test_partition_size_changes_output_only_by_rounding():
    from paged_kv_attention_26_amd import runner
    batch = W.config3(16, small=True)
    g = runner.prepare(batch)
    runner.store_step(g)
    outs = [out_f64(runner.decode_step(g, partition_tokens=p)) for p in (64, 256, 1024)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) < 1e-2


@pytest.mark.parametrize("small", [True, False])
def test_fp8_fork_store_copy_and_decode(small):
    from paged_kv_attention_26_amd import runner
    say(f"[gpu] fp8 fork small={small}")
    fb = W.config5(small=small)
    snap = {}

    def before(cache, beams, bm):
        table = torch.from_numpy(bm.block_tables(beams, bm.unused_block())).cuda()
        lens = torch.full((len(beams),), fb.shared_len, dtype=torch.int32, device="cuda")
        q = torch.from_numpy(np.repeat(fb.q[:1], len(beams), 0).view(np.int16)).view(torch.bfloat16).cuda()
        from paged_kv_attention_26_amd import binding as pa
        snap["out"] = pa.decode(cache, q, table, lens, fb.shared_len, fb.scale).clone()
        snap["one"] = [pa.decode(cache, q[b:b + 1].contiguous(), table[b:b + 1].contiguous(), lens[b:b + 1].contiguous(),
                                 fb.shared_len, fb.scale).clone() for b in range(len(beams))]

    gf = runner.run_fork(fb, snapshot=before)
    out = runner.fork_decode(gf)
    torch.cuda.synchronize()
    st = OS.build_fork(fb)
    # copy-on-write decisions and block contents, bit for bit
    assert gf.copy_pairs.tolist() == [list(p) for p in st.copy_pairs]
    assert len(gf.copy_pairs) == fb.beams - 1
    assert np.array_equal(bits(gf.cache.k_cache, "fp8"), st.kc)
    assert np.array_equal(bits(gf.cache.v_cache, "fp8"), st.vc)
    # forked beams read identical blocks before divergence.  Decoded one at a
    # time (the same launch for each), their outputs are bit-identical.  In one
    # batch the work is split differently for each beam, and probabilities
    # are rounded to bf16 (relative error <= 2^-9 each) against the running
    # maximum of each piece.  Over ~2k weights that reweighting moves the fp32
    # result by ~1e-4 at most in expectation; the bound allows 2^-12 for it,
    # plus up to two bf16 ulps of the value for the final rounding on either
    # side (a result may cross a binade).
    b0 = snap["one"][0].view(torch.int16)
    for b in range(1, fb.beams):
        assert torch.equal(snap["one"][b].view(torch.int16), b0)
    one = snap["one"][0][0].float()
    ulp = torch.ldexp(torch.ones_like(one), torch.frexp(one)[1] - 8)      # bf16 ulp of |one|
    drift = max(float((snap["out"][b].float() - one).abs().max()) for b in range(fb.beams))
    say(f"      batched beams vs one-at-a-time: max abs drift {drift:.3e}")
    for b in range(fb.beams):
        excess = (snap["out"][b].float() - one).abs() - (2 * ulp + 2.0 ** -12)
        assert float(excess.max()) <= 0, b
    ref = OS.fork_decode_ref(fb, st)
    err = np.max(np.abs(out_f64(out) - ref))
    say(f"      max abs err {err:.3e}")
    assert err < TOL["fp8"]


def test_fp8_codes_round_trip_through_store_and_decode():
    """Values that are exact e4m3 numbers (scale 1) are stored as their codes
    and a one-token decode returns them exactly: checks the device encoder
    and the hardware e4m3 -> fp32 conversion on every finite code."""
    from oracle import fp8_e4m3
    from paged_kv_attention_26_amd import binding as pa
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8_e4m3.decode(codes)                                   # 254 exact values
    row = np.zeros((1, 2, 128), np.float32)
    row.reshape(-1)[:254] = vals
    bits_in = W.to_bf16_bits(row)                                   # exact in bf16
    assert np.array_equal(W.bf16_bits_to_f32(bits_in).astype(np.float64), row.astype(np.float64))
    one = np.ones(2, np.float32)
    cache = pa.alloc_cache(4, 2, 16, 128, "fp8", k_scale=one, v_scale=one)
    x = torch.from_numpy(bits_in.view(np.int16)).view(torch.bfloat16).cuda()
    pa.store_kv(cache, x, x, torch.tensor([32], dtype=torch.int32, device="cuda"))   # block 2, offset 0
    k = cache.k_cache.cpu().numpy()
    v = cache.v_cache.cpu().numpy()
    assert np.array_equal(k[2, :, 0, :].reshape(-1)[:254], codes)
    assert np.array_equal(v[2, :, :, 0].reshape(-1)[:254], codes)
    # a one-token context returns that token's value exactly
    q = torch.zeros((1, 8, 128), dtype=torch.bfloat16, device="cuda")
    table = torch.tensor([[2]], dtype=torch.int32, device="cuda")
    out = pa.decode(cache, q, table, torch.tensor([1], dtype=torch.int32, device="cuda"), 1, 0.088)
    got = out.float().cpu().numpy().astype(np.float64)              # [1, 8, 128]
    want = np.repeat(row.astype(np.float64), 4, axis=1)             # kv head h -> q heads 4h..4h+3
    assert np.array_equal(got[0], want[0])


# ------------------------------------------------------------ chunked prefill
def chunk_batch(name, P, q, B=16, Hq=32, Hkv=8, seed=41, kv="bf16"):
    rng = np.random.default_rng(seed)
    n = len(P)
    return W.paged_batch(name, seed, kv_dtype=kv, io_dtype="bf16", Hq=Hq, Hkv=Hkv, d=128, B=B,
                         prior_lens=P, new_lens=q, is_chunk=np.ones(n, bool), rng=rng)


def spiky_batch(name, P, q, spikes=((1 / 3, 8.0), (2 / 3, 3.0), (1.0, 6.0))):
    """A chunk batch whose keys at a few late positions are scaled up, so that
    a query column's running maximum jumps well after the first key tile: by
    more than 2^8 in exp2 units for the larger factors (the attention kernels
    rescale their accumulators), by less for the smaller one (they keep the
    stale maximum)."""
    b = chunk_batch(name, P, q, Hq=8, Hkv=2)
    off = b.tok_offsets
    kf = W.bf16_bits_to_f32(b.k).copy()
    for s in range(b.num_seqs):
        L = int(b.prior_lens[s] + b.new_lens[s])
        for frac, f in spikes:
            pos = min(L - 1, int(frac * L))
            if pos >= 32:                                 # past the first key tile
                kf[off[s] + pos] *= f
    b.k = W.to_bf16_bits(kf)
    return b


def many_chunks():
    """300 chunk sequences: more than the prefill kernel ranks by work in
    LDS, so they run in launch order."""
    rng = np.random.default_rng(80)
    P = rng.integers(0, 120, 300)
    q = rng.integers(1, 41, 300)
    return W.paged_batch("many-chunks", 80, kv_dtype="bf16", io_dtype="bf16", Hq=8, Hkv=2, d=128, B=16,
                         prior_lens=P, new_lens=q, is_chunk=np.ones(300, bool), rng=rng)


CHUNKS = {
    "many": many_chunks,
    "spike": lambda: spiky_batch("spike", [300, 1000, 40, 0], [64, 37, 100, 80]),
    "spike-verify": lambda: spiky_batch("spike-verify", [300, 1000, 4100], [5, 8, 3]),
    "c4s": lambda: W.config4(small=True),
    "prefix0": lambda: chunk_batch("prefix0", [0, 0], [37, 64]),
    "ragged": lambda: chunk_batch("ragged", [5, 100, 33, 512, 0], [1, 31, 33, 97, 129]),
    "ragged-b32": lambda: chunk_batch("ragged-b32", [5, 100, 33, 512, 0], [1, 31, 33, 97, 129], B=32),
    "g1": lambda: chunk_batch("g1", [17, 300], [45, 70], Hq=8, Hkv=8),
    "g2": lambda: chunk_batch("g2", [17, 300], [45, 70], Hq=16, Hkv=8),
    "g8": lambda: chunk_batch("g8", [17, 300], [45, 70], Hq=32, Hkv=4),
    # speculative-verification shapes: at most 32 / G tokens per chunk
    "verify-k4": lambda: chunk_batch("verify-k4", [0, 1, 15, 16, 31, 100, 511, 512, 1023, 4100], [5] * 10),
    "verify-mixed-b32": lambda: chunk_batch("verify-mixed-b32", [3, 64, 700, 2000, 33], [1, 8, 3, 7, 2], B=32),
    "verify-long": lambda: chunk_batch("verify-long", [6000, 9000], [5, 8]),
    "verify-g1": lambda: chunk_batch("verify-g1", [40, 1000], [32, 17], Hq=8, Hkv=8),
    "verify-g2": lambda: chunk_batch("verify-g2", [40, 1000], [16, 9], Hq=16, Hkv=8),
    "verify-g8": lambda: chunk_batch("verify-g8", [40, 1000, 0], [4, 3, 4], Hq=32, Hkv=4),
    "verify-batch-small": lambda: W.verify_batch(small=True),
    # fp8 e4m3 caches (bf16 queries): both kernels
    "fp8-c4s": lambda: W.config4(small=True, kv_dtype="fp8"),
    "fp8-ragged-b32": lambda: chunk_batch("fp8-ragged-b32", [5, 100, 33, 512, 0], [1, 31, 33, 97, 129], B=32,
                                          kv="fp8"),
    "fp8-verify": lambda: chunk_batch("fp8-verify", [0, 15, 1023, 4100], [5, 8, 1, 5], kv="fp8"),
}


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("B", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_prefill_every_compiled_shape(kv, B, G):
    """Every (cache dtype, block size, group) the chunked prefill compiles,
    in both of its kernels: chunks longer than 32 / G tokens (tiles of 32
    query rows of one head) and chunks of at most 32 / G tokens (verification:
    (head, token) columns), on prefixes that end inside a block and at block
    ends, against the oracle."""
    from paged_kv_attention_26_amd import runner
    for form, P, q in (("chunks", [0, 37, 160, 500], [70, 33, 97, 1]), ("verify", [5, 64, 900], [32 // G, 1, max(1, 16 // G)])):
        batch = chunk_batch(f"every-{form}-{kv}-b{B}-g{G}", P, q, B=B, Hq=2 * G, Hkv=2, seed=900 + G + B, kv=kv)
        say(f"[gpu] prefill {batch.name}")
        g = runner.prepare(batch)
        runner.store_step(g)
        got = out_f64(runner.chunk_step(g))
        torch.cuda.synchronize()
        st = OS.build(batch)
        err = np.max(np.abs(got - OS.chunk_ref(batch, st)))
        say(f"      max abs err {err:.3e}")
        assert np.all(np.isfinite(got)) and err < TOL[kv]


@pytest.mark.parametrize("name", list(CHUNKS))
def test_prefill_chunk_matches_oracle(name):
    from paged_kv_attention_26_amd import runner
    say(f"[gpu] prefill {name}")
    batch = CHUNKS[name]()
    g = runner.prepare(batch)
    runner.store_step(g)
    out = runner.chunk_step(g)
    torch.cuda.synchronize()
    st = OS.build(batch)
    ref = OS.chunk_ref(batch, st)
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    err = np.max(np.abs(got - ref))
    say(f"      max abs err {err:.3e}")
    assert err < TOL[batch.kv_dtype]
    if (~batch.is_chunk).any():                      # the mixed batch's decode half too
        dref = OS.decode_ref(batch, st)
        derr = np.max(np.abs(out_f64(runner.decode_step(g)) - dref))
        say(f"      decode max abs err {derr:.3e}")
        assert derr < TOL[batch.kv_dtype]


def test_prefill_chunk_of_one_row_matches_decode():
    from paged_kv_attention_26_amd import binding as pa, runner
    batch = chunk_batch("one-row", [0, 1, 15, 16, 200, 511], [1, 1, 1, 1, 1, 1])
    g = runner.prepare(batch)
    runner.store_step(g)
    pre = out_f64(runner.chunk_step(g))
    c = g.chunk
    dec = out_f64(pa.decode(g.cache, c["q"], c["table"], c["seq_lens"], c["max_seq"], batch.scale))
    assert np.max(np.abs(pre - dec)) < 1e-2


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_prefill_full_mixed_batch(kv):
    """The full mixed chunked-prefill batch as benchmarked (8 chunks of 512 on
    prefixes up to 7680, 64 decodes beside them), bf16 and fp8 caches: every
    output row of every chunk, and every decode output, against the oracle;
    the 4160-row store of the step bit for bit over the whole pool."""
    from paged_kv_attention_26_amd import runner
    say(f"[gpu] prefill full mixed batch {kv}")
    batch = W.config4(kv_dtype=kv)
    g = runner.prepare(batch)
    runner.store_step(g)
    out = out_f64(runner.chunk_step(g))
    dec = out_f64(runner.decode_step(g))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(dec))
    st = OS.build(batch)
    assert np.array_equal(bits(g.cache.k_cache, kv), oracle_bits(st.kc, kv))
    assert np.array_equal(bits(g.cache.v_cache, kv), oracle_bits(st.vc, kv))
    del g
    from oracle import paged
    ch = np.flatnonzero(batch.is_chunk)
    cu = np.concatenate([[0], np.cumsum(batch.new_lens[ch])])
    worst = 0.0
    for j, i in enumerate(ch):
        tab = OS.table_array([st.tables[i]], st.pad_block)
        ref = paged.prefill_chunk_attention(st.kc, st.vc, kv, batch.q_chunk[cu[j]:cu[j + 1]], "bf16",
                                            [0, int(batch.new_lens[i])], [int(batch.total_lens[i])], tab,
                                            batch.scale, batch.k_scale, batch.v_scale)
        err = np.max(np.abs(out[cu[j]:cu[j + 1]] - ref))
        worst = max(worst, err)
        say(f"      chunk {j} (prefix {int(batch.prior_lens[i])}) max abs err {err:.3e}")
        assert err < TOL[kv]
    derr = np.max(np.abs(dec - OS.decode_ref(batch, st)))
    say(f"      all {len(ch)} chunks max abs err {worst:.3e}; {int((~batch.is_chunk).sum())} decodes {derr:.3e}")
    assert derr < TOL[kv]


# ------------------------------------------------ pack (KV hand-off)
@pytest.mark.parametrize("name", ["c1", "c2s", "c3s32", "edge16", "skew", "many"])
def test_pack_is_bit_exact(name):
    from oracle import paged
    from paged_kv_attention_26_amd import runner
    say(f"[gpu] pack {name}")
    batch = SMALL[name]()
    g = runner.prepare(batch)
    runner.store_step(g)
    k, v = runner.pack_all(g)
    torch.cuda.synchronize()
    st = OS.build(batch)
    wk, wv = paged.pack_kv(st.kc, st.vc, st.tables, batch.total_lens)
    assert np.array_equal(bits(k, batch.kv_dtype), oracle_bits(wk, batch.kv_dtype))
    assert np.array_equal(bits(v, batch.kv_dtype), oracle_bits(wv, batch.kv_dtype))


def test_pack_full_qwen3_layer():
    """The hand-off pack the bench times (the Qwen3-8B decode layer's 32
    sequences, 72k tokens, 296 MB) bit for bit against the oracle's gather."""
    from oracle import paged
    from paged_kv_attention_26_amd import runner
    say("[gpu] pack full qwen3-8b layer")
    batch = W.config2()
    g = runner.prepare(batch)
    runner.store_step(g)
    k, v = runner.pack_all(g)
    torch.cuda.synchronize()
    st = OS.build(batch)
    wk, wv = paged.pack_kv(st.kc, st.vc, st.tables, batch.total_lens)
    assert np.array_equal(bits(k, "bf16"), wk) and np.array_equal(bits(v, "bf16"), wv)
    say(f"      {k.shape[0]} rows bit-exact")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_handoff_round_trip(kv):
    """Pack every sequence out of one cache and store the rows into another
    cache with its own block layout (fp8: codes stored as they are): the
    second cache packs to the same bytes and decodes bit-identically."""
    from paged_kv_attention_26_amd import binding as pa, runner
    say(f"[gpu] hand-off round trip {kv}")
    src = W.config2(small=True)
    if kv == "fp8":
        src = W.paged_batch("handoff-fp8", 12, kv_dtype="fp8", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                            prior_lens=src.prior_lens, new_lens=src.new_lens, is_chunk=src.is_chunk,
                            rng=np.random.default_rng(12))
    ga = runner.prepare(src)
    runner.store_step(ga)
    k, v = runner.pack_all(ga)
    dst = copy.copy(src)
    dst.free_order = np.random.default_rng(78).permutation(src.num_blocks)
    gb = runner.prepare(dst, fill=False)
    slots = runner.all_slots(gb)                 # the receiving side's slots for the same tokens
    pa.store_kv(gb.cache, k, v, slots)
    k2, v2 = runner.pack_all(gb)
    torch.cuda.synchronize()
    assert torch.equal(k2.view(torch.uint8), k.view(torch.uint8)) and torch.equal(v2.view(torch.uint8), v.view(torch.uint8))
    oa, ob = runner.decode_step(ga), runner.decode_step(gb)
    torch.cuda.synchronize()
    assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))


# ------------------------------------------------ full sizes, bench launch configuration
def test_decode_full_qwen3_layer():
    """The Qwen3-8B decode layer at full size (32 seqs, 72k tokens), in the
    launch configuration the benchmark times (default partition): every
    sequence against the oracle."""
    from paged_kv_attention_26_amd import binding as pa, runner
    say("[gpu] decode full qwen3-8b layer")
    batch = W.config2()
    g = runner.prepare(batch)
    runner.store_step(g)
    ws = pa.decode_workspace(1, 1, batch.head_dim, 1, 0)
    got = out_f64(runner.decode_step(g, partition_tokens=64, workspace=ws))
    torch.cuda.synchronize()
    err = np.max(np.abs(got - OS.decode_ref(batch, OS.build(batch))))
    say(f"      max abs err {err:.3e}")
    assert err < TOL["bf16"]


_LONG = {}


def _long_context(B):
    if 16 not in _LONG:
        _LONG.clear()
        _LONG[16] = W.config3(16)
    if B not in _LONG:
        _LONG[B] = W.config3_at_block(_LONG[16], B)
    return _LONG[B]


@pytest.mark.parametrize("B", [16, 32])
def test_decode_full_long_context(B):
    """Long-context decode at full size (128 seqs, 713k tokens, contexts up
    to 28k) with 512-token partitions, as benchmarked: every sequence against
    the oracle.  The bulk store that filled the pool (the bench's bulk-store
    case) is checked bit for bit over the whole poisoned pool, and at block
    16 so is the bench's bulk copy (every free block receives a copy of a
    used one: 11 164 pairs of 64 KB per pool pair)."""
    from oracle import paged
    from paged_kv_attention_26_amd import binding as pa, runner
    say(f"[gpu] decode full long context B{B}")
    batch = _long_context(B)
    g = runner.prepare(batch)
    runner.store_step(g)
    ws = pa.decode_workspace(1, 1, batch.head_dim, 1, 512)
    got = out_f64(runner.decode_step(g, partition_tokens=512, workspace=ws))
    torch.cuda.synchronize()
    assert np.all(np.isfinite(got))
    st = OS.build(batch)
    assert np.array_equal(bits(g.cache.k_cache, "bf16"), oracle_bits(st.kc, "bf16"))
    assert np.array_equal(bits(g.cache.v_cache, "bf16"), oracle_bits(st.vc, "bf16"))
    say("      whole pool bit-exact after the bulk store")
    if B == 16:
        used = sorted({blk for row in g.tables for blk in row})
        free = sorted(set(range(batch.num_blocks)) - set(used))
        n = min(len(used), len(free))
        pairs = np.stack([np.array(used[:n]), np.array(free[:n])], 1).astype(np.int32)
        pa.copy_blocks(g.cache, torch.from_numpy(pairs).cuda())
        torch.cuda.synchronize()
        kc, vc = st.kc.copy(), st.vc.copy()
        paged.copy_blocks(kc, vc, pairs)
        assert np.array_equal(bits(g.cache.k_cache, "bf16"), kc)
        assert np.array_equal(bits(g.cache.v_cache, "bf16"), vc)
        say(f"      bulk copy of {n} pairs bit-exact over the whole pool")
        del kc, vc
    del g
    lens = batch.total_lens
    tables = OS.table_array(st.tables, st.pad_block)
    worst = 0.0
    for i0 in range(0, len(lens), 32):
        ref = paged.decode_attention(st.kc, st.vc, "bf16", batch.q_decode[i0:i0 + 32], "bf16",
                                     tables[i0:i0 + 32], lens[i0:i0 + 32], batch.scale)
        err = np.max(np.abs(got[i0:i0 + 32] - ref))
        worst = max(worst, err)
        say(f"      seqs {i0}..{min(i0 + 32, len(lens)) - 1} (L {int(lens[i0:i0 + 32].min())}.."
            f"{int(lens[i0:i0 + 32].max())}) max abs err {err:.3e}")
        assert err < TOL["bf16"]
    say(f"      all {len(lens)} sequences: max abs err {worst:.3e}")


def test_verify_full_batch():
    """Speculative verification at full size (32 seqs, 5-token chunks on
    prefixes up to 4096): every output against the oracle."""
    from paged_kv_attention_26_amd import runner
    say("[gpu] verify full batch")
    batch = W.verify_batch()
    g = runner.prepare(batch)
    runner.store_step(g)
    got = out_f64(runner.chunk_step(g))
    torch.cuda.synchronize()
    err = np.max(np.abs(got - OS.chunk_ref(batch, OS.build(batch))))
    say(f"      max abs err {err:.3e}")
    assert err < TOL["bf16"]


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_verify_split_and_whole_launches(kv):
    """Speculative verification in both launch forms: with a workspace (the
    batch's key tiles cut into equal stretches, one per CU, items cut between
    stretches merged in the kernel) and without (one workgroup per (sequence,
    kv head)).  Empty chunks sit between long and short contexts, so
    stretches start and end inside items, on items of other heads and past
    sequences without units; both forms against the oracle, and three calls
    in a row of the split form bit-identical (its counters return to zero)."""
    from paged_kv_attention_26_amd import binding as pa, runner
    batch = chunk_batch(f"verify-split-{kv}", [50, 3000, 10, 700, 0, 2500, 9000, 31, 4100],
                        [5, 0, 5, 3, 8, 0, 1, 5, 2], kv=kv, seed=77)
    say(f"[gpu] verify split / whole {batch.name}")
    g = runner.prepare(batch)
    runner.store_step(g)
    c = g.chunk
    ref = OS.chunk_ref(batch, OS.build(batch))
    call = lambda split: pa.prefill_chunk(g.cache, c["q"], c["cu"], c["seq_lens"], c["table"], c["max_q"],
                                          c["max_seq"], batch.scale, split=split)
    whole = out_f64(call(False))
    outs = [call(True).clone() for _ in range(3)]
    torch.cuda.synchronize()
    got = out_f64(outs[0])
    ew, es = np.max(np.abs(whole - ref)), np.max(np.abs(got - ref))
    say(f"      max abs err: whole {ew:.3e}, split {es:.3e}")
    assert np.all(np.isfinite(got)) and np.all(np.isfinite(whole))
    assert ew < TOL[kv] and es < TOL[kv]
    assert all(torch.equal(outs[0], o) for o in outs[1:])


def test_verify_cut_stretches_over_64_sequences():
    """A split verification launch over more than 64 sequences (the unit
    prefix then lives in LDS, built by the whole workgroup): 90 short
    contexts, some with empty chunks, around two long ones, so the launch cuts
    the batch into stretches; against the oracle."""
    from paged_kv_attention_26_amd import runner
    rng = np.random.default_rng(91)
    P = rng.integers(0, 300, 92)
    P[17], P[70] = 12000, 7000
    q = rng.integers(1, 6, 92)
    q[[3, 40, 41, 88]] = 0
    batch = chunk_batch("verify-cut-92", P, q, seed=91)
    say(f"[gpu] verify {batch.name}")
    g = runner.prepare(batch)
    runner.store_step(g)
    got = out_f64(runner.chunk_step(g))
    torch.cuda.synchronize()
    err = np.max(np.abs(got - OS.chunk_ref(batch, OS.build(batch))))
    say(f"      max abs err {err:.3e}")
    assert np.all(np.isfinite(got)) and err < TOL["bf16"]


def test_verify_long_context_full_launch():
    """Speculative verification over the long-context prefixes at full size
    (128 seqs, 713k tokens, contexts up to 28k), as benchmarked: the launch
    cuts the batch into equal stretches, so the long contexts are merged from
    several workgroups.  Every output is finite; every third sequence and the
    16 longest against the oracle."""
    from oracle import paged
    from paged_kv_attention_26_amd import runner
    say("[gpu] verify long context full")
    batch = W.verify_long_batch()
    g = runner.prepare(batch)
    runner.store_step(g)
    got = out_f64(runner.chunk_step(g))
    torch.cuda.synchronize()
    del g
    assert np.all(np.isfinite(got))
    st = OS.build(batch)
    lens = batch.total_lens
    q_lens = batch.new_lens
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    sel = sorted(set(range(0, len(lens), 3)) | set(np.argsort(lens)[-16:].tolist()))
    tables = OS.table_array([st.tables[i] for i in sel], st.pad_block)
    qs = np.concatenate([batch.q_chunk[cu[i]:cu[i + 1]] for i in sel])
    rows = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in sel])
    cu_sel = np.concatenate([[0], np.cumsum(q_lens[sel])]).astype(np.int64)
    ref = paged.prefill_chunk_attention(st.kc, st.vc, "bf16", qs, "bf16", cu_sel, lens[sel], tables, batch.scale)
    err = np.max(np.abs(got[rows] - ref))
    say(f"      {len(sel)} sequences (L up to {int(lens.max())}): max abs err {err:.3e}")
    assert err < TOL["bf16"]


def test_debug_bounds_mode(monkeypatch):
    """PA_DEBUG_BOUNDS=1: every call first checks the values in its device
    index arrays on the host.  Valid calls give the same bits as without the
    checks; calls with a planted bad value are rejected with PA_ERR_BOUNDS
    before any launch.  (The planted values are ones that would stay inside
    the pools even if launched: a repeated copy destination, a context length
    above max_context_len over a table that covers it, a negative fp8 scale.
    Slots past the pool are covered on the CPU, by pa_check_slots.)"""
    from paged_kv_attention_26_amd import _lib as L, binding as pa, runner
    say("[gpu] PA_DEBUG_BOUNDS")
    batch = W.config2(small=True)
    g = runner.prepare(batch)
    runner.store_step(g)
    want = runner.decode_step(g).clone()
    wk, wv = runner.pack_all(g)
    cb = W.config4(small=True, kv_dtype="fp8")
    gc = runner.prepare(cb)
    runner.store_step(gc)
    wc = runner.chunk_step(gc).clone()
    torch.cuda.synchronize()
    monkeypatch.setenv("PA_DEBUG_BOUNDS", "1")
    runner.store_step(g)                                        # the same rows again: same bits
    got = runner.decode_step(g)
    k, v = runner.pack_all(g)
    gotc = runner.chunk_step(gc)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert torch.equal(k.view(torch.int16), wk.view(torch.int16)) and torch.equal(v.view(torch.int16), wv.view(torch.int16))
    assert torch.equal(gotc.view(torch.int16), wc.view(torch.int16))
    d = g.dec
    with pytest.raises(L.PaError) as e:                         # a length above max_context_len
        pa.decode(g.cache, d["q"], d["table"], d["lens"], d["max_len"] - 1, batch.scale)
    assert e.value.code == L.PA_ERR_BOUNDS
    used = sorted({b for row in g.tables for b in row})
    free = [b for b in range(batch.num_blocks) if b not in set(used)]
    before = bits(g.cache.k_cache, "bf16").copy()
    with pytest.raises(L.PaError) as e:                         # one destination twice
        pa.copy_blocks(g.cache, torch.tensor([[used[0], free[0]], [used[1], free[0]]], dtype=torch.int32,
                                             device="cuda"))
    assert e.value.code == L.PA_ERR_BOUNDS
    torch.cuda.synchronize()
    assert np.array_equal(bits(g.cache.k_cache, "bf16"), before)   # nothing was launched
    gc.cache.k_scale[0] = -1.0                                  # an fp8 scale below zero
    c = gc.dec
    with pytest.raises(L.PaError) as e:
        pa.decode(gc.cache, c["q"], c["table"], c["lens"], c["max_len"], cb.scale)
    assert e.value.code == L.PA_ERR_BOUNDS
    say("      valid calls bit-identical; planted values rejected before launch")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_speculative_branches_copy_on_write(kv):
    """Speculative decoding over copy-on-write branches: a draft branch is
    forked from each target, its first append copies the shared tail
    (pa_copy_blocks), the drafts are stored and verified in one
    pa_prefill_chunk call over the branches, the targets keep the accepted
    drafts and the branches are released.  Copy pairs, tables, reference
    counts and the whole pool (bit for bit) match the oracle's run, and so
    do the verification and the targets' next decode, within tolerance."""
    from paged_kv_attention_26_amd import runner
    w = W.spec_branch(kv)
    say(f"[gpu] speculative branches {w.name}")
    got = runner.run_spec_branch(w)
    torch.cuda.synchronize()
    ref = OS.build_spec_branch(w)
    assert got.copy_pairs.tolist() == [list(p) for p in ref.copy_pairs]
    assert len(ref.copy_pairs) == int(np.sum(w.prefix_lens % w.block_size != 0))
    assert got.branch_tables == ref.branch_tables and got.target_tables == ref.target_tables
    assert [got.bm.ref_count(b) for b in range(w.num_blocks)] == ref.ref_count
    assert got.bm.used_blocks == ref.used_blocks
    assert np.array_equal(bits(got.cache.k_cache, kv), oracle_bits(ref.kc, kv))
    assert np.array_equal(bits(got.cache.v_cache, kv), oracle_bits(ref.vc, kv))
    ev = np.max(np.abs(out_f64(got.verify_out) - ref.verify_out))
    ed = np.max(np.abs(out_f64(got.decode_out) - ref.decode_out))
    say(f"      {len(ref.copy_pairs)} copies; verify err {ev:.3e}, next decode err {ed:.3e}")
    assert ev < TOL[kv] and ed < TOL[kv]


@pytest.mark.parametrize("kv,B,d", [("bf16", 16, 64), ("bf16", 32, 128), ("f32", 16, 128), ("f32", 32, 128),
                                    ("f32", 32, 64), ("fp8", 16, 128), ("fp8", 32, 64)])
def test_copy_blocks_many_pairs_bit_exact(kv, B, d):
    """pa_copy_blocks with thousands of pairs over pools of 8 kv heads (blocks
    of 16 KB to 128 KB per pool, so the per-block loop of the larger ones runs
    several passes), random contents, destinations distinct and never a
    source, sources repeated: the whole pools bit for bit against the
    oracle's copy."""
    from oracle import paged
    from paged_kv_attention_26_amd import binding as pa
    Hkv = 8
    es = {"f32": 4, "bf16": 2, "fp8": 1}[kv]
    block = Hkv * B * d * es
    n = min(4000, (192 << 20) // block)
    nb = 2 * n + 64
    say(f"[gpu] copy blocks {kv} B{B} d{d}: {n} pairs of {block} B")
    rng = np.random.default_rng(900 + B + d + es)
    perm = rng.permutation(nb)
    pairs = np.stack([rng.choice(perm[n:], n), perm[:n]], 1).astype(np.int32)
    kb = rng.integers(0, 256, size=(nb, Hkv, B, d * es), dtype=np.uint8)
    vb = rng.integers(0, 256, size=(nb, Hkv, d, B * es), dtype=np.uint8)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[kv]
    k = torch.from_numpy(kb).cuda().view(tdt)
    v = torch.from_numpy(vb).cuda().view(tdt)
    scale = torch.ones(Hkv, dtype=torch.float32, device="cuda") if kv == "fp8" else None
    cache = pa.KVCache(k, v, kv, scale, scale)
    pa.copy_blocks(cache, torch.from_numpy(pairs).cuda())
    torch.cuda.synchronize()
    paged.copy_blocks(kb, vb, pairs)
    assert np.array_equal(k.view(torch.uint8).cpu().numpy(), kb)
    assert np.array_equal(v.view(torch.uint8).cpu().numpy(), vb)


@pytest.mark.parametrize("kv,small", [("bf16", True), ("fp8", True), ("bf16", False)])
def test_prefix_cache_conversations(kv, small):
    """Multi-turn conversations sharing a system prompt through the prefix
    cache: the library's block manager takes the oracle's decisions, chunked
    prefill and decode over the shared blocks match the oracle, and the
    blocks the cache holds at the end are bit-identical."""
    from paged_kv_attention_26_amd import runner
    w = W.prefix_agent(small=small, kv_dtype=kv)
    say(f"[gpu] prefix cache {w.name}")
    cache, bm, got = runner.run_prefix_agent(w)
    torch.cuda.synchronize()
    kc, vc, mgr, oc, ref = OS.build_prefix_agent(w)
    for t, (g, r) in enumerate(zip(got, ref), start=1):
        assert g.active == r.active and g.hits == r.hits and g.tables == r.tables, t
        ep = np.max(np.abs(out_f64(g.prefill_out) - r.prefill_out))
        ed = np.max(np.abs(out_f64(g.decode_out) - r.decode_out))
        say(f"      turn {t}: hits {g.hits} prefill err {ep:.3e} decode err {ed:.3e}")
        assert ep < TOL[kv] and ed < TOL[kv]
    st = bm.prefix_stats()
    assert (st["hits"], st["misses"], st["cached_blocks"]) == (oc.hits, oc.misses, len(oc.table))
    held = sorted(oc.table.values())
    assert held == [b for b in range(w.num_blocks) if bm.ref_count(b)]
    assert np.array_equal(bits(cache.k_cache, kv)[held], oracle_bits(kc, kv)[held])
    assert np.array_equal(bits(cache.v_cache, kv)[held], oracle_bits(vc, kv)[held])


# ------------------------------------------------ seeded random shapes
def random_decode_batch(seed):
    """A seeded random decode batch: batch size, length mix (empty, single
    token, block edges, long), group size, block size, head dim, cache dtype
    and split grain all drawn from the supported set."""
    rng = np.random.default_rng(9000 + seed)
    kv = ["bf16", "fp8", "f32"][seed % 3]
    d = 64 if kv == "f32" else int(rng.choice([64, 128]))
    if kv == "fp8":
        d = 128
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([16, 32]))
    S = int(rng.integers(1, 90))
    kinds = rng.integers(0, 5, S)
    lens = np.where(kinds == 0, 0, np.where(kinds == 1, rng.integers(1, 3, S),
                    np.where(kinds == 2, B * rng.integers(1, 8, S) + rng.integers(-1, 2, S),
                             rng.integers(1, 3000, S))))
    lens = np.maximum(lens, 0)
    prior = np.maximum(lens - 1, 0)
    new = (lens > 0).astype(np.int64)
    io = "f32" if kv == "f32" else "bf16"
    b = W.paged_batch(f"rand-dec-{seed}", 9000 + seed, kv_dtype=kv, io_dtype=io, Hq=G * Hkv, Hkv=Hkv, d=d, B=B,
                      prior_lens=prior, new_lens=new, is_chunk=np.zeros(S, bool), rng=rng)
    return b, int(rng.choice([0, 64, 128, 256, 512]))


@pytest.mark.parametrize("seed", range(12))
def test_decode_random_shapes(seed):
    from paged_kv_attention_26_amd import runner
    batch, part = random_decode_batch(seed)
    say(f"[gpu] random decode {batch.name}: S={batch.num_seqs} {batch.kv_dtype} d={batch.head_dim} "
        f"G={batch.num_q_heads // batch.num_kv_heads} Hkv={batch.num_kv_heads} B={batch.block_size} part={part}")
    g = runner.prepare(batch)
    runner.store_step(g)
    out = out_f64(runner.decode_step(g, partition_tokens=part))
    torch.cuda.synchronize()
    st = OS.build(batch)
    ref = OS.decode_ref(batch, st)
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(out - ref)) if out.size else 0.0
    say(f"      max abs err {err:.3e}")
    assert err < TOL[batch.kv_dtype]
    _append_vs_store_then_decode(batch, partitions=(part,))   # the store inside the launch: bit for bit


def random_chunk_batch(seed):
    """A seeded random chunked-prefill batch (chunks of 1 to 300 tokens on
    prefixes of 0 to 2000, some sequences decoding beside them); every fourth
    seed keeps chunks within 32 / G tokens, the speculative-verification form."""
    rng = np.random.default_rng(9500 + seed)
    kv = ["bf16", "fp8"][seed % 2]
    G = int(rng.choice([1, 2, 4, 8]))
    Hkv = int(rng.choice([1, 2, 4]))
    B = int(rng.choice([16, 32]))
    S = int(rng.integers(1, 24))
    is_chunk = rng.random(S) < 0.7
    is_chunk[0] = True
    P = rng.integers(0, 2000, S)
    qmax = max(2, 32 // G + 1) if seed % 4 == 3 else 300
    q = np.where(is_chunk, rng.integers(1, qmax, S), 1)
    return W.paged_batch(f"rand-chunk-{seed}", 9500 + seed, kv_dtype=kv, io_dtype="bf16", Hq=G * Hkv, Hkv=Hkv,
                         d=128, B=B, prior_lens=P, new_lens=q, is_chunk=is_chunk, rng=rng)


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random_shapes(seed):
    from paged_kv_attention_26_amd import runner
    batch = random_chunk_batch(seed)
    say(f"[gpu] random prefill {batch.name}: S={batch.num_seqs} {batch.kv_dtype} "
        f"G={batch.num_q_heads // batch.num_kv_heads} Hkv={batch.num_kv_heads} B={batch.block_size}")
    g = runner.prepare(batch)
    runner.store_step(g)
    out = out_f64(runner.chunk_step(g))
    torch.cuda.synchronize()
    st = OS.build(batch)
    ref = OS.chunk_ref(batch, st)
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(out - ref))
    say(f"      max abs err {err:.3e}")
    assert err < TOL[batch.kv_dtype]
    if (~batch.is_chunk).any():
        dref = OS.decode_ref(batch, st)
        derr = np.max(np.abs(out_f64(runner.decode_step(g)) - dref))
        say(f"      decode max abs err {derr:.3e}")
        assert derr < TOL[batch.kv_dtype]
