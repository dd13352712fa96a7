"""Pins for the oracle's store / copy / attention (CPU only).

Attention is pinned to torch's fp64 ``scaled_dot_product_attention`` (math
path, CPU) over contiguous K/V built straight from the generated values,
with explicit GQA repetition (contiguous head groups) and, for chunks, an
explicit causal mask aligned to the end of the keys.  The fp8 dense check
quantises through torch's float8_e4m3fn cast.  Closed forms and invariants
(block permutation, fork before divergence, chunk splitting, split-K merge)
cover what the dense check cannot see.
"""
import copy
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import workloads as W
from oracle import fp8_e4m3, paged
from tests import oracle_setup as OS


# --------------------------------------------------------------- dense refs
def io_to_f64(x, io_dtype):
    if io_dtype == "f32":
        return np.asarray(x, np.float32).astype(np.float64)
    return W.bf16_bits_to_f32(x).astype(np.float64)


def kv_dense_values(batch_k, io_dtype, kv_dtype, head_scale):
    """The values a cache of kv_dtype holds for these input rows [n, Hkv, d]."""
    x = io_to_f64(batch_k, io_dtype)
    if kv_dtype != "fp8":
        return x
    s = torch.from_numpy(np.asarray(head_scale, np.float32))[None, :, None]
    q = (torch.from_numpy(x.astype(np.float32)) / s).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * s.to(torch.float64)).numpy()


def sdpa(q, k, v, mask=None, is_causal=False, scale=None):
    """q [Hq, n, d], k/v [Hkv, L, d] fp64 -> [Hq, n, d]; GQA by repeat_interleave.

    ``scale`` is the fp32-rounded 1/sqrt(d) that the kernels receive; None
    leaves torch's own default (exact for d = 64)."""
    G = q.shape[0] // k.shape[0]
    kt = torch.from_numpy(k).repeat_interleave(G, dim=0)[None]
    vt = torch.from_numpy(v).repeat_interleave(G, dim=0)[None]
    qt = torch.from_numpy(q)[None]
    m = None if mask is None else torch.from_numpy(mask)[None, None]
    return F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=is_causal, scale=scale)[0].numpy()


def dense_decode(batch):
    K = kv_dense_values(batch.k, batch.io_dtype, batch.kv_dtype, batch.k_scale)
    V = kv_dense_values(batch.v, batch.io_dtype, batch.kv_dtype, batch.v_scale)
    Q = io_to_f64(batch.q_decode, batch.io_dtype)
    off = batch.tok_offsets
    outs = []
    for j, i in enumerate(np.flatnonzero(~batch.is_chunk)):
        a, L = int(off[i]), int(batch.total_lens[i])
        k = K[a:a + L].transpose(1, 0, 2).copy()
        v = V[a:a + L].transpose(1, 0, 2).copy()
        outs.append(sdpa(Q[j][:, None, :], k, v, scale=batch.scale)[:, 0, :])
    return np.stack(outs)


def dense_chunk(batch):
    K = kv_dense_values(batch.k, batch.io_dtype, batch.kv_dtype, batch.k_scale)
    V = kv_dense_values(batch.v, batch.io_dtype, batch.kv_dtype, batch.v_scale)
    Q = io_to_f64(batch.q_chunk, batch.io_dtype)
    off = batch.tok_offsets
    outs, r = [], 0
    for i in np.flatnonzero(batch.is_chunk):
        a, P, n = int(off[i]), int(batch.prior_lens[i]), int(batch.new_lens[i])
        k = K[a:a + P + n].transpose(1, 0, 2).copy()
        v = V[a:a + P + n].transpose(1, 0, 2).copy()
        q = Q[r:r + n].transpose(1, 0, 2).copy()
        mask = np.zeros((n, P + n))
        for t in range(n):                     # query t (absolute P+t) sees keys 0..P+t
            mask[t, P + t + 1:] = -np.inf
        outs.append(sdpa(q, k, v, mask=mask, scale=batch.scale).transpose(1, 0, 2))
        r += n
    return np.concatenate(outs)


SMALL = {
    "c1": lambda: W.config1(),
    "c2s": lambda: W.config2(small=True),
    "c3s16": lambda: W.config3(16, small=True),
    "c3s32": lambda: W.config3(32, small=True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_matches_dense_sdpa(name):
    batch = SMALL[name]()
    st = OS.build(batch)
    ours = OS.decode_ref(batch, st)
    ref = dense_decode(batch)
    assert np.max(np.abs(ours - ref)) < 1e-12


def test_chunk_matches_dense_sdpa():
    batch = W.config4(small=True)
    st = OS.build(batch)
    assert np.max(np.abs(OS.chunk_ref(batch, st) - dense_chunk(batch))) < 1e-12
    assert np.max(np.abs(OS.decode_ref(batch, st) - dense_decode(batch))) < 1e-12


def test_verify_chunk_matches_dense_sdpa():
    """Speculative verification (5-token chunks on paged prefixes) against
    dense attention with an explicit end-aligned causal mask."""
    batch = W.verify_batch(small=True)
    st = OS.build(batch)
    assert np.max(np.abs(OS.chunk_ref(batch, st) - dense_chunk(batch))) < 1e-12


def test_fp8_chunk_matches_dense_sdpa():
    """Chunks over an fp8 cache: the stored codes times the per-head scales,
    attended densely with the end-aligned causal mask."""
    batch = W.config4(small=True, kv_dtype="fp8")
    st = OS.build(batch)
    assert np.max(np.abs(OS.chunk_ref(batch, st) - dense_chunk(batch))) < 1e-12


def test_fp8_decode_matches_dense_sdpa():
    """Shared-prefix beams of the small fork config as a plain decode batch."""
    fb = W.config5(small=True)
    st = OS.build_fork(fb)
    ours = OS.fork_decode_ref(fb, st)
    K = kv_dense_values(np.concatenate([fb.k_shared[None].repeat(fb.beams, 0).transpose(1, 0, 2, 3),
                                        fb.k_beam]), "bf16", "fp8", fb.k_scale)     # [T, beams, Hkv, d]
    V = kv_dense_values(np.concatenate([fb.v_shared[None].repeat(fb.beams, 0).transpose(1, 0, 2, 3),
                                        fb.v_beam]), "bf16", "fp8", fb.v_scale)
    Q = io_to_f64(fb.q, "bf16")
    for b in range(fb.beams):
        k = K[:, b].transpose(1, 0, 2).copy()
        v = V[:, b].transpose(1, 0, 2).copy()
        ref = sdpa(Q[b][:, None, :], k, v, scale=fb.scale)[:, 0, :]
        assert np.max(np.abs(ours[b] - ref)) < 1e-12


def test_prefix_zero_is_library_causal_attention():
    rng = np.random.default_rng(7)
    batch = W.paged_batch("p0", 7, kv_dtype="f32", io_dtype="f32", Hq=4, Hkv=2, d=64, B=16,
                          prior_lens=[0, 0], new_lens=[37, 64], is_chunk=[True, True], rng=rng)
    st = OS.build(batch)
    ours = OS.chunk_ref(batch, st)
    K, V, Q = batch.k.astype(np.float64), batch.v.astype(np.float64), batch.q_chunk.astype(np.float64)
    r = 0
    for n in (37, 64):
        ref = sdpa(Q[r:r + n].transpose(1, 0, 2).copy(), K[r:r + n].transpose(1, 0, 2).copy(),
                   V[r:r + n].transpose(1, 0, 2).copy(), is_causal=True).transpose(1, 0, 2)
        assert np.max(np.abs(ours[r:r + n] - ref)) < 1e-12
        r += n


# ------------------------------------------------------------ closed forms
def _one_seq_cache(keys, vals, B=16, perm_seed=0):
    """Pools holding one sequence's rows [L, Hkv, d] (f32) through a permuted table."""
    L, Hkv, d = keys.shape
    nb = math.ceil(L / B) + 3
    table = np.random.default_rng(perm_seed).permutation(nb)[: math.ceil(L / B)]
    kc, vc = paged.new_pools(nb, Hkv, B, d, "f32")
    slots = np.array([table[i // B] * B + i % B for i in range(L)])
    paged.store_kv(kc, vc, "f32", keys.astype(np.float32), vals.astype(np.float32), "f32", slots)
    return kc, vc, table[None, :].astype(np.int32)


def test_single_token_returns_its_value_exactly():
    rng = np.random.default_rng(3)
    k = rng.standard_normal((1, 2, 64)).astype(np.float32)
    v = rng.standard_normal((1, 2, 64)).astype(np.float32)
    q = rng.standard_normal((1, 4, 64)).astype(np.float32)
    kc, vc, tab = _one_seq_cache(k, v)
    out = paged.decode_attention(kc, vc, "f32", q, "f32", tab, [1], 0.125)
    assert np.array_equal(out[0, :2], np.repeat(v[0, :1].astype(np.float64), 2, 0))
    assert np.array_equal(out[0, 2:], np.repeat(v[0, 1:].astype(np.float64), 2, 0))


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(4)
    L = 77
    k = np.repeat(rng.standard_normal((1, 2, 64)).astype(np.float32), L, 0)
    v = rng.standard_normal((L, 2, 64)).astype(np.float32)
    q = rng.standard_normal((1, 4, 64)).astype(np.float32)
    kc, vc, tab = _one_seq_cache(k, v)
    out = paged.decode_attention(kc, vc, "f32", q, "f32", tab, [L], 0.125)
    mean = v.astype(np.float64).mean(axis=0)
    assert np.allclose(out[0, 0], mean[0], atol=1e-13) and np.allclose(out[0, 3], mean[1], atol=1e-13)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(5)
    L = 50
    k = rng.standard_normal((L, 1, 64)).astype(np.float32) * 0.01
    q = np.zeros((1, 1, 64), np.float32)
    q[0, 0, 0] = 1.0
    k[31, 0, 0] = 4000.0                     # score 4000/8 = 500 above the rest
    v = rng.standard_normal((L, 1, 64)).astype(np.float32)
    kc, vc, tab = _one_seq_cache(k, v)
    out = paged.decode_attention(kc, vc, "f32", q, "f32", tab, [L], 0.125)
    assert np.allclose(out[0, 0], v[31, 0], atol=1e-12)


def test_empty_context_gives_zero():
    kc, vc = paged.new_pools(4, 2, 16, 64, "bf16")
    q = W.to_bf16_bits(np.ones((2, 4, 64), np.float32))
    out = paged.decode_attention(kc, vc, "bf16", q, "bf16", np.zeros((2, 1), np.int32), [0, 0], 0.125)
    assert np.array_equal(out, np.zeros_like(out))


def test_softmax_of_shifted_scores_is_unchanged():
    """A dropped max-subtraction would overflow here (scores ~ 1e3)."""
    rng = np.random.default_rng(6)
    L = 40
    k = (rng.standard_normal((L, 1, 64)) * 30).astype(np.float32)
    v = rng.standard_normal((L, 1, 64)).astype(np.float32)
    q = (rng.standard_normal((1, 1, 64)) * 30).astype(np.float32)
    kc, vc, tab = _one_seq_cache(k, v)
    out = paged.decode_attention(kc, vc, "f32", q, "f32", tab, [L], 0.125)
    assert np.all(np.isfinite(out))
    ref = sdpa(q[0][:, None, :].astype(np.float64), k.transpose(1, 0, 2).astype(np.float64),
               v.transpose(1, 0, 2).astype(np.float64))[:, 0]
    assert np.max(np.abs(out[0] - ref)) < 1e-12


# -------------------------------------------------------------- invariants
def test_block_permutation_leaves_output_bit_identical():
    a = W.config2(small=True)
    b = W.config2(small=True)
    b.free_order = np.random.default_rng(99).permutation(b.num_blocks)
    sa, sb = OS.build(a), OS.build(b)
    assert sa.tables != sb.tables
    assert np.array_equal(OS.decode_ref(a, sa), OS.decode_ref(b, sb))


def test_forked_beams_identical_before_divergence():
    fb = W.config5(small=True)
    seen = {}

    def check(kc, vc, beams):
        tables = OS.table_array([b.block_table for b in beams], 0)
        q = np.repeat(fb.q[:1], len(beams), 0)
        out = paged.decode_attention(kc, vc, "fp8", q, "bf16", tables, [b.length for b in beams], fb.scale,
                                     fb.k_scale, fb.v_scale)
        seen["out"] = out

    st = OS.build_fork(fb, check_before_divergence=check)
    out = seen["out"]
    for b in range(1, fb.beams):
        assert np.array_equal(out[b], out[0])
    # 7 (here beams-1) copies of the shared tail; right after the copies every
    # beam still reads the same values
    assert len(st.copy_pairs) == fb.beams - 1
    assert len({s for s, _ in st.copy_pairs}) == 1


def test_literal_fork_at_full_block_copies_nothing():
    fb = W.config5(small=True, literal_fork=True)
    assert fb.shared_len % fb.block_size == 0
    st = OS.build_fork(fb)
    assert st.copy_pairs == []
    fb2 = W.config5(small=True)
    assert len(OS.build_fork(fb2).copy_pairs) == fb2.beams - 1


def test_full_size_fork_counts():
    """The 2048-token prompt forked at 2049 tokens into 8 beams: 7 copies, and
    a context of 2049 + 64 = 2113 per beam; at exactly 2048 there is no copy."""
    from oracle.block_manager import BlockManager, Sequence
    for shared, want_pairs in ((2049, 7), (2048, 0)):
        mgr = BlockManager(1000, 16)
        p = Sequence(mgr, 0)
        p.append_slots(shared)
        beams = [p] + [p.fork(i) for i in range(1, 8)]
        assert all(mgr.ref_count[b] == 8 for b in p.block_table)
        for _ in range(64):
            for b in beams:
                b.append_slot()
        assert len(mgr.take_copies()) == want_pairs
        assert {b.length for b in beams} == {shared + 64}


def test_chunk_split_in_two_matches_one_chunk():
    rng = np.random.default_rng(8)
    one = W.paged_batch("one", 8, kv_dtype="bf16", io_dtype="bf16", Hq=8, Hkv=2, d=128, B=16,
                        prior_lens=[133], new_lens=[80], is_chunk=[True], rng=rng)
    st = OS.build(one)
    full = OS.chunk_ref(one, st)
    tab = OS.table_array(st.tables, st.pad_block)
    halves = []
    for lo, hi in ((0, 40), (40, 80)):
        halves.append(paged.prefill_chunk_attention(st.kc, st.vc, "bf16", one.q_chunk[lo:hi], "bf16",
                                                    [0, hi - lo], [133 + hi], tab, one.scale))
    assert np.max(np.abs(np.concatenate(halves) - full)) < 1e-13


def test_chunk_of_one_equals_decode():
    batch = W.config4(small=True)
    st = OS.build(batch)
    i = int(np.flatnonzero(batch.is_chunk)[0])
    tab = OS.table_array([st.tables[i]], st.pad_block)
    P = int(batch.prior_lens[i])
    for t in (0, 17, int(batch.new_lens[i]) - 1):
        q = batch.q_chunk[t:t + 1]
        c = paged.prefill_chunk_attention(st.kc, st.vc, "bf16", q, "bf16", [0, 1], [P + t + 1], tab,
                                          batch.scale)
        d = paged.decode_attention(st.kc, st.vc, "bf16", q, "bf16", tab, [P + t + 1], batch.scale)
        assert np.max(np.abs(c - d)) < 1e-13


def test_split_k_log_sum_exp_merge_identity():
    """Partials over 512-token partitions merged by max-rescaling reproduce the
    oracle's one-pass result (the identity the split-K kernels rely on)."""
    batch = W.config3(16, small=True)
    st = OS.build(batch)
    ref = OS.decode_ref(batch, st)
    G = batch.num_q_heads // batch.num_kv_heads
    qf = W.bf16_bits_to_f32(batch.q_decode).astype(np.float64)
    for s in range(batch.num_seqs):
        L = int(batch.total_lens[s])
        k, v = paged.gather_kv(st.kc, st.vc, "bf16", st.tables[s], L)
        for h in (0, batch.num_q_heads - 1):
            ms, ls, accs = [], [], []
            for p0 in range(0, L, 512):
                sc = batch.scale * (k[p0:p0 + 512, h // G] @ qf[s, h])
                m = sc.max()
                e = np.exp(sc - m)
                ms.append(m), ls.append(e.sum()), accs.append(e @ v[p0:p0 + 512, h // G])
            M = max(ms)
            w = np.exp(np.array(ms) - M)
            o = (w[:, None] * np.array(accs)).sum(0) / (w * np.array(ls)).sum()
            assert np.max(np.abs(o - ref[s, h])) < 1e-12


# ------------------------------------------------------------- store, copy
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_store_places_rows_and_leaves_poison(kv):
    rng = np.random.default_rng(11)
    io = "f32" if kv == "f32" else "bf16"
    T, Hkv, d, B, nb = 20, 2, 64, 16, 6
    x = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    y = rng.standard_normal((T, Hkv, d)).astype(np.float32)
    xs = x if io == "f32" else W.to_bf16_bits(x)
    ys = y if io == "f32" else W.to_bf16_bits(y)
    slots = rng.permutation(nb * B)[:T]
    slots[3] = -1
    ksc = np.array([0.01, 0.02], np.float32) if kv == "fp8" else None
    kc, vc = paged.new_pools(nb, Hkv, B, d, kv)
    paged.store_kv(kc, vc, kv, xs, ys, io, slots, ksc, ksc)
    want_k = kv_dense_values(xs, io, kv, ksc)
    want_v = kv_dense_values(ys, io, kv, ksc)
    written = np.zeros((nb, B), bool)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        b, o = divmod(int(sl), B)
        written[b, o] = True
        got_k = paged._stored_to_f64(kc[b, :, o, :], kv, ksc)
        got_v = paged._stored_to_f64(vc[b, :, :, o], kv, ksc)
        assert np.array_equal(got_k, want_k[t]) and np.array_equal(got_v, want_v[t])
    # untouched slots keep the NaN poison
    kdec = paged._stored_to_f64(kc.transpose(0, 2, 1, 3), kv, ksc)      # [nb, B, Hkv, d]
    vdec = paged._stored_to_f64(vc.transpose(0, 3, 1, 2), kv, ksc)
    assert np.all(np.isnan(kdec[~written])) and np.all(np.isnan(vdec[~written]))


def test_copy_blocks_copies_whole_blocks():
    rng = np.random.default_rng(12)
    kc = rng.integers(0, 2 ** 16, size=(10, 2, 16, 64), dtype=np.uint16)
    vc = rng.integers(0, 2 ** 16, size=(10, 2, 64, 16), dtype=np.uint16)
    k0, v0 = kc.copy(), vc.copy()
    paged.copy_blocks(kc, vc, [[1, 7], [4, 2], [1, 9]])
    for s, dd in ((1, 7), (4, 2), (1, 9)):
        assert np.array_equal(kc[dd], k0[s]) and np.array_equal(vc[dd], v0[s])
    for b in (0, 1, 3, 4, 5, 6, 8):
        assert np.array_equal(kc[b], k0[b]) and np.array_equal(vc[b], v0[b])


# ------------------------------------------------------- pack (KV hand-off)
@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_pack_returns_the_stored_rows_in_token_order(kv):
    """Packing every sequence gives back, row for row, what was stored: the
    generator's own values (f32 / bf16) or their e4m3 codes (fp8)."""
    if kv == "f32":
        batch = W.config1()
    elif kv == "bf16":
        batch = W.config2(small=True)
    else:
        batch = W.config3(16, small=True)
        batch = W.paged_batch("fp8-pack", 9, kv_dtype="fp8", io_dtype="bf16", Hq=8, Hkv=2, d=64, B=16,
                              prior_lens=batch.prior_lens, new_lens=batch.new_lens, is_chunk=batch.is_chunk,
                              rng=np.random.default_rng(9))
    st = OS.build(batch)
    k, v = paged.pack_kv(st.kc, st.vc, st.tables, batch.total_lens)
    if kv == "fp8":
        want_k = fp8_e4m3.quantize(W.bf16_bits_to_f32(batch.k), batch.k_scale[None, :, None])
        want_v = fp8_e4m3.quantize(W.bf16_bits_to_f32(batch.v), batch.v_scale[None, :, None])
    else:
        want_k, want_v = batch.k, batch.v
    assert k.dtype == st.kc.dtype and k.shape == want_k.shape
    assert np.array_equal(k, want_k) and np.array_equal(v, want_v)


def test_pack_then_store_elsewhere_keeps_attention_bit_identical():
    """Hand-off round trip: pack from one pool, store into a pool with another
    block layout (the receiving side's slot mapping), and decode both."""
    batch = W.config2(small=True)
    st = OS.build(batch)
    k, v = paged.pack_kv(st.kc, st.vc, st.tables, batch.total_lens)
    other = copy.copy(batch)
    other.free_order = np.random.default_rng(77).permutation(batch.num_blocks)
    mgr, tables, prior, step, pad = OS.allocate(other)
    kc, vc = paged.new_pools(other.num_blocks, other.num_kv_heads, other.block_size, other.head_dim, "bf16")
    slots = np.concatenate([np.concatenate([p, s]) for p, s in zip(prior, step)]).astype(np.int64)
    paged.store_kv(kc, vc, "bf16", k, v, "bf16", slots)
    k2, v2 = paged.pack_kv(kc, vc, tables, batch.total_lens)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
    dec = np.flatnonzero(~batch.is_chunk)
    a = paged.decode_attention(st.kc, st.vc, "bf16", batch.q_decode, "bf16",
                               OS.table_array([st.tables[i] for i in dec], st.pad_block), batch.total_lens[dec],
                               batch.scale)
    b = paged.decode_attention(kc, vc, "bf16", batch.q_decode, "bf16",
                               OS.table_array([tables[i] for i in dec], pad), batch.total_lens[dec], batch.scale)
    assert np.array_equal(a, b)


def test_pack_of_empty_sequences_is_empty():
    kc, vc = paged.new_pools(4, 2, 16, 64, "bf16")
    k, v = paged.pack_kv(kc, vc, [[0], [1, 2]], [0, 0])
    assert k.shape == (0, 2, 64) and v.shape == (0, 2, 64)
