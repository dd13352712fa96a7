"""Lay a generated workload onto the GPU through libpa (product side).

Allocation goes through libpa's own host block manager; pools are filled by
pa_store_kv; the step then runs store -> attention.  Allocation order:
sequences in listed order, each taking slots for its cached tokens and then
for the tokens of the step.  Block-table rows are padded with a block that
no sequence holds.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

from . import binding as pa


def _t(x: np.ndarray, device, dtype=None) -> torch.Tensor:
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        t = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(x)
    if dtype is not None and t.dtype != dtype:
        t = t.to(dtype)
    return t.to(device)


def _table_rows(rows: List[list], pad: int, width: Optional[int] = None) -> np.ndarray:
    w = max([1] + [len(r) for r in rows]) if width is None else width
    out = np.full((len(rows), w), pad, dtype=np.int32)
    for i, r in enumerate(rows):
        out[i, :len(r)] = r
    return out


@dataclass
class GpuBatch:
    batch: object
    cache: pa.KVCache
    bm: pa.BlockManager
    tables: List[list]
    pad: int
    prior_slots: torch.Tensor
    k_prior: torch.Tensor
    v_prior: torch.Tensor
    step_slots: torch.Tensor
    k_step: torch.Tensor
    v_step: torch.Tensor
    dec: dict = field(default_factory=dict)
    chunk: dict = field(default_factory=dict)


def prepare(batch, device="cuda", fill=True) -> GpuBatch:
    """Allocate, upload and (if ``fill``) store the cached tokens of a PagedBatch."""
    bm = pa.BlockManager(batch.num_blocks, batch.block_size, batch.free_order)
    prior, step = [], []
    for i in range(batch.num_seqs):
        s = bm.seq_new()
        prior.append(bm.append(s, int(batch.prior_lens[i])))
        step.append(bm.append(s, int(batch.new_lens[i])))
    tables = [bm.block_table(i) for i in range(batch.num_seqs)]
    pad = bm.unused_block()
    off = batch.tok_offsets
    pidx, sidx = [], []
    for i in range(batch.num_seqs):
        a, p, n = int(off[i]), int(batch.prior_lens[i]), int(batch.new_lens[i])
        pidx.append(np.arange(a, a + p))
        sidx.append(np.arange(a + p, a + p + n))
    pidx = np.concatenate(pidx).astype(np.int64)
    sidx = np.concatenate(sidx).astype(np.int64)
    cache = pa.alloc_cache(batch.num_blocks, batch.num_kv_heads, batch.block_size, batch.head_dim,
                           batch.kv_dtype, device=device, k_scale=batch.k_scale, v_scale=batch.v_scale)
    g = GpuBatch(batch, cache, bm, tables, pad,
                 _t(np.concatenate(prior).astype(np.int32), device), _t(batch.k[pidx], device),
                 _t(batch.v[pidx], device),
                 _t(np.concatenate(step).astype(np.int32), device), _t(batch.k[sidx], device),
                 _t(batch.v[sidx], device))
    dec = np.flatnonzero(~batch.is_chunk)
    if len(dec):
        lens = batch.total_lens[dec]
        g.dec = dict(idx=dec, q=_t(batch.q_decode, device),
                     table=_t(_table_rows([tables[i] for i in dec], pad), device),
                     lens=_t(lens.astype(np.int32), device), max_len=int(lens.max()), host_lens=lens)
    ch = np.flatnonzero(batch.is_chunk)
    if len(ch):
        ql = batch.new_lens[ch]
        cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        tl = batch.total_lens[ch]
        g.chunk = dict(idx=ch, q=_t(batch.q_chunk, device), cu=_t(cu, device),
                       seq_lens=_t(tl.astype(np.int32), device),
                       table=_t(_table_rows([tables[i] for i in ch], pad), device),
                       max_q=int(ql.max()), max_seq=int(tl.max()), host_prefix=(tl - ql), host_q=ql)
    if fill:
        fill_prior(g)
    return g


def fill_prior(g: GpuBatch) -> None:
    if g.prior_slots.numel():
        pa.store_kv(g.cache, g.k_prior, g.v_prior, g.prior_slots)


def store_step(g: GpuBatch) -> None:
    if g.step_slots.numel():
        pa.store_kv(g.cache, g.k_step, g.v_step, g.step_slots)


def decode_step(g: GpuBatch, out=None, partition_tokens=64, workspace=None) -> torch.Tensor:
    d = g.dec
    return pa.decode(g.cache, d["q"], d["table"], d["lens"], d["max_len"], g.batch.scale, out=out,
                     partition_tokens=partition_tokens, workspace=workspace)


def decode_step_append(g: GpuBatch, out=None, partition_tokens=64, workspace=None) -> torch.Tensor:
    """The decode step's store and attention in one pa_decode_append call: a
    batch of decodes only, one new token per sequence (the step rows, in
    sequence order)."""
    b = g.batch
    new = np.asarray(b.new_lens)
    if b.is_chunk.any() or np.any(new > 1) or np.any((new == 0) & (np.asarray(b.total_lens) > 0)):
        raise ValueError("decode_step_append takes a batch of decodes with one new token each (or empty ones)")
    d = g.dec
    S, H, D = b.num_seqs, b.num_kv_heads, b.head_dim
    k_new, v_new = g.k_step.view(-1, H, D), g.v_step.view(-1, H, D)
    if np.any(new == 0):                               # empty sequences: rows that nothing stores
        idx = torch.from_numpy(np.flatnonzero(new == 1)).to(k_new.device)
        k_full = torch.zeros((S, H, D), dtype=k_new.dtype, device=k_new.device)
        v_full = torch.zeros_like(k_full)
        k_full[idx], v_full[idx] = k_new, v_new
        k_new, v_new = k_full, v_full
    return pa.decode_append(g.cache, k_new, v_new, d["q"], d["table"], d["lens"], d["max_len"], b.scale, out=out,
                            partition_tokens=partition_tokens, workspace=workspace)


def pack_args(g: GpuBatch, device="cuda") -> dict:
    """Device arguments of pa_pack_kv for every sequence's tokens (cached and
    stepped), in order."""
    lens = np.asarray(g.batch.total_lens, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    return dict(table=_t(_table_rows(g.tables, g.pad), device), lens=_t(lens.astype(np.int32), device),
                cu=_t(cu, device), max_len=int(lens.max(initial=0)), rows=int(lens.sum()))


def pack_all(g: GpuBatch, device="cuda", k_out=None, v_out=None, args=None):
    """pa_pack_kv of every sequence's tokens (cached and stepped), in order."""
    p = args if args is not None else pack_args(g, device)
    return pa.pack_kv(g.cache, p["table"], p["lens"], p["cu"], p["max_len"], p["rows"], k_out=k_out, v_out=v_out)


def all_slots(g: GpuBatch, device="cuda") -> torch.Tensor:
    """The slots of every sequence's tokens (cached, then stepped), in
    sequence order: where packed rows of the same batch land in g's cache."""
    pri, stp = g.prior_slots.cpu().numpy(), g.step_slots.cpu().numpy()
    out, pi, si = [], 0, 0
    for i in range(g.batch.num_seqs):
        p, n = int(g.batch.prior_lens[i]), int(g.batch.new_lens[i])
        out.append(np.concatenate([pri[pi:pi + p], stp[si:si + n]]))
        pi += p
        si += n
    return _t(np.concatenate(out).astype(np.int32), device)


def chunk_step(g: GpuBatch, out=None) -> torch.Tensor:
    c = g.chunk
    return pa.prefill_chunk(g.cache, c["q"], c["cu"], c["seq_lens"], c["table"], c["max_q"], c["max_seq"],
                            g.batch.scale, out=out)


@dataclass
class GpuFork:
    fb: object
    cache: pa.KVCache
    bm: pa.BlockManager
    beams: list
    pad: int
    copy_pairs: np.ndarray
    step_slots: np.ndarray   # [steps, beams]
    snap_before_divergence: Optional[torch.Tensor] = None


def run_fork(fb, device="cuda", snapshot=None) -> GpuFork:
    """Store the shared prompt, fork into beams, then append the beams' tokens
    one step at a time: each step's copy pairs are copied before its store.
    ``snapshot(cache, beams, bm)`` is called right after the fork."""
    bm = pa.BlockManager(fb.num_blocks, fb.block_size, fb.free_order)
    parent = bm.seq_new()
    shared = bm.append(parent, fb.shared_len)
    cache = pa.alloc_cache(fb.num_blocks, fb.num_kv_heads, fb.block_size, fb.head_dim, fb.kv_dtype,
                           device=device, k_scale=fb.k_scale, v_scale=fb.v_scale)
    pa.store_kv(cache, _t(fb.k_shared, device), _t(fb.v_shared, device), _t(shared.astype(np.int32), device))
    beams = [parent] + [bm.fork(parent) for _ in range(fb.beams - 1)]
    if snapshot is not None:
        snapshot(cache, beams, bm)
    pairs_all, slots_all = [], []
    kb = _t(fb.k_beam, device)
    vb = _t(fb.v_beam, device)
    for t in range(fb.steps):
        slots = np.array([bm.append(b, 1)[0] for b in beams], dtype=np.int32)
        pairs = bm.take_copies()
        if len(pairs):
            pa.copy_blocks(cache, _t(pairs.astype(np.int32), device))
        pa.store_kv(cache, kb[t], vb[t], _t(slots, device))
        pairs_all.append(pairs)
        slots_all.append(slots)
    return GpuFork(fb, cache, bm, beams, bm.unused_block(), np.concatenate(pairs_all).reshape(-1, 2),
                   np.stack(slots_all))


def fork_decode(gf: GpuFork, device="cuda", out=None, partition_tokens=64, workspace=None) -> torch.Tensor:
    bm = gf.bm
    table = _t(bm.block_tables(gf.beams, gf.pad), device)
    lens = np.array([bm.seq_len(b) for b in gf.beams], dtype=np.int32)
    return pa.decode(gf.cache, _t(gf.fb.q, device), table, _t(lens, device), int(lens.max()), gf.fb.scale,
                     out=out, partition_tokens=partition_tokens, workspace=workspace)


@dataclass
class PrefixTurn:
    active: list             # users taking part, in order
    hits: list               # tokens each found in the prefix cache
    tables: list             # block tables after the first reply token
    prefill_out: torch.Tensor
    decode_out: torch.Tensor


def run_prefix_agent(w, device="cuda"):
    """Multi-turn conversations through libpa's prefix cache.  Per turn: every
    active user starts from the longest cached prefix of its prompt, the rest
    of the prompt is stored and attended as one chunked prefill over the
    shared blocks, the first reply token is stored and decoded, the rest of
    the reply is stored, then the prompt and reply are recorded in the cache
    and the sequence is released.  Returns (cache, block manager, turns)."""
    bm = pa.BlockManager(w.num_blocks, w.block_size, w.free_order)
    bm.set_prefix_capacity(w.capacity_blocks)
    cache = pa.alloc_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.kv_dtype,
                           device=device, k_scale=w.k_scale, v_scale=w.v_scale)

    def store(parts, slots):
        k = np.concatenate([w.k_rows(u, lo, hi) for u, lo, hi in parts])
        v = np.concatenate([w.v_rows(u, lo, hi) for u, lo, hi in parts])
        pa.store_kv(cache, _t(k, device), _t(v, device), _t(np.concatenate(slots).astype(np.int32), device))

    turns = []
    for t in range(1, w.turns + 1):
        active = [u for u in range(w.users) if w.join_turn[u] <= t]
        seqs, hits, lens, slots = [], [], [], []
        for u in active:
            n = w.prompt_len(u, t)
            s = bm.seq_new_prefixed(w.ids(u, 0, n))
            hit = bm.seq_len(s)
            slots.append(bm.append(s, n - hit))
            seqs.append(s), hits.append(hit), lens.append(n)
        store([(u, h, n) for u, h, n in zip(active, hits, lens)], slots)
        q_lens = np.array([n - h for h, n in zip(hits, lens)])
        cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
        q = np.concatenate([w.q_rows(u, h, n) for u, h, n in zip(active, hits, lens)])
        table = bm.block_tables(seqs, bm.unused_block())
        out_p = pa.prefill_chunk(cache, _t(q, device), _t(cu, device), _t(np.array(lens, np.int32), device),
                                 _t(table, device), int(q_lens.max()), max(lens), w.scale).clone()
        store([(u, n, n + 1) for u, n in zip(active, lens)], [bm.append(s, 1) for s in seqs])
        table = bm.block_tables(seqs, bm.unused_block())
        ctx = np.array(lens, np.int32) + 1
        qd = np.stack([w.q_rows(u, n, n + 1)[0] for u, n in zip(active, lens)])
        out_d = pa.decode(cache, _t(qd, device), _t(table, device), _t(ctx, device), int(ctx.max()),
                          w.scale).clone()
        tables = [bm.block_table(s) for s in seqs]
        rest = w.reply_len - 1
        store([(u, n + 1, n + 1 + rest) for u, n in zip(active, lens)], [bm.append(s, rest) for s in seqs])
        for u, s, n in zip(active, seqs, lens):
            bm.prefix_insert(s, w.ids(u, 0, n + w.reply_len))
            bm.release(s)
        turns.append(PrefixTurn(active, hits, tables, out_p, out_d))
    return cache, bm, turns


@dataclass
class SpecBranchRun:
    cache: pa.KVCache
    bm: pa.BlockManager
    copy_pairs: np.ndarray
    branch_tables: list
    target_tables: list
    verify_out: torch.Tensor
    decode_out: torch.Tensor


def run_spec_branch(w, device="cuda") -> SpecBranchRun:
    """Speculative decoding over copy-on-write branches through libpa: store
    the targets' prefixes, fork one draft branch per target, append the
    drafts to the branches (their first append copies the shared tail: the
    queued pairs go to pa_copy_blocks before the drafts' pa_store_kv), verify
    the drafts with pa_prefill_chunk over the branches, append the accepted
    drafts to the targets and store them, release the branches, and decode
    the targets' next token."""
    bm = pa.BlockManager(w.num_blocks, w.block_size, w.free_order)
    S = len(w.prefix_lens)
    cache = pa.alloc_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.kv_dtype,
                           device=device, k_scale=w.k_scale, v_scale=w.v_scale)
    targets = [bm.seq_new() for _ in range(S)]
    slots = [bm.append(t, int(n)) for t, n in zip(targets, w.prefix_lens)]
    pa.store_kv(cache, _t(w.k_prefix, device), _t(w.v_prefix, device),
                _t(np.concatenate(slots).astype(np.int32), device))
    branches = [bm.fork(t) for t in targets]
    dslots = [bm.append(b, w.draft) for b in branches]
    pairs = bm.take_copies()
    if len(pairs):
        pa.copy_blocks(cache, _t(pairs.astype(np.int32), device))
    Hkv, d = w.num_kv_heads, w.head_dim
    pa.store_kv(cache, _t(w.k_draft.reshape(-1, Hkv, d), device), _t(w.v_draft.reshape(-1, Hkv, d), device),
                _t(np.concatenate(dslots).astype(np.int32), device))
    btables = [bm.block_table(b) for b in branches]
    cu = (np.arange(S + 1) * w.draft).astype(np.int32)
    lens = (w.prefix_lens + w.draft).astype(np.int32)
    verify = pa.prefill_chunk(cache, _t(w.q_verify, device), _t(cu, device), _t(lens, device),
                              _t(bm.block_tables(branches, bm.unused_block()), device), w.draft,
                              int(lens.max()), w.scale).clone()
    aslots = [bm.append(t, int(a)) for t, a in zip(targets, w.accepted)]
    if len(bm.take_copies()):
        raise RuntimeError("a target's tail was still shared after its branch copied it")
    rows = [(i, j) for i in range(S) for j in range(int(w.accepted[i]))]
    if rows:
        ii, jj = np.array(rows).T
        pa.store_kv(cache, _t(w.k_draft[ii, jj], device), _t(w.v_draft[ii, jj], device),
                    _t(np.concatenate(aslots).astype(np.int32), device))
    for b in branches:
        bm.release(b)
    ctx = (w.prefix_lens + w.accepted).astype(np.int32)
    dec = pa.decode(cache, _t(w.q_next, device), _t(bm.block_tables(targets, bm.unused_block()), device),
                    _t(ctx, device), int(ctx.max()), w.scale).clone()
    return SpecBranchRun(cache, bm, pairs, btables, [bm.block_table(t) for t in targets], verify, dec)
