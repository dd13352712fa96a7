"""Test helpers: lay a generated batch into oracle pools (CPU, oracle only).

Allocation order (both the oracle here and the library's own block manager
follow it): sequences in listed order, each taking slots for all of its
cached tokens and then for the tokens of the step.  Block-table rows are
padded with the id of a block that no sequence holds, so that a read past a
sequence's blocks meets NaN poison instead of another sequence's data.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from oracle import paged
from oracle.block_manager import BlockManager, Sequence


@dataclass
class OracleState:
    kc: np.ndarray
    vc: np.ndarray
    tables: list          # per sequence: list of block ids
    prior_slots: list     # per sequence: slots of its cached tokens
    step_slots: list      # per sequence: slots of the step's tokens
    pad_block: int
    mgr: BlockManager


def table_array(tables, pad, min_width=1):
    width = max([min_width] + [len(t) for t in tables])
    out = np.full((len(tables), width), pad, dtype=np.int32)
    for i, t in enumerate(tables):
        out[i, :len(t)] = t
    return out


def allocate(batch):
    mgr = BlockManager(batch.num_blocks, batch.block_size, batch.free_order)
    seqs = [Sequence(mgr, i) for i in range(batch.num_seqs)]
    prior, step = [], []
    for i, s in enumerate(seqs):
        prior.append(s.append_slots(int(batch.prior_lens[i])))
        step.append(s.append_slots(int(batch.new_lens[i])))
    held = {b for s in seqs for b in s.block_table}
    free = [b for b in range(batch.num_blocks) if b not in held]
    pad = free[0] if free else 0
    return mgr, [list(s.block_table) for s in seqs], prior, step, pad


def rows_of(batch, which):
    """Token rows [n, Hkv, d] of the cached ('prior') or new ('step') tokens, in
    sequence order, with their slots."""
    off = batch.tok_offsets
    idx = []
    for i in range(batch.num_seqs):
        a = int(off[i])
        p, n = int(batch.prior_lens[i]), int(batch.new_lens[i])
        idx.extend(range(a, a + p) if which == "prior" else range(a + p, a + p + n))
    idx = np.asarray(idx, dtype=np.int64)
    return batch.k[idx], batch.v[idx]


def build(batch) -> OracleState:
    mgr, tables, prior, step, pad = allocate(batch)
    kc, vc = paged.new_pools(batch.num_blocks, batch.num_kv_heads, batch.block_size,
                             batch.head_dim, batch.kv_dtype)
    kp, vp = rows_of(batch, "prior")
    paged.store_kv(kc, vc, batch.kv_dtype, kp, vp, batch.io_dtype, np.concatenate(prior + [[]]).astype(np.int64),
                   batch.k_scale, batch.v_scale)
    ks, vs = rows_of(batch, "step")
    paged.store_kv(kc, vc, batch.kv_dtype, ks, vs, batch.io_dtype, np.concatenate(step + [[]]).astype(np.int64),
                   batch.k_scale, batch.v_scale)
    return OracleState(kc, vc, tables, prior, step, pad, mgr)


def decode_ref(batch, st: OracleState):
    dec = np.flatnonzero(~batch.is_chunk)
    tables = table_array([st.tables[i] for i in dec], st.pad_block)
    lens = batch.total_lens[dec]
    return paged.decode_attention(st.kc, st.vc, batch.kv_dtype, batch.q_decode, batch.io_dtype, tables,
                                  lens, batch.scale, batch.k_scale, batch.v_scale)


def chunk_ref(batch, st: OracleState):
    ch = np.flatnonzero(batch.is_chunk)
    tables = table_array([st.tables[i] for i in ch], st.pad_block)
    q_lens = batch.new_lens[ch]
    cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
    return paged.prefill_chunk_attention(st.kc, st.vc, batch.kv_dtype, batch.q_chunk, batch.io_dtype, cu,
                                         batch.total_lens[ch], tables, batch.scale, batch.k_scale,
                                         batch.v_scale)


@dataclass
class ForkState:
    kc: np.ndarray
    vc: np.ndarray
    beams: list
    copy_pairs: list       # all (src, dst) pairs, in the order recorded
    step_slots: list       # per step: slots of the beams' tokens, beam order
    pad_block: int
    mgr: BlockManager


def build_fork(fb, check_before_divergence=None) -> ForkState:
    """Store the shared prompt, fork, then append the beams' tokens one step at
    a time (copy pairs of a step are carried out before that step's store)."""
    mgr = BlockManager(fb.num_blocks, fb.block_size, fb.free_order)
    parent = Sequence(mgr, 0)
    shared_slots = parent.append_slots(fb.shared_len)
    kc, vc = paged.new_pools(fb.num_blocks, fb.num_kv_heads, fb.block_size, fb.head_dim, fb.kv_dtype)
    paged.store_kv(kc, vc, fb.kv_dtype, fb.k_shared, fb.v_shared, fb.io_dtype, np.asarray(shared_slots),
                   fb.k_scale, fb.v_scale)
    beams = [parent] + [parent.fork(i + 1) for i in range(fb.beams - 1)]
    if check_before_divergence is not None:
        check_before_divergence(kc, vc, beams)
    pairs_all, slots_all = [], []
    for t in range(fb.steps):
        slots = [b.append_slot() for b in beams]
        pairs = mgr.take_copies()
        paged.copy_blocks(kc, vc, pairs)
        paged.store_kv(kc, vc, fb.kv_dtype, fb.k_beam[t], fb.v_beam[t], fb.io_dtype, np.asarray(slots),
                       fb.k_scale, fb.v_scale)
        pairs_all.extend(pairs)
        slots_all.append(slots)
    held = {b for s in beams for b in s.block_table}
    free = [b for b in range(fb.num_blocks) if b not in held]
    return ForkState(kc, vc, beams, pairs_all, slots_all, free[0] if free else 0, mgr)


def fork_decode_ref(fb, st: ForkState):
    tables = table_array([b.block_table for b in st.beams], st.pad_block)
    lens = np.array([b.length for b in st.beams])
    return paged.decode_attention(st.kc, st.vc, fb.kv_dtype, fb.q, fb.io_dtype, tables, lens, fb.scale,
                                  fb.k_scale, fb.v_scale)
