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


@dataclass
class PrefixTurnRef:
    active: list
    hits: list
    tables: list
    prefill_out: np.ndarray
    decode_out: np.ndarray


def build_prefix_agent(w):
    """The oracle's run of the multi-turn prefix-cache conversations, in the
    same order of decisions as the library's runner: returns (K pool,
    V pool, manager, cache, turns)."""
    from oracle.prefix_cache import PrefixCache

    mgr = BlockManager(w.num_blocks, w.block_size, w.free_order)
    cache = PrefixCache(mgr, w.capacity_blocks)
    kc, vc = paged.new_pools(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.kv_dtype)

    def store(parts, slots):
        k = np.concatenate([w.k_rows(u, lo, hi) for u, lo, hi in parts])
        v = np.concatenate([w.v_rows(u, lo, hi) for u, lo, hi in parts])
        paged.store_kv(kc, vc, w.kv_dtype, k, v, w.io_dtype, np.concatenate(slots).astype(np.int64),
                       w.k_scale, w.v_scale)

    def pad():
        return next((b for b in range(w.num_blocks) if mgr.ref_count[b] == 0), 0)

    turns = []
    for t in range(1, w.turns + 1):
        active = [u for u in range(w.users) if w.join_turn[u] <= t]
        seqs, hits, lens, slots = [], [], [], []
        for u in active:
            n = w.prompt_len(u, t)
            s = cache.start(len(turns) * 100 + u, list(w.ids(u, 0, n)))
            hits.append(s.length)
            slots.append(s.append_slots(n - s.length))
            seqs.append(s), lens.append(n)
        store([(u, h, n) for u, h, n in zip(active, hits, lens)], slots)
        q_lens = np.array([n - h for h, n in zip(hits, lens)])
        cu = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int64)
        q = np.concatenate([w.q_rows(u, h, n) for u, h, n in zip(active, hits, lens)])
        out_p = paged.prefill_chunk_attention(kc, vc, w.kv_dtype, q, w.io_dtype, cu, np.array(lens),
                                              table_array([s.block_table for s in seqs], pad()), w.scale,
                                              w.k_scale, w.v_scale)
        store([(u, n, n + 1) for u, n in zip(active, lens)], [s.append_slots(1) for s in seqs])
        qd = np.stack([w.q_rows(u, n, n + 1)[0] for u, n in zip(active, lens)])
        out_d = paged.decode_attention(kc, vc, w.kv_dtype, qd, w.io_dtype,
                                       table_array([s.block_table for s in seqs], pad()),
                                       np.array(lens) + 1, w.scale, w.k_scale, w.v_scale)
        tables = [list(s.block_table) for s in seqs]
        rest = w.reply_len - 1
        store([(u, n + 1, n + 1 + rest) for u, n in zip(active, lens)], [s.append_slots(rest) for s in seqs])
        for u, s, n in zip(active, seqs, lens):
            cache.insert(list(w.ids(u, 0, n + w.reply_len)), s.block_table)
            s.release()
        turns.append(PrefixTurnRef(active, hits, tables, out_p, out_d))
    return kc, vc, mgr, cache, turns


@dataclass
class SpecBranchRef:
    kc: np.ndarray
    vc: np.ndarray
    copy_pairs: list       # pairs the branches' first appends recorded
    branch_tables: list    # branch block tables at verification
    target_tables: list    # target block tables after the accepted tokens
    ref_count: list
    used_blocks: int
    verify_out: np.ndarray
    decode_out: np.ndarray


def build_spec_branch(w) -> SpecBranchRef:
    """The oracle's run of speculative decoding over copy-on-write branches
    (nanoPD page, 分页KV缓存: copy on write serves speculative branches;
    serving-stack page section 7: the target checks the k draft tokens in one
    pass and keeps the accepted ones): store the targets' prefixes, fork a
    branch per target, append the drafts to the branches (copy pairs run
    before the drafts' store), verify over the branches, append the accepted
    drafts to the targets, release the branches, decode the targets."""
    mgr = BlockManager(w.num_blocks, w.block_size, w.free_order)
    S = len(w.prefix_lens)
    targets = [Sequence(mgr, i) for i in range(S)]
    kc, vc = paged.new_pools(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.kv_dtype)
    slots = [t.append_slots(int(n)) for t, n in zip(targets, w.prefix_lens)]
    paged.store_kv(kc, vc, w.kv_dtype, w.k_prefix, w.v_prefix, w.io_dtype,
                   np.concatenate(slots).astype(np.int64), w.k_scale, w.v_scale)
    branches = [t.fork(100 + i) for i, t in enumerate(targets)]
    dslots = [b.append_slots(w.draft) for b in branches]
    pairs = mgr.take_copies()
    paged.copy_blocks(kc, vc, pairs)
    paged.store_kv(kc, vc, w.kv_dtype, w.k_draft.reshape(-1, w.num_kv_heads, w.head_dim),
                   w.v_draft.reshape(-1, w.num_kv_heads, w.head_dim), w.io_dtype,
                   np.concatenate(dslots).astype(np.int64), w.k_scale, w.v_scale)
    held = {blk for s in targets + branches for blk in s.block_table}
    pad = next(b for b in range(w.num_blocks) if b not in held)
    cu = np.arange(S + 1, dtype=np.int64) * w.draft
    btables = [list(b.block_table) for b in branches]
    verify = paged.prefill_chunk_attention(kc, vc, w.kv_dtype, w.q_verify, w.io_dtype, cu,
                                           w.prefix_lens + w.draft, table_array(btables, pad), w.scale,
                                           w.k_scale, w.v_scale)
    aslots = [t.append_slots(int(a)) for t, a in zip(targets, w.accepted)]
    assert not mgr.take_copies()                 # the targets' tails are theirs alone now
    rows = [(i, j) for i in range(S) for j in range(int(w.accepted[i]))]
    if rows:
        ii, jj = np.array(rows).T
        paged.store_kv(kc, vc, w.kv_dtype, w.k_draft[ii, jj], w.v_draft[ii, jj], w.io_dtype,
                       np.concatenate(aslots).astype(np.int64), w.k_scale, w.v_scale)
    for b in branches:
        b.release()
    held = {blk for s in targets for blk in s.block_table}
    pad = next(b for b in range(w.num_blocks) if b not in held)
    ttables = [list(t.block_table) for t in targets]
    dec = paged.decode_attention(kc, vc, w.kv_dtype, w.q_next, w.io_dtype, table_array(ttables, pad),
                                 w.prefix_lens + w.accepted, w.scale, w.k_scale, w.v_scale)
    return SpecBranchRef(kc, vc, [tuple(p) for p in pairs], btables, ttables, list(mgr.ref_count),
                         mgr.used_blocks, verify, dec)
