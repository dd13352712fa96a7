"""Pins for the oracle's host block manager (CPU only).

Fork demo of the serving-stack page (chenxutan.com), section 2.3: a pool of
64 blocks of 16 tokens, a 100-token prompt, 4 forks, then one more token in
each child.  The page prints no numbers; it states that forking leaves the
usage (almost) unchanged and that only the last block is copied on write.
Traced by hand from the page's rules:

* 100 tokens fill ceil(100/16) = 7 blocks -> usage 7/64;
* forking adds references, not blocks -> still 7/64, every block count 5;
* each child's append lands at offset 100 % 16 = 4 of the shared tail block;
  every child finds that block shared and copies it (its count drops
  5 -> 4 -> 3 -> 2 -> 1, and the parent keeps the original)
  -> 7 + 4 = 11 blocks, usage 11/64.
"""
import random

import numpy as np
import pytest

from oracle.block_manager import BlockManager, Sequence


def test_fork_demo_traced_counts():
    mgr = BlockManager(64, 16)
    s = Sequence(mgr, 0)
    s.append_slots(100)
    assert len(s.block_table) == 7 and mgr.used_blocks == 7
    assert mgr.usage == pytest.approx(7 / 64)
    before = mgr.usage
    kids = [s.fork(i + 1) for i in range(4)]
    assert mgr.usage == before                   # the page: usage barely changes
    assert all(mgr.ref_count[b] == 5 for b in s.block_table)
    tail = s.block_table[-1]
    for k in kids:
        k.append_slot()
    assert mgr.used_blocks == 11 and mgr.usage == pytest.approx(11 / 64)
    pairs = mgr.take_copies()
    assert [p[0] for p in pairs] == [tail] * 4     # only the tail block is copied
    assert len({p[1] for p in pairs}) == 4
    assert mgr.ref_count[tail] == 1 and s.block_table[-1] == tail
    for k in kids:                                 # children share the 6 full blocks
        assert k.block_table[:6] == s.block_table[:6]
        assert k.block_table[6] != tail


def test_exhaustion_returns_none_and_cow_raises():
    mgr = BlockManager(2, 4)
    a = Sequence(mgr, 0)
    a.append_slots(5)                 # 2 blocks, second holds 1 token
    assert mgr.allocate() is None
    b = a.fork(1)
    with pytest.raises(MemoryError):
        b.append_slot()               # shared tail, no free block to copy into
    with pytest.raises(MemoryError):
        Sequence(mgr, 2).append_slot()


def test_fork_and_release_refuse_while_copies_are_queued():
    """Append (a CoW of a shared tail), fork, append again: with the first
    pair still queued, the second append would copy out of the first pair's
    destination (a chain), and the parent's new token would be copied before
    it is stored.  Fork and release refuse until the pairs are taken; after
    that the same trace queues one plain pair per step."""
    mgr = BlockManager(16, 4)
    a = Sequence(mgr, 0)
    a.append_slots(2)
    b = a.fork(1)                         # tail (2 tokens) shared, count 2
    a.append_slot()                       # CoW: a takes a copy of the tail
    assert len(mgr.pending_copies) == 1
    with pytest.raises(RuntimeError):
        a.fork(2)
    with pytest.raises(RuntimeError):
        b.release()
    (src, dst), = mgr.take_copies()
    c = a.fork(2)                         # a's new tail (dst) is shared now
    assert mgr.ref_count[dst] == 2
    a.append_slot()                       # a copies dst on write: one pair, no chain
    (src2, dst2), = mgr.take_copies()
    assert src2 == dst and dst2 not in (src, dst)
    assert c.block_table[-1] == dst and a.block_table[-1] == dst2
    b.release()
    assert mgr.ref_count[src] == 0


def test_free_list_order_and_release():
    mgr = BlockManager(5, 4, free_order=[3, 1, 4, 0, 2])
    s = Sequence(mgr, 0)
    s.append_slots(9)                 # pops from the end of the list: 2, 0, 4
    assert s.block_table == [2, 0, 4]
    s.release()
    assert mgr.used_blocks == 0 and mgr.free_ids[-3:] == [2, 0, 4]


def test_slots_are_block_times_size_plus_offset():
    mgr = BlockManager(8, 16, free_order=[5, 7, 1, 0, 2, 3, 4, 6])
    s = Sequence(mgr, 0)
    slots = s.append_slots(40)
    assert slots[:16] == list(range(6 * 16, 7 * 16))
    assert slots[16:32] == list(range(4 * 16, 5 * 16))
    assert slots[32:] == list(range(3 * 16, 3 * 16 + 8))


def _simulate(seed, steps=400, pool=48, B=4):
    """Random fork / append / release traffic; the content of every block is
    tracked token by token, copies applied as recorded.  Returns False as soon
    as some sequence would read back a token other than its own."""
    rng = random.Random(seed)
    mgr = BlockManager(pool, B, free_order=np.random.default_rng(seed).permutation(pool))
    content = {}                      # (block, offset) -> token label
    seqs = {0: (Sequence(mgr, 0), [])}
    next_id, label = 1, 0
    for _ in range(steps):
        op = rng.random()
        sid = rng.choice(list(seqs))
        seq, toks = seqs[sid]
        try:
            if op < 0.6:
                slot = seq.append_slot()
                for src, dst in mgr.take_copies():
                    for o in range(B):
                        if (src, o) in content:
                            content[(dst, o)] = content[(src, o)]
                content[divmod(slot, B)] = label
                toks.append(label)
                label += 1
            elif op < 0.8 and len(seqs) < 10:
                child = seq.fork(next_id)
                seqs[next_id] = (child, list(toks))
                next_id += 1
            elif op < 0.9 and len(seqs) > 1:
                seq.release()
                del seqs[sid]
        except MemoryError:
            mgr.take_copies()
            seq.release()
            del seqs[sid]
            if not seqs:
                seqs[next_id] = (Sequence(mgr, next_id), [])
                next_id += 1
        for s2, t2 in seqs.values():
            got = [content.get((s2.block_table[i // B], i % B)) for i in range(s2.length)]
            if got != t2:
                return False
            # internal fragmentation: at most B-1 unused slots per sequence
            if len(s2.block_table) * B - s2.length > B - 1:
                return False
        held = sum(mgr.ref_count)
        if held != sum(len(s2.block_table) for s2, _ in seqs.values()):
            return False
    return True


@pytest.mark.parametrize("seed", range(12))
def test_random_fork_append_release_keeps_every_sequence_readable(seed):
    assert _simulate(seed)


def test_a_missing_copy_would_be_caught():
    """Plant a mistake (CoW that writes in place) and check that the simulated
    token trace notices it."""
    orig = BlockManager.cow
    try:
        BlockManager.cow = lambda self, bid: bid
        assert not all(_simulate(s) for s in range(12))
    finally:
        BlockManager.cow = orig
