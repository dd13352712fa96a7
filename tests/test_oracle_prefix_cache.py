"""Pins for the oracle's prefix cache (CPU only).

Multi-turn agent example of the serving-stack page (chenxutan.com),
section 4.3: blocks of 16 tokens, a fixed 1000-token system prompt, per turn
a 60-token user message appended to the whole history, then a 120-token
reply; 7 turns, capacity 4096 blocks.  The page states that from the second
turn on more than 90% of each prompt is a cache hit and that the share grows
with the conversation; it prints no per-turn numbers.  Closed forms used
here, from the chain rule (a hit covers whole blocks, up to the first block
that was never recorded):

* prompt_t = 1060 + 180 (t - 1) tokens;
* recording each turn's prompt only: hit_t = 16 floor(|prompt_(t-1)| / 16);
* recording the prompt and its reply: hit_t = 16 floor((|prompt_(t-1)| + 120) / 16).

Section 4.4, rule 1: a value that changes per request at the very front
(a timestamp) changes the first block's key, so nothing ever hits.

A second, independent formulation (a dict keyed by the whole prefix up to
the end of each block, with the same LRU policy) must take the same
decisions on random traces: chain keys name exactly the prefix they end.
"""
import random
from collections import OrderedDict

import numpy as np
import pytest

from oracle.block_manager import BlockManager
from oracle.prefix_cache import PrefixCache

B = 16


def _agent(turns=7, record_reply=False, stamp=False):
    mgr = BlockManager(4096, B)
    cache = PrefixCache(mgr, 4096)
    history = list(range(1000))
    out = []
    for t in range(1, turns + 1):
        user = list(range(90000 + t * 100, 90000 + t * 100 + 60))
        prompt = ([700000 + t] if stamp else []) + history + user
        seq = cache.start(t, prompt)
        hit = seq.length
        seq.append_slots(len(prompt) - hit)
        reply = list(range(80000 + t * 50, 80000 + t * 50 + 120))
        if record_reply:
            seq.append_slots(len(reply))
            cache.insert(prompt + reply, seq.block_table)
        else:
            cache.insert(prompt, seq.block_table)
        out.append((len(prompt), hit))
        seq.release()
        history = history + user + reply
    return out, cache, mgr


def test_agent_prompt_only_closed_form():
    rows, cache, _ = _agent()
    for t, (n, hit) in enumerate(rows, start=1):
        assert n == 1060 + 180 * (t - 1)
        want = 0 if t == 1 else B * ((1060 + 180 * (t - 2)) // B)
        assert hit == want, (t, hit, want)
    assert (cache.hits, cache.misses) == (6, 1)


def test_agent_with_replies_reaches_the_pages_hit_rate():
    rows, cache, _ = _agent(record_reply=True)
    rates = []
    for t, (n, hit) in enumerate(rows, start=1):
        want = 0 if t == 1 else B * ((1060 + 180 * (t - 2) + 120) // B)
        assert hit == want, (t, hit, want)
        rates.append(hit / n)
    assert rates[0] == 0
    assert all(r > 0.9 for r in rates[1:])
    assert all(a < b for a, b in zip(rates[1:], rates[2:]))
    assert cache.hit_rate == pytest.approx(6 / 7)


def test_a_changing_first_token_means_no_hits():
    rows, cache, _ = _agent(stamp=True)
    assert all(hit == 0 for _, hit in rows)
    assert (cache.hits, cache.misses, cache.hit_rate) == (0, 7, 0.0)


def test_cached_blocks_outlive_their_sequence_and_are_shared():
    rows, cache, mgr = _agent(record_reply=True)
    # Nothing but the cache holds blocks now: every cached block has count 1.
    assert sorted(cache.table.values()) == sorted(b for b in range(mgr.num_blocks) if mgr.ref_count[b])
    assert all(mgr.ref_count[b] == 1 for b in cache.table.values())
    prompt = list(range(1000)) + list(range(90100, 90160))
    a, b = cache.start(100, prompt), cache.start(101, prompt)
    assert a.block_table == b.block_table and a.length == b.length == B * (1060 // B)
    assert all(mgr.ref_count[x] == 3 for x in a.block_table)
    # The next token of each opens a private block: the shared ones are full.
    sa, sb = a.append_slot(), b.append_slot()
    assert sa // B != sb // B and sa % B == 0 and sb % B == 0
    assert mgr.take_copies() == []


def test_a_break_stops_the_walk_even_if_later_blocks_match():
    mgr = BlockManager(64, B)
    cache = PrefixCache(mgr, 64)
    toks = list(range(5 * B))
    s = cache.start(0, toks)
    s.append_slots(len(toks))
    assert cache.insert(toks, s.block_table) == 5 and len(cache.table) == 5
    assert cache.insert(toks, s.block_table) == 0
    probe = list(toks)
    probe[2 * B + 3] = -1                       # third block differs
    hit, blocks = cache.lookup(probe)
    assert hit == 2 * B and blocks == s.block_table[:2]
    # Blocks 4 and 5 of probe equal cached ones, but their parent key differs.
    hit, _ = cache.lookup(toks[:B] + toks[3 * B:])
    assert hit == B
    # A missing block is not skipped: with [b0, b2] cached as a chain too,
    # [b0, x, b2] still hits b0 only.
    other = toks[:B] + toks[2 * B:3 * B]
    s2 = cache.start(1, other)
    s2.append_slots(len(other) - s2.length)
    cache.insert(other, s2.block_table)
    assert cache.lookup(other)[0] == 2 * B
    hit, _ = cache.lookup(toks[:B] + [-5] * B + toks[2 * B:3 * B])
    assert hit == B
    # A partial last block is never a hit.
    hit, _ = cache.lookup(toks[:3 * B - 1])
    assert hit == 2 * B


def test_lru_eviction_order_and_freeing():
    mgr = BlockManager(16, B)
    cache = PrefixCache(mgr, 3)
    A = list(range(2 * B))
    C_ = list(range(1000, 1000 + B))
    D = list(range(2000, 2000 + B))
    E = list(range(3000, 3000 + B))
    seqs = {}
    for name, toks in (("A", A), ("C", C_)):
        s = cache.start(len(seqs), toks)
        s.append_slots(len(toks))
        cache.insert(toks, s.block_table)
        seqs[name] = s
    assert len(cache.table) == 3
    assert cache.lookup(A)[0] == 2 * B            # A's two blocks now most recent
    s = cache.start(9, D)
    s.append_slots(B)
    cache.insert(D, s.block_table)                # evicts C (least recent)
    assert cache.lookup(C_)[0] == 0 and cache.lookup(A)[0] == 2 * B
    assert cache.lookup(D)[0] == B
    cblock = seqs["C"].block_table[0]
    assert mgr.ref_count[cblock] == 1             # only C's sequence holds it now
    seqs["C"].release()
    assert mgr.ref_count[cblock] == 0 and cblock in mgr.free_ids
    s2 = cache.start(10, E)
    s2.append_slots(B)
    cache.insert(E, s2.block_table)               # evicts A's first block
    assert cache.lookup(A)[0] == 0                # the chain lost its front
    assert cache.lookup(D)[0] == B and cache.lookup(E)[0] == B


class _PrefixDict:
    """Same policy, keyed by the whole prefix up to each block's end."""

    def __init__(self, capacity):
        self.capacity = capacity
        self.table = OrderedDict()   # prefix tuple -> block, least recent first
        self.hits = self.misses = 0

    def lookup(self, toks):
        blocks = []
        for end in range(B, len(toks) + 1, B):
            k = tuple(toks[:end])
            if k not in self.table:
                break
            blocks.append(self.table[k])
            self.table.move_to_end(k)
        if blocks:
            self.hits += 1
        else:
            self.misses += 1
        return len(blocks) * B, blocks

    def insert(self, toks, table):
        for j, end in enumerate(range(B, len(toks) + 1, B)):
            k = tuple(toks[:end])
            if k not in self.table:
                if len(self.table) >= self.capacity:
                    self.table.popitem(last=False)
                self.table[k] = table[j]
            self.table.move_to_end(k)


@pytest.mark.parametrize("seed", range(6))
def test_chain_keys_equal_whole_prefix_keys_on_random_traces(seed):
    rng = random.Random(seed)
    mgr = BlockManager(400, B)
    cache = PrefixCache(mgr, rng.choice([4, 9, 30]))
    ref = _PrefixDict(cache.capacity)
    stems = [[rng.randrange(5) for _ in range(rng.randint(0, 90))] for _ in range(4)]
    live = []
    for step in range(150):
        toks = list(rng.choice(stems)) + [rng.randrange(3) for _ in range(rng.randint(0, 40))]
        hit_ref = ref.lookup(toks)
        s = cache.start(step, toks)
        assert (s.length, s.block_table) == hit_ref
        s.append_slots(len(toks) - s.length)
        ref.insert(toks, s.block_table)
        cache.insert(toks, s.block_table)
        assert sorted(cache.table.values()) == sorted(ref.table.values())
        live.append(s)
        if len(live) > 6:
            live.pop(rng.randrange(len(live))).release()
    assert (cache.hits, cache.misses) == (ref.hits, ref.misses)
    for s in live:
        s.release()
    # Only the cache holds blocks now: exactly one reference per cached entry.
    held = [b for b in range(mgr.num_blocks) if mgr.ref_count[b]]
    assert sorted(held) == sorted(set(cache.table.values()))
    assert all(mgr.ref_count[b] == list(cache.table.values()).count(b) for b in held)


def _dense(q, k, v, scale):
    """softmax(scale q k^T) v for one head over logical rows (fp64)."""
    s = scale * (k @ q)
    p = np.exp(s - s.max())
    return (p @ v) / p.sum()


def _f64(bits):
    from oracle.paged import values_f64
    return values_f64(bits, "bf16")


def test_agent_conversations_reuse_exact_kv():
    """The paged run of the shared-prefix conversations (the same run the GPU
    parity test mirrors) against the closed-form hits and against attention
    over each user's logical K/V rows, read without any block table."""
    import workloads as W
    from tests.oracle_setup import build_prefix_agent

    w = W.prefix_agent(small=True)
    kc, vc, mgr, cache, turns = build_prefix_agent(w)
    sys_blocks = w.sys_len // B
    for t, tr in enumerate(turns, start=1):
        for u, hit, table in zip(tr.active, tr.hits, tr.tables):
            tau = w.local_turn(u, t)
            if tau == 1:
                want = 0 if t == 1 else B * sys_blocks
            else:
                want = B * ((w.sys_len + (tau - 1) * w.turn_len) // B)
            assert hit == want, (t, u, hit, want)
        if t >= 2:   # everyone reads the one copy of the system prompt
            heads = {tuple(tb[:sys_blocks]) for tb in tr.tables}
            assert len(heads) == 1
        G = w.num_q_heads // w.num_kv_heads
        for i, u in enumerate(tr.active):
            n = w.prompt_len(u, t)
            k = _f64(w.k_rows(u, 0, n + 1))
            v = _f64(w.v_rows(u, 0, n + 1))
            q = _f64(w.q_rows(u, n, n + 1))[0]
            for h in range(w.num_q_heads):
                g = h // G
                ref = _dense(q[h], k[:, g], v[:, g], w.scale)
                assert np.allclose(tr.decode_out[i, h], ref, rtol=0, atol=1e-12)
    # Afterwards only the cache holds blocks, one reference per entry.
    held = [b for b in range(w.num_blocks) if mgr.ref_count[b]]
    assert sorted(held) == sorted(cache.table.values())
