"""Prefix cache over a BlockManager (oracle; test infrastructure only).

Written from the serving-stack page (chenxutan.com), section 4 (前缀缓存),
4.2 (the hash-chain route) and 4.3 (its minimal form):

* the unit is a full block of ``block_size`` token ids; a block's key chains
  its parent's key with the block's own ids, so one key names a whole prefix
  path, and equal keys mean equal prefixes;
* finding the longest cached prefix walks the prompt's full blocks from the
  front and stops at the first block not in the cache: after a break in the
  chain nothing further can match;
* ``insert`` records the blocks of a computed prefix; when the cache holds
  ``capacity_blocks`` entries, the least recently used entry goes; a lookup
  hit and an insert both count as a use;
* a lookup with any hit counts as a hit, else as a miss.

Readings taken here (the page's listing leaves them open):

* ``insert`` takes the token ids a sequence has computed and its block
  table, and records every full block of them.  The page's lookup returns
  the chain only up to its first miss, so inserting that chain as printed
  would add one new block per request; recording every full block is the
  reading under which the page's multi-turn example reaches the hit rates
  the page reports for it (above 90% from the second turn on, when each
  turn's computed tokens, its generated reply included, are recorded);
* the page hashes (parent, ids, extra) into a 32-hex-digit SHA-256 prefix;
  here a key is the exact pair (parent key, ids of the block), interned to
  a small integer: the same chain with no collisions.  The extra field
  (multimodal inputs) is not modelled;
* the cache holds one reference of its own on every cached block (through
  the block manager), so a cached block outlives the sequence that computed
  it; evicting an entry drops that reference, freeing the block when no
  sequence holds it;
* a sequence that starts from a cached prefix shares those blocks (one more
  reference each) and has the prefix's length; its next token opens a new
  block, since a cached prefix is whole blocks.
"""
from __future__ import annotations

from collections import OrderedDict
from typing import Dict, List, Sequence as Seq, Tuple

from .block_manager import BlockManager, Sequence


class PrefixCache:
    def __init__(self, mgr: BlockManager, capacity_blocks: int):
        if capacity_blocks <= 0:
            raise ValueError("capacity_blocks must be positive")
        self.mgr = mgr
        self.capacity = int(capacity_blocks)
        self._key_ids: Dict[Tuple[int, Tuple[int, ...]], int] = {}   # (parent key, ids) -> key
        self.table: Dict[int, int] = {}                               # key -> physical block
        self.lru: "OrderedDict[int, None]" = OrderedDict()            # keys, least recent first
        self.hits = 0
        self.misses = 0

    def _key(self, parent: int, ids: Seq[int], create: bool) -> int:
        k = (parent, tuple(int(x) for x in ids))
        key = self._key_ids.get(k, -1)
        if key < 0 and create:
            key = len(self._key_ids)
            self._key_ids[k] = key
        return key

    def _touch(self, key: int) -> None:
        self.lru.pop(key, None)
        self.lru[key] = None

    def lookup(self, token_ids: Seq[int]) -> Tuple[int, List[int]]:
        """(tokens covered by the longest cached prefix, its physical blocks)."""
        B = self.mgr.block_size
        parent, blocks = -1, []
        for i in range(0, len(token_ids) - B + 1, B):
            key = self._key(parent, token_ids[i:i + B], create=False)
            if key < 0 or key not in self.table:
                break
            blocks.append(self.table[key])
            self._touch(key)
            parent = key
        if blocks:
            self.hits += 1
        else:
            self.misses += 1
        return len(blocks) * B, blocks

    def insert(self, token_ids: Seq[int], block_ids: Seq[int]) -> int:
        """Record the full blocks of token_ids, held in block_ids (a block
        table); returns how many entries were added."""
        B = self.mgr.block_size
        parent, added = -1, 0
        for j, i in enumerate(range(0, len(token_ids) - B + 1, B)):
            key = self._key(parent, token_ids[i:i + B], create=True)
            if key not in self.table:
                if len(self.table) >= self.capacity:
                    victim, _ = self.lru.popitem(last=False)
                    self.mgr.free(self.table.pop(victim))
                self.table[key] = int(block_ids[j])
                self.mgr.incref(int(block_ids[j]))
                added += 1
            self._touch(key)
            parent = key
        return added

    @property
    def hit_rate(self) -> float:
        n = self.hits + self.misses
        return self.hits / n if n else 0.0

    def start(self, seq_id: int, token_ids: Seq[int]) -> Sequence:
        """A new sequence holding the longest cached prefix of token_ids."""
        hit, blocks = self.lookup(token_ids)
        s = Sequence(self.mgr, seq_id)
        for b in blocks:
            self.mgr.incref(b)
        s.block_table = list(blocks)
        s.length = hit
        return s
