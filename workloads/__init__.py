"""Seeded synthetic inputs for paged attention (shared by the tests, the bench
and the oracle's timing leg).

This module draws random numbers and lays out plain arrays.  It holds none of
the method's arithmetic: no slot or block-table computation, no attention,
no fp8 encoding.  Block tables and slots are produced by a block manager
(the oracle's or the library's own) from the ``free_order`` and lengths
drawn here.

Recipe (every draw from ``numpy.random.default_rng(seed)``, PCG64, in this
order): sequence lengths -> pool permutation (the block manager's initial
free list) -> K values -> V values -> Q values, all N(0, 1) float32, then a
round-to-nearest-even cast to bf16 where the config is bf16 (torch's CPU
cast).  K and V are drawn for every token of every sequence in the order
the sequences are listed, tokens in logical order; fp8 configs pass K and V
to the store as bf16 and quantise there with per-kv-head scales
``amax(|x|) / 448`` taken over that head's bf16 values (fp32).

The shapes follow one Qwen3-8B attention layer (32 query heads, 8 kv heads,
head_dim 128); nothing here depends on model weights.
"""
from __future__ import annotations

import copy
import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

E4M3_MAX = 448.0


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even (torch cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass
class PagedBatch:
    """One step over a batch of sequences sharing one paged pool.

    Sequence i already holds ``prior_lens[i]`` cached tokens and stores
    ``new_lens[i]`` more during the step.  Decode sequences (``is_chunk``
    False) store one token and ask one query; chunk sequences store a chunk
    of ``new_lens[i]`` tokens whose rows are all queries.
    """
    name: str
    seed: int
    kv_dtype: str            # "f32" | "bf16" | "fp8"   (cache storage)
    io_dtype: str            # "f32" | "bf16"           (q / out / new K,V)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray   # int64 [num_blocks]
    prior_lens: np.ndarray   # int64 [S]
    new_lens: np.ndarray     # int64 [S]
    is_chunk: np.ndarray     # bool  [S]
    k: np.ndarray            # [sum(prior+new), Hkv, d]  io_dtype storage
    v: np.ndarray
    q_decode: np.ndarray     # [n_decode, Hq, d]          io_dtype storage
    q_chunk: np.ndarray      # [sum new of chunk seqs, Hq, d]
    k_scale: Optional[np.ndarray] = None   # float32 [Hkv] (fp8 only)
    v_scale: Optional[np.ndarray] = None
    scale: float = 0.0
    partition_tokens: int = 512
    notes: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.prior_lens)

    @property
    def tok_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.prior_lens + self.new_lens)]).astype(np.int64)

    @property
    def total_lens(self) -> np.ndarray:
        return (self.prior_lens + self.new_lens).astype(np.int64)


@dataclass
class ForkBatch:
    """A shared prompt forked into beams that then diverge token by token."""
    name: str
    seed: int
    kv_dtype: str
    io_dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray
    shared_len: int          # tokens in the sequence at the moment of the fork
    beams: int               # sequences after the fork (parent included)
    steps: int               # divergent tokens appended per beam
    k_shared: np.ndarray     # [shared_len, Hkv, d]
    v_shared: np.ndarray
    k_beam: np.ndarray       # [steps, beams, Hkv, d]
    v_beam: np.ndarray
    q: np.ndarray            # [beams, Hq, d]
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    scale: float = 0.0
    partition_tokens: int = 512


def _values(rng, shape, io_dtype):
    x = rng.standard_normal(shape, dtype=np.float32)
    return to_bf16_bits(x) if io_dtype == "bf16" else x


def _pool_size(total_lens, block_size, factor=1.25):
    need = int(sum(math.ceil(int(L) / block_size) for L in total_lens))
    return max(1, int(math.ceil(factor * need)))


def _head_scales(k_bits, v_bits):
    """Per-kv-head fp32 scale amax/448 over that head's bf16 values."""
    kf = np.abs(bf16_bits_to_f32(k_bits)).reshape(-1, k_bits.shape[-2], k_bits.shape[-1])
    vf = np.abs(bf16_bits_to_f32(v_bits)).reshape(-1, v_bits.shape[-2], v_bits.shape[-1])
    ks = (kf.max(axis=(0, 2)) / np.float32(E4M3_MAX)).astype(np.float32)
    vs = (vf.max(axis=(0, 2)) / np.float32(E4M3_MAX)).astype(np.float32)
    return ks, vs


def paged_batch(name, seed, *, kv_dtype, io_dtype, Hq, Hkv, d, B, prior_lens, new_lens, is_chunk,
                rng, pool=None, pool_factor=1.25, partition_tokens=512) -> PagedBatch:
    prior_lens = np.asarray(prior_lens, dtype=np.int64)
    new_lens = np.asarray(new_lens, dtype=np.int64)
    is_chunk = np.asarray(is_chunk, dtype=bool)
    total = prior_lens + new_lens
    nb = pool if pool is not None else _pool_size(total, B, pool_factor)
    free_order = rng.permutation(nb).astype(np.int64)
    N = int(total.sum())
    k = _values(rng, (N, Hkv, d), io_dtype)
    v = _values(rng, (N, Hkv, d), io_dtype)
    n_dec = int((~is_chunk).sum())
    n_chunk_rows = int(new_lens[is_chunk].sum())
    q_decode = _values(rng, (n_dec, Hq, d), io_dtype)
    q_chunk = _values(rng, (n_chunk_rows, Hq, d), io_dtype)
    ks = vs = None
    if kv_dtype == "fp8":
        ks, vs = _head_scales(k, v)
    scale = float(np.float32(1.0 / math.sqrt(d)))
    return PagedBatch(name, seed, kv_dtype, io_dtype, Hq, Hkv, d, B, nb, free_order,
                      prior_lens, new_lens, is_chunk, k, v, q_decode, q_chunk, ks, vs, scale,
                      partition_tokens)


# ----------------------------------------------------------------- configs
def config1(small=False) -> PagedBatch:
    """Tiny fp32 decode: lens {17,33,64,100}, Hq 4 / Hkv 2, d 64, B 16, pool 64."""
    rng = np.random.default_rng(1)
    lens = np.array([17, 33, 64, 100])
    return paged_batch("tiny-fp32-decode", 1, kv_dtype="f32", io_dtype="f32", Hq=4, Hkv=2, d=64, B=16,
                       prior_lens=lens - 1, new_lens=np.ones(4, np.int64), is_chunk=np.zeros(4, bool),
                       rng=rng, pool=64)


def config2(small=False) -> PagedBatch:
    """Qwen3-8B decode layer: 32 seqs, L ~ U{512..4096}, bf16, B 16, pool 1.25x."""
    seed = 2 if not small else 102
    rng = np.random.default_rng(seed)
    if small:
        lens = rng.integers(1, 1400, size=6)
    else:
        lens = rng.integers(512, 4097, size=32)
    return paged_batch("qwen3-8b-decode-32seq" if not small else "qwen3-8b-decode-small", seed,
                       kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                       prior_lens=lens - 1, new_lens=np.ones(len(lens), np.int64),
                       is_chunk=np.zeros(len(lens), bool), rng=rng)


def config3_lengths() -> np.ndarray:
    """The 128 context lengths of the long-context config (its first draw)."""
    rng = np.random.default_rng(3)
    return np.round(np.exp(rng.uniform(np.log(128), np.log(32768), size=128))).astype(np.int64)


def config3_sample(n=24, seed=303) -> PagedBatch:
    """A bounded sample of the long-context config for timing the oracle on
    the host: its first n context lengths, fresh K/V/Q values of the same
    distribution (seed 303), bf16, B 16, pool 1.25x."""
    lens = config3_lengths()[:n]
    rng = np.random.default_rng(seed)
    return paged_batch("long-context-decode-sample", seed, kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8,
                       d=128, B=16, prior_lens=lens - 1, new_lens=np.ones(n, np.int64),
                       is_chunk=np.zeros(n, bool), rng=rng)


def store_sample(tokens=16384, seqs=8, seed=304) -> PagedBatch:
    """A bulk-store sample of the long-context shape for timing the oracle's
    store on the host: ``seqs`` sequences of tokens / seqs new tokens each
    (no cached prefix), bf16, Qwen3-8B heads, B 16, pool 1.25x."""
    rng = np.random.default_rng(seed)
    n = tokens // seqs
    return paged_batch("bulk-store-sample", seed, kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                       prior_lens=np.zeros(seqs, np.int64), new_lens=np.full(seqs, n, np.int64),
                       is_chunk=np.zeros(seqs, bool), rng=rng)


def config3(block_size=16, small=False) -> PagedBatch:
    """Long-context decode: 128 seqs, L log-uniform [128, 32768], bf16, split-K 512.

    The block-32 run reuses the lengths and the K/V/Q values of the block-16
    run; only the pool (1.25x of the blocks needed at 32) and its permutation
    are new (drawn from a second generator seeded 1003 / 1103).
    """
    seed = 3 if not small else 103
    rng = np.random.default_rng(seed)
    if small:
        lens = np.round(np.exp(rng.uniform(np.log(1), np.log(3000), size=8))).astype(np.int64)
    else:
        lens = np.round(np.exp(rng.uniform(np.log(128), np.log(32768), size=128))).astype(np.int64)
    base = paged_batch("long-context-decode-b16" if not small else "long-context-decode-small", seed,
                       kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                       prior_lens=lens - 1, new_lens=np.ones(len(lens), np.int64),
                       is_chunk=np.zeros(len(lens), bool), rng=rng)
    if block_size == 16:
        return base
    return config3_at_block(base, block_size)


def config3_at_block(base: PagedBatch, block_size: int) -> PagedBatch:
    """Config 3's run at another block size: the same lengths and K/V/Q
    values as ``base`` (the block-16 batch), a new 1.25x pool and permutation
    drawn from a generator seeded base.seed + 1000."""
    b = copy.copy(base)
    rng2 = np.random.default_rng(base.seed + 1000)
    nb = _pool_size(b.total_lens, block_size)
    b.name = base.name.replace("b16", f"b{block_size}")
    b.block_size = block_size
    b.num_blocks = nb
    b.free_order = rng2.permutation(nb).astype(np.int64)
    return b


def config4(small=False, kv_dtype="bf16") -> PagedBatch:
    """Mixed chunked-prefill batch: 8 chunks of 512 on prefixes U{0..7680} + 64 decodes U{256..4096}.
    kv_dtype "fp8" stores the same values as e4m3 with per-head scales."""
    seed = 4 if not small else 104
    rng = np.random.default_rng(seed)
    if small:
        n_chunk, chunk, n_dec = 3, 80, 5
        P = rng.integers(0, 601, size=n_chunk)
        Ld = rng.integers(1, 700, size=n_dec)
    else:
        n_chunk, chunk, n_dec = 8, 512, 64
        P = rng.integers(0, 7681, size=n_chunk)
        Ld = rng.integers(256, 4097, size=n_dec)
    prior = np.concatenate([P, Ld - 1])
    new = np.concatenate([np.full(n_chunk, chunk), np.ones(n_dec, np.int64)])
    is_chunk = np.concatenate([np.ones(n_chunk, bool), np.zeros(n_dec, bool)])
    name = "mixed-chunked-prefill" if not small else "mixed-chunked-prefill-small"
    return paged_batch(name if kv_dtype == "bf16" else name + "-" + kv_dtype, seed,
                       kv_dtype=kv_dtype, io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                       prior_lens=prior, new_lens=new, is_chunk=is_chunk, rng=rng)


def verify_batch(small=False, draft=4) -> PagedBatch:
    """Speculative verification on the Qwen3-8B decode layer: 32 seqs with a
    prefix of L ~ U{512..4096} accepted tokens, each appending a chunk of
    draft + 1 tokens (the last accepted token and the draft), bf16, B 16,
    pool 1.25x.  The chunk's K/V is stored before attention."""
    seed = 6 if not small else 106
    rng = np.random.default_rng(seed)
    n = 6 if small else 32
    P = rng.integers(1, 1400, size=n) if small else rng.integers(512, 4097, size=n)
    return paged_batch("qwen3-8b-verify" if not small else "qwen3-8b-verify-small", seed,
                       kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                       prior_lens=P, new_lens=np.full(n, draft + 1, np.int64), is_chunk=np.ones(n, bool),
                       rng=rng)


def verify_long_batch(draft=4, n=None) -> PagedBatch:
    """Speculative verification over the long-context config's prefixes: its
    128 context lengths (log-uniform 128..32768, the first draw) as accepted
    prefixes, each appending a chunk of draft + 1 tokens, Qwen3-8B heads,
    bf16, B 16, pool 1.25x (seed 7).  ``n``: only the first n sequences."""
    lens = config3_lengths()
    if n is not None:
        lens = lens[:n]
    rng = np.random.default_rng(7)
    return paged_batch("long-context-verify", 7, kv_dtype="bf16", io_dtype="bf16", Hq=32, Hkv=8, d=128, B=16,
                       prior_lens=lens, new_lens=np.full(len(lens), draft + 1, np.int64),
                       is_chunk=np.ones(len(lens), bool), rng=rng)


def config5(small=False, literal_fork=False) -> ForkBatch:
    """CoW fork with fp8 KV: a 2048-token prompt plus the parent's first generated
    token (2049 shared tokens, so the tail block is partly filled and shared)
    forked into 8 beams, 64 divergent tokens each.  ``literal_fork`` forks at
    exactly 2048 tokens instead (a full tail block: no copy-on-write)."""
    seed = 5 if not small else 105
    rng = np.random.default_rng(seed)
    if small:
        prompt, beams, steps, Hq, Hkv, d = 48, 4, 21, 8, 2, 128
    else:
        prompt, beams, steps, Hq, Hkv, d = 2048, 8, 64, 32, 8, 128
    shared = prompt if literal_fork else prompt + 1
    B = 16
    full_shared = shared // B          # blocks no beam ever writes again
    blocks_needed = full_shared + beams * (math.ceil((shared + steps) / B) - full_shared)
    nb = int(math.ceil(1.25 * blocks_needed))
    free_order = rng.permutation(nb).astype(np.int64)
    k_shared = _values(rng, (shared, Hkv, d), "bf16")
    v_shared = _values(rng, (shared, Hkv, d), "bf16")
    k_beam = _values(rng, (steps, beams, Hkv, d), "bf16")
    v_beam = _values(rng, (steps, beams, Hkv, d), "bf16")
    q = _values(rng, (beams, Hq, d), "bf16")
    ks, vs = _head_scales(np.concatenate([k_shared.reshape(-1, Hkv, d), k_beam.reshape(-1, Hkv, d)]),
                          np.concatenate([v_shared.reshape(-1, Hkv, d), v_beam.reshape(-1, Hkv, d)]))
    name = "cow-fork-fp8" + ("-literal2048" if literal_fork else "") + ("-small" if small else "")
    return ForkBatch(name, seed, "fp8", "bf16", Hq, Hkv, d, B, nb, free_order, shared, beams, steps,
                     k_shared, v_shared, k_beam, v_beam, q, ks, vs,
                     float(np.float32(1.0 / math.sqrt(d))))


def chunk_tokens_of(batch: PagedBatch):
    """Helpers for laying out step inputs: per-sequence slices into k / v."""
    off = batch.tok_offsets
    return [(int(off[i]), int(batch.prior_lens[i]), int(batch.new_lens[i])) for i in range(batch.num_seqs)]


@dataclass
class PrefixAgent:
    """Multi-turn agent conversations sharing one system prompt, for the
    prefix cache: every user's prompt at its local turn tau is the system
    prompt, the user's whole history of (message, reply) pairs, then a new
    message; after it, a reply is generated.  Users join at ``join_turn``.

    Token ids: the system prompt is 0..sys_len-1; user u's own tokens are
    ``1_000_000 (u + 1) + i`` for i along its conversation.  K, V and Q rows
    are drawn per token position of each user's stream; system-prompt
    positions take the shared rows, so equal token prefixes carry equal K/V.
    """
    name: str
    seed: int
    kv_dtype: str
    io_dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray
    capacity_blocks: int
    sys_len: int
    user_len: int
    reply_len: int
    turns: int
    join_turn: list          # per user, first turn (1-based) it takes part in
    k_sys: np.ndarray        # [sys_len, Hkv, d]
    v_sys: np.ndarray
    k_conv: np.ndarray       # [users, conv_len, Hkv, d]
    v_conv: np.ndarray
    q_all: np.ndarray        # [users, sys_len + conv_len, Hq, d]
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    scale: float = 0.0

    @property
    def users(self) -> int:
        return len(self.join_turn)

    @property
    def turn_len(self) -> int:
        return self.user_len + self.reply_len

    def local_turn(self, u: int, t: int) -> int:
        return t - self.join_turn[u] + 1

    def prompt_len(self, u: int, t: int) -> int:
        return self.sys_len + (self.local_turn(u, t) - 1) * self.turn_len + self.user_len

    def ids(self, u: int, lo: int, hi: int) -> np.ndarray:
        pos = np.arange(lo, hi, dtype=np.int64)
        own = 1_000_000 * (u + 1) + (pos - self.sys_len)
        return np.where(pos < self.sys_len, pos, own).astype(np.int32)

    def _rows(self, shared, own, u, lo, hi):
        parts = []
        if lo < self.sys_len:
            parts.append(shared[lo:min(hi, self.sys_len)])
        if hi > self.sys_len:
            parts.append(own[u, max(lo, self.sys_len) - self.sys_len:hi - self.sys_len])
        return np.concatenate(parts) if parts else shared[:0]

    def k_rows(self, u, lo, hi):
        return self._rows(self.k_sys, self.k_conv, u, lo, hi)

    def v_rows(self, u, lo, hi):
        return self._rows(self.v_sys, self.v_conv, u, lo, hi)

    def q_rows(self, u, lo, hi):
        return self.q_all[u, lo:hi]


def prefix_agent(small=False, kv_dtype="bf16") -> PrefixAgent:
    """The multi-turn agent example of the serving stack's prefix-cache
    section: a 1000-token system prompt, 60-token user messages, 120-token
    replies, 7 turns, 16-token blocks, a 4096-block cache; here four users
    start together and a fifth joins at turn 2 (Qwen3-8B layer shapes).
    ``small``: 100 / 12 / 20 tokens, 3 turns, 2 + 1 users, 8 / 2 heads."""
    seed = 7 if not small else 107
    rng = np.random.default_rng(seed)
    if small:
        sys_len, user_len, reply_len, turns, join = 100, 12, 20, 3, [1, 1, 2]
        Hq, Hkv, d = 8, 2, 128
    else:
        sys_len, user_len, reply_len, turns, join = 1000, 60, 120, 7, [1, 1, 1, 1, 2]
        Hq, Hkv, d = 32, 8, 128
    B, cap = 16, 4096
    conv_len = turns * (user_len + reply_len)
    U = len(join)
    # Room for every user's whole stream twice over (turn-1 prompts are
    # computed before any of them is recorded, so the system prompt is held
    # U times at once), plus slack.
    nb = int(math.ceil(2 * U * math.ceil((sys_len + conv_len) / B))) + 8
    free_order = rng.permutation(nb).astype(np.int64)
    k_sys = _values(rng, (sys_len, Hkv, d), "bf16")
    v_sys = _values(rng, (sys_len, Hkv, d), "bf16")
    k_conv = _values(rng, (U, conv_len, Hkv, d), "bf16")
    v_conv = _values(rng, (U, conv_len, Hkv, d), "bf16")
    q_all = _values(rng, (U, sys_len + conv_len, Hq, d), "bf16")
    ks = vs = None
    if kv_dtype == "fp8":
        ks, vs = _head_scales(np.concatenate([k_sys, k_conv.reshape(-1, Hkv, d)]),
                              np.concatenate([v_sys, v_conv.reshape(-1, Hkv, d)]))
    name = f"prefix-agent-{kv_dtype}" + ("-small" if small else "")
    return PrefixAgent(name, seed, kv_dtype, "bf16", Hq, Hkv, d, B, nb, free_order, cap, sys_len, user_len,
                       reply_len, turns, join, k_sys, v_sys, k_conv, v_conv, q_all, ks, vs,
                       float(np.float32(1.0 / math.sqrt(d))))


@dataclass
class SpecBranch:
    """Speculative decoding over copy-on-write branches: every target
    sequence holds ``prefix_lens[i]`` tokens; a draft branch forked from it
    appends ``draft`` tokens (its first append copies the shared tail block),
    a verification chunk attends over the branch, the target then appends
    the ``accepted[i]`` first draft tokens and the branch is released.

    Rows: ``k_prefix`` / ``v_prefix`` [sum(prefix_lens), Hkv, d] in sequence
    order; ``k_draft`` / ``v_draft`` [S, draft, Hkv, d]; ``q_verify``
    [S * draft, Hq, d] (the verification rows, sequence-major); ``q_next``
    [S, Hq, d] (the target's next decode query)."""
    name: str
    seed: int
    kv_dtype: str
    io_dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    free_order: np.ndarray
    prefix_lens: np.ndarray
    draft: int
    accepted: np.ndarray
    k_prefix: np.ndarray
    v_prefix: np.ndarray
    k_draft: np.ndarray
    v_draft: np.ndarray
    q_verify: np.ndarray
    q_next: np.ndarray
    k_scale: Optional[np.ndarray] = None
    v_scale: Optional[np.ndarray] = None
    scale: float = 0.0


def spec_branch(kv_dtype="bf16", draft=4) -> SpecBranch:
    """Eight targets with Qwen3-8B layer heads, bf16 or fp8 KV, block 16;
    prefixes mix partly filled tails (so every branch copies its tail on
    write), a full tail (the branch opens a new block: no copy) and long
    contexts; accepted counts 0..draft, fixed so that every case occurs."""
    seed = 8
    rng = np.random.default_rng(seed)
    Hq, Hkv, d, B = 32, 8, 128, 16
    prefix = np.array([37, 200, 511, 1000, 2049, 64, 3001, 1], dtype=np.int64)
    accepted = np.array([0, 1, 2, 3, 4, 2, 4, 1], dtype=np.int64)
    S = len(prefix)
    # targets and branches at once, plus a block per target for its accepted tokens
    need = int(sum(math.ceil((int(p) + draft) / B) + 2 for p in prefix))
    nb = int(math.ceil(1.25 * need))
    free_order = rng.permutation(nb).astype(np.int64)
    k_prefix = _values(rng, (int(prefix.sum()), Hkv, d), "bf16")
    v_prefix = _values(rng, (int(prefix.sum()), Hkv, d), "bf16")
    k_draft = _values(rng, (S, draft, Hkv, d), "bf16")
    v_draft = _values(rng, (S, draft, Hkv, d), "bf16")
    q_verify = _values(rng, (S * draft, Hq, d), "bf16")
    q_next = _values(rng, (S, Hq, d), "bf16")
    ks = vs = None
    if kv_dtype == "fp8":
        ks, vs = _head_scales(np.concatenate([k_prefix, k_draft.reshape(-1, Hkv, d)]),
                              np.concatenate([v_prefix, v_draft.reshape(-1, Hkv, d)]))
    return SpecBranch(f"spec-branch-{kv_dtype}", seed, kv_dtype, "bf16", Hq, Hkv, d, B, nb, free_order, prefix,
                      draft, accepted, k_prefix, v_prefix, k_draft, v_draft, q_verify, q_next, ks, vs,
                      float(np.float32(1.0 / math.sqrt(d))))
