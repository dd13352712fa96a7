"""Paged KV store / copy and fp64 attention through a block table (oracle).

TEST INFRASTRUCTURE ONLY.  Plain numpy, fp64 arithmetic, no blocking or
fusion beyond the definitions below.

Cache layout (a definition of this library's interface; the pages leave the
physical layout open):

* K pool: ``k_cache[num_blocks, num_kv_heads, block_size, head_dim]``
  -- a token's key row for one kv head is contiguous;
* V pool: ``v_cache[num_blocks, num_kv_heads, head_dim, block_size]``
  -- each block stores V transposed, so one head-dim column of a block's
  tokens is contiguous.

A token's slot is ``physical_block * block_size + offset`` (serving-stack
page, section 2.2: the block table maps logical block i to a physical
block, and a read adds the in-block offset).

Storage dtypes held by the oracle:
``"f32"``  -> numpy float32;  ``"bf16"`` -> numpy uint16 holding the bf16 bits;
``"fp8"``  -> numpy uint8 holding OCP E4M3FN codes, with one fp32 scale per kv
head for K and one for V (a stored code c of head h means c * scale[h]).

Attention follows the definition: for sequence s and query head h, with
``g = h // (Hq // Hkv)`` (contiguous GQA groups; the PD-engineering page,
section 6.2, shares 8 KV heads among 32 query heads),
``o = sum_i softmax_i(scale * <q, k_i>) * v_i`` over the sequence's logical
tokens i, each read through ``block_table[s][i // B]`` at offset ``i % B``.
Decode attends to tokens 0..L-1 (L = context length, which includes the
token just stored).  A prefill chunk token at absolute position P + t
(P = tokens before the chunk) attends to tokens 0..P+t (the chunked-prefill
sections: nanoPD page "分块预填充", PD-engineering page 6.1, serving-stack
page 5.2).  An empty context gives 0.
"""
from __future__ import annotations

import numpy as np

from . import fp8_e4m3

STORAGE = {"f32": np.float32, "bf16": np.uint16, "fp8": np.uint8}


# ---------------------------------------------------------------- decoding
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (the top half of an fp32)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def values_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 value of stored f32 / bf16 data (not fp8: that needs a scale)."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    raise ValueError(dtype)


def _stored_to_f64(codes: np.ndarray, dtype: str, head_scale: np.ndarray | None) -> np.ndarray:
    """Stored rows [..., Hkv, d] -> fp64; fp8 codes are multiplied by their head's scale."""
    if dtype == "fp8":
        v = fp8_e4m3.decode(codes)
        return v * np.asarray(head_scale, dtype=np.float32).astype(np.float64)[:, None]
    return values_f64(codes, dtype)


def _encode_rows(x: np.ndarray, in_dtype: str, kv_dtype: str, head_scale) -> np.ndarray:
    """Input rows [Hkv, d] (storage of in_dtype) -> cache storage of kv_dtype."""
    if kv_dtype == in_dtype:
        return np.asarray(x, dtype=STORAGE[kv_dtype])
    if kv_dtype == "fp8" and in_dtype == "bf16":
        xf = bf16_bits_to_f64(x).astype(np.float32)       # exact
        sc = np.asarray(head_scale, dtype=np.float32)[:, None]
        return fp8_e4m3.quantize(xf, sc)
    raise ValueError(f"unsupported store {in_dtype} -> {kv_dtype}")


# ------------------------------------------------------------ store / copy
def new_pools(num_blocks, num_kv_heads, block_size, head_dim, kv_dtype):
    """Pools filled with a NaN poison so that stray reads show up."""
    kshape = (num_blocks, num_kv_heads, block_size, head_dim)
    vshape = (num_blocks, num_kv_heads, head_dim, block_size)
    poison = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "fp8": np.uint8(0x7F)}[kv_dtype]
    dt = STORAGE[kv_dtype]
    kc = np.full(kshape, poison, dtype=dt)
    vc = np.full(vshape, poison, dtype=dt)
    return kc, vc


def store_kv(k_cache, v_cache, kv_dtype, k_new, v_new, in_dtype, slot_mapping,
             k_scale=None, v_scale=None):
    """Scatter new rows [T, Hkv, d] to their slots; slot < 0 means skip.

    ``cache[slot // B, h, slot % B, :] = enc(x[t, h, :])`` for K, and the
    transposed placement ``[slot // B, h, :, slot % B]`` for V.
    """
    B = k_cache.shape[2]
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        blk, off = divmod(int(slot), B)
        k_cache[blk, :, off, :] = _encode_rows(k_new[t], in_dtype, kv_dtype, k_scale)
        v_cache[blk, :, :, off] = _encode_rows(v_new[t], in_dtype, kv_dtype, v_scale)


def copy_blocks(k_cache, v_cache, pairs):
    """Copy-on-write block copies: ``cache[dst] = cache[src]`` for every pair."""
    for src, dst in np.asarray(pairs, dtype=np.int64).reshape(-1, 2).tolist():
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def pack_kv(k_cache, v_cache, block_tables, seq_lens):
    """The KV hand-off gather (nanoPD page, 异步KV传输; PD-engineering page
    section 3): every sequence's stored K and V, token by token, as rows
    [sum(seq_lens), Hkv, d] of the cache's own storage (no decoding), in
    sequence order.  Row i of sequence s is its token i, read at
    ``cache[table[s][i // B], h, i % B, :]`` (K) and ``[.., h, :, i % B]`` (V).
    """
    B = k_cache.shape[2]
    ks, vs = [], []
    for table_row, n in zip(block_tables, seq_lens):
        i = np.arange(int(n))
        blk = np.asarray(table_row, dtype=np.int64)[i // B]
        off = i % B
        ks.append(k_cache[blk, :, off, :])
        vs.append(v_cache[blk, :, :, off])
    shape = (0,) + k_cache.shape[1:2] + k_cache.shape[3:]
    return (np.concatenate(ks) if ks else np.zeros(shape, k_cache.dtype),
            np.concatenate(vs) if vs else np.zeros(shape, v_cache.dtype))


# --------------------------------------------------------------- attention
def gather_kv(k_cache, v_cache, kv_dtype, table_row, n_tokens, k_scale=None, v_scale=None):
    """Logical tokens 0..n-1 of one sequence, read through its block table.

    Returns K, V as fp64 arrays [n, Hkv, d].
    """
    B = k_cache.shape[2]
    i = np.arange(n_tokens)
    blk = np.asarray(table_row, dtype=np.int64)[i // B]
    off = i % B
    k = k_cache[blk, :, off, :]            # [n, Hkv, d]
    v = v_cache[blk, :, :, off]            # [n, Hkv, d]
    return (_stored_to_f64(k, kv_dtype, k_scale), _stored_to_f64(v, kv_dtype, v_scale))


def _softmax_weighted(scores: np.ndarray, v: np.ndarray) -> np.ndarray:
    """Two-pass max-subtracted softmax over the last axis, then weights @ v."""
    m = scores.max(axis=-1, keepdims=True)
    p = np.exp(scores - m)
    return (p @ v) / p.sum(axis=-1, keepdims=True)


def decode_attention(k_cache, v_cache, kv_dtype, q, q_dtype, block_table, context_lens,
                     scale, k_scale=None, v_scale=None):
    """One query token per sequence.  q: [S, Hq, d] storage -> fp64 [S, Hq, d]."""
    qf = values_f64(q, q_dtype)
    S, Hq, d = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros((S, Hq, d), dtype=np.float64)
    for s in range(S):
        L = int(context_lens[s])
        if L == 0:
            continue
        k, v = gather_kv(k_cache, v_cache, kv_dtype, block_table[s], L, k_scale, v_scale)
        for h in range(Hq):
            g = h // G
            scores = scale * (k[:, g, :] @ qf[s, h])          # [L]
            out[s, h] = _softmax_weighted(scores[None, :], v[:, g, :])[0]
    return out


def prefill_chunk_attention(k_cache, v_cache, kv_dtype, q, q_dtype, cu_q_lens, seq_lens,
                            block_table, scale, k_scale=None, v_scale=None):
    """Causal chunk over a paged prefix.  q: [sum_q, Hq, d] -> fp64 [sum_q, Hq, d].

    Sequence j owns query rows cu_q_lens[j]..cu_q_lens[j+1]; its chunk of n
    tokens sits at absolute positions P..P+n-1 with P = seq_lens[j] - n, and
    row t attends to keys 0..P+t.
    """
    qf = values_f64(q, q_dtype)
    _, Hq, d = qf.shape
    Hkv = k_cache.shape[1]
    G = Hq // Hkv
    out = np.zeros(qf.shape, dtype=np.float64)
    for j in range(len(seq_lens)):
        r0, r1 = int(cu_q_lens[j]), int(cu_q_lens[j + 1])
        n = r1 - r0
        total = int(seq_lens[j])
        if n == 0:
            continue
        P = total - n
        if P < 0:
            raise ValueError("seq_len shorter than its chunk")
        k, v = gather_kv(k_cache, v_cache, kv_dtype, block_table[j], total, k_scale, v_scale)
        key_pos = np.arange(total)[None, :]
        q_pos = P + np.arange(n)[:, None]
        allowed = key_pos <= q_pos                                  # [n, total]
        for h in range(Hq):
            g = h // G
            scores = scale * (qf[r0:r1, h, :] @ k[:, g, :].T)      # [n, total]
            scores = np.where(allowed, scores, -np.inf)
            out[r0:r1, h] = _softmax_weighted(scores, v[:, g, :])
    return out
