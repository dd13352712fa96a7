"""KV-cache byte model (oracle; test infrastructure only).

The PD-engineering page (ybb.press), section 3 (KV Cache 传输协议), counts the
KV of one token of one layer as 2 (K and V) * kv_heads * head_dim * bytes per
element; the serving-stack page (chenxutan.com), section 1.3, multiplies that
by layers, sequence length and batch.  Decode reads every stored byte of
every context token once per step, which makes these bytes the algorithmic
traffic of paged decode.
"""
from __future__ import annotations

ELEM_BYTES = {"f32": 4, "bf16": 2, "fp16": 2, "fp8": 1}


def kv_bytes_per_token(kv_heads: int, head_dim: int, dtype: str, layers: int = 1) -> int:
    return 2 * layers * kv_heads * head_dim * ELEM_BYTES[dtype]


def kv_cache_bytes(layers, kv_heads, head_dim, seq_len, dtype="bf16", batch=1) -> int:
    return kv_bytes_per_token(kv_heads, head_dim, dtype, layers) * seq_len * batch


def decode_kv_bytes(context_lens, kv_heads, head_dim, dtype) -> int:
    """Bytes of K and V a decode step must read: every context token once."""
    return sum(int(L) for L in context_lens) * kv_bytes_per_token(kv_heads, head_dim, dtype)


def prefill_chunk_flops(prefix_lens, q_lens, num_q_heads, head_dim) -> int:
    """Unmasked multiply-adds of QK^T and PV, 2 flops each: 4*d*Hq per (query, key) pair."""
    pairs = 0
    for P, n in zip(prefix_lens, q_lens):
        P, n = int(P), int(n)
        pairs += n * P + n * (n + 1) // 2      # row t sees P + t + 1 keys
    return 4 * head_dim * num_q_heads * pairs
