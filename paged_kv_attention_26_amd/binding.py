"""Python binding of libpa: torch tensors in, C ABI calls out.

Marshalling only: shape / dtype / device checks, pointers, the current HIP
stream.  All computation happens in libpa's kernels.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np
import torch

from . import _lib as L

DTYPE_CODES = {"f32": L.PA_F32, "bf16": L.PA_BF16, "fp8": L.PA_FP8_E4M3}
CACHE_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}
IO_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.bfloat16}
# NaN patterns written into fresh pools so that a stray read shows up as NaN
POISON = {"f32": (torch.int32, 0x7FC00000), "bf16": (torch.int16, 0x7FC0), "fp8": (torch.uint8, 0x7F)}


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None) -> C.c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return C.c_void_p(t.data_ptr())


class KVCache:
    """A paged KV cache: K pool [NB, Hkv, B, D] and transposed V pool [NB, Hkv, D, B]."""

    def __init__(self, k_cache: torch.Tensor, v_cache: torch.Tensor, dtype: str,
                 k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None):
        if dtype not in DTYPE_CODES:
            raise ValueError(f"unknown cache dtype {dtype}")
        nb, hkv, bs, d = k_cache.shape
        if tuple(v_cache.shape) != (nb, hkv, d, bs):
            raise ValueError(f"v_cache must be [NB, Hkv, D, B] = {(nb, hkv, d, bs)}, got {tuple(v_cache.shape)}")
        _dev(k_cache, "k_cache", CACHE_TORCH[dtype])
        _dev(v_cache, "v_cache", CACHE_TORCH[dtype])
        if dtype == "fp8":
            _dev(k_scale, "k_scale", torch.float32)
            _dev(v_scale, "v_scale", torch.float32)
        self.k_cache, self.v_cache, self.dtype = k_cache, v_cache, dtype
        self.k_scale, self.v_scale = k_scale, v_scale
        self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim = nb, hkv, bs, d
        self.desc = L.PaKvCache(k_cache.data_ptr(), v_cache.data_ptr(),
                                k_scale.data_ptr() if k_scale is not None else None,
                                v_scale.data_ptr() if v_scale is not None else None,
                                nb, hkv, bs, d, DTYPE_CODES[dtype])

    @property
    def io_dtype(self) -> torch.dtype:
        return IO_TORCH[self.dtype]


def alloc_cache(num_blocks, num_kv_heads, block_size, head_dim, dtype, device="cuda",
                k_scale=None, v_scale=None, poison=True) -> KVCache:
    tdt = CACHE_TORCH[dtype]
    k = torch.empty((num_blocks, num_kv_heads, block_size, head_dim), dtype=tdt, device=device)
    v = torch.empty((num_blocks, num_kv_heads, head_dim, block_size), dtype=tdt, device=device)
    if poison:
        view_dt, bits = POISON[dtype]
        k.view(view_dt).fill_(bits)
        v.view(view_dt).fill_(bits)
    if dtype == "fp8":
        k_scale = torch.as_tensor(k_scale, dtype=torch.float32).to(device).contiguous()
        v_scale = torch.as_tensor(v_scale, dtype=torch.float32).to(device).contiguous()
    return KVCache(k, v, dtype, k_scale, v_scale)


def store_kv(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, slot_mapping: torch.Tensor,
             stream=None) -> None:
    T = slot_mapping.numel()
    shape = (T, cache.num_kv_heads, cache.head_dim)
    if tuple(k_new.shape) != shape or tuple(v_new.shape) != shape:
        raise ValueError(f"k_new / v_new must be {shape}")
    if cache.dtype == "fp8" and k_new.dtype == CACHE_TORCH["fp8"]:   # e4m3 codes, stored as they are
        io, tdt = DTYPE_CODES["fp8"], CACHE_TORCH["fp8"]
    else:
        io, tdt = (DTYPE_CODES["f32"] if cache.dtype == "f32" else DTYPE_CODES["bf16"]), cache.io_dtype
    L.check(L.lib().pa_store_kv(C.byref(cache.desc), _dev(k_new, "k_new", tdt), _dev(v_new, "v_new", tdt), io,
                                _dev(slot_mapping, "slot_mapping", torch.int32), T, _stream(stream)),
            "pa_store_kv")


def pack_kv(cache: KVCache, block_table: torch.Tensor, seq_lens: torch.Tensor, cu_rows: torch.Tensor,
            max_seq_len: int, rows: int, k_out: Optional[torch.Tensor] = None,
            v_out: Optional[torch.Tensor] = None, stream=None):
    """Gather the sequences' cached K/V into contiguous rows [rows, Hkv, D] of
    the cache dtype (pa_pack_kv).  Returns (k_out, v_out)."""
    S = seq_lens.numel()
    if block_table.dim() != 2 or block_table.shape[0] != S or cu_rows.numel() != S:
        raise ValueError("block_table must be [S, max_blocks], seq_lens and cu_rows [S]")
    shape = (rows, cache.num_kv_heads, cache.head_dim)
    tdt = CACHE_TORCH[cache.dtype]
    if k_out is None:
        k_out = torch.empty(shape, dtype=tdt, device=cache.k_cache.device)
    if v_out is None:
        v_out = torch.empty(shape, dtype=tdt, device=cache.k_cache.device)
    if tuple(k_out.shape) != shape or tuple(v_out.shape) != shape:
        raise ValueError(f"k_out / v_out must be {shape}")
    L.check(L.lib().pa_pack_kv(C.byref(cache.desc), _dev(block_table, "block_table", torch.int32),
                               block_table.shape[1], _dev(seq_lens, "seq_lens", torch.int32),
                               _dev(cu_rows, "cu_rows", torch.int32), S, int(max_seq_len),
                               _dev(k_out, "k_out", tdt), _dev(v_out, "v_out", tdt), _stream(stream)),
            "pa_pack_kv")
    return k_out, v_out


def copy_blocks(cache: KVCache, pairs: torch.Tensor, stream=None) -> None:
    n = pairs.shape[0] if pairs.numel() else 0
    if n and tuple(pairs.shape) != (n, 2):
        raise ValueError("pairs must be [n, 2]")
    ptr = _dev(pairs, "pairs", torch.int32) if n else None
    L.check(L.lib().pa_copy_blocks(C.byref(cache.desc), ptr, n, _stream(stream)), "pa_copy_blocks")


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens=0) -> int:
    return int(L.lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len,
                                                 partition_tokens))


def decode_workspace(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens=0,
                     device="cuda") -> torch.Tensor:
    """Workspace for pa_decode: partial results and per-item arrival counters.
    It is zero-filled here, once; every pa_decode call leaves it ready for the
    next.  Calls that may run at the same time need workspaces of their own."""
    n = decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_tokens)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)


_default_workspaces = {}


def _default_workspace(head_dim, device, stream_handle) -> torch.Tensor:
    """One zero-filled workspace per (device, stream, head_dim), kept for the
    process: calls on one stream run one after another, so they may share it."""
    key = (torch.device(device).index, stream_handle, int(head_dim))
    ws = _default_workspaces.get(key)
    if ws is None:
        ws = decode_workspace(1, 1, head_dim, 1, 0, device=device)
        _default_workspaces[key] = ws
    return ws


def decode(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
           max_context_len: int, scale: float, out: Optional[torch.Tensor] = None, partition_tokens: int = 64,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode.  partition_tokens: a multiple of the block size (64, the
    default, is the fastest split), or 0 for no split."""
    S, Hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _default_workspace(D, q.device, _stream(stream).value)
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_table must be [S, max_blocks] and context_lens [S]")
    io = DTYPE_CODES["f32"] if cache.dtype == "f32" else DTYPE_CODES["bf16"]
    L.check(L.lib().pa_decode(C.byref(cache.desc), _dev(q, "q", cache.io_dtype), io,
                              _dev(out, "out", cache.io_dtype), io, S, Hq, float(scale),
                              _dev(block_table, "block_table", torch.int32), block_table.shape[1],
                              _dev(context_lens, "context_lens", torch.int32), int(max_context_len),
                              int(partition_tokens), _dev(workspace, "workspace"), workspace.numel(),
                              _stream(stream)),
            "pa_decode")
    return out


def decode_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                  block_table: torch.Tensor, context_lens: torch.Tensor, max_context_len: int, scale: float,
                  out: Optional[torch.Tensor] = None, partition_tokens: int = 64,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """pa_decode_append: store each sequence's new token (k_new / v_new rows
    [S, Hkv, d], at position context_lens[s] - 1) and decode, in one launch;
    the same results as store_kv followed by decode."""
    S, Hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = _default_workspace(D, q.device, _stream(stream).value)
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_table must be [S, max_blocks] and context_lens [S]")
    if tuple(k_new.shape) != (S, cache.num_kv_heads, D) or tuple(v_new.shape) != (S, cache.num_kv_heads, D):
        raise ValueError("k_new / v_new must be [S, num_kv_heads, head_dim]")
    io = DTYPE_CODES["f32"] if cache.dtype == "f32" else DTYPE_CODES["bf16"]
    L.check(L.lib().pa_decode_append(C.byref(cache.desc), _dev(k_new, "k_new", cache.io_dtype),
                                     _dev(v_new, "v_new", cache.io_dtype), _dev(q, "q", cache.io_dtype), io,
                                     _dev(out, "out", cache.io_dtype), io, S, Hq, float(scale),
                                     _dev(block_table, "block_table", torch.int32), block_table.shape[1],
                                     _dev(context_lens, "context_lens", torch.int32), int(max_context_len),
                                     int(partition_tokens), _dev(workspace, "workspace"), workspace.numel(),
                                     _stream(stream)),
            "pa_decode_append")
    return out


def decode_noalloc(cache: KVCache, q: torch.Tensor, block_table: torch.Tensor, context_lens: torch.Tensor,
                   max_context_len: int, scale: float, out: Optional[torch.Tensor] = None,
                   partition_tokens: int = 64, stream=None) -> torch.Tensor:
    """pa_decode_noalloc: decode with the library's own per-device scratch
    instead of a workspace (no allocation beyond ``out`` when it is given).
    Calls that may overlap on one GPU race."""
    S, Hq, D = q.shape
    if D != cache.head_dim:
        raise ValueError("q head_dim does not match the cache")
    if out is None:
        out = torch.empty_like(q)
    if block_table.dim() != 2 or block_table.shape[0] != S or context_lens.numel() != S:
        raise ValueError("block_table must be [S, max_blocks] and context_lens [S]")
    io = DTYPE_CODES["f32"] if cache.dtype == "f32" else DTYPE_CODES["bf16"]
    L.check(L.lib().pa_decode_noalloc(C.byref(cache.desc), _dev(q, "q", cache.io_dtype), io,
                                      _dev(out, "out", cache.io_dtype), io, S, Hq, float(scale),
                                      _dev(block_table, "block_table", torch.int32), block_table.shape[1],
                                      _dev(context_lens, "context_lens", torch.int32), int(max_context_len),
                                      int(partition_tokens), _stream(stream)),
            "pa_decode_noalloc")
    return out


def time_next_decode(start: Optional[torch.cuda.Event], stop: Optional[torch.cuda.Event]) -> None:
    """Arm pa_decode_time_next: the next decode() on this thread records the
    two events with its kernel's own start and end timestamps.  The events
    must exist already (torch creates one at its first record())."""
    ptrs = []
    for e in (start, stop):
        if e is None:
            ptrs.append(None)
            continue
        if not isinstance(e, torch.cuda.Event) or not e.cuda_event:
            raise ValueError("pass torch.cuda.Event objects that have been recorded once (so that they exist)")
        ptrs.append(C.c_void_p(e.cuda_event))
    L.check(L.lib().pa_decode_time_next(ptrs[0], ptrs[1]), "pa_decode_time_next")


def prefill_chunk(cache: KVCache, q: torch.Tensor, cu_q_lens: torch.Tensor, seq_lens: torch.Tensor,
                  block_table: torch.Tensor, max_q_len: int, max_seq_len: int, scale: float,
                  out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  split: bool = True, stream=None) -> torch.Tensor:
    """pa_prefill_chunk.  split: give the verification kernel a workspace
    (``workspace``, else the stream's default one, shared with decode), so
    that it cuts the batch's keys into equal stretches; False passes none."""
    T, Hq, D = q.shape
    S = seq_lens.numel()
    if out is None:
        out = torch.empty_like(q)
    if cu_q_lens.numel() != S + 1 or block_table.dim() != 2 or block_table.shape[0] != S:
        raise ValueError("cu_q_lens must be [S+1] and block_table [S, max_blocks]")
    ws_ptr, ws_bytes = None, 0
    if split:
        if workspace is None:
            workspace = _default_workspace(D, q.device, _stream(stream).value)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel()
    L.check(L.lib().pa_prefill_chunk(C.byref(cache.desc), _dev(q, "q", torch.bfloat16), DTYPE_CODES["bf16"],
                                     _dev(out, "out", torch.bfloat16), DTYPE_CODES["bf16"], S, Hq, float(scale),
                                     _dev(cu_q_lens, "cu_q_lens", torch.int32),
                                     _dev(seq_lens, "seq_lens", torch.int32),
                                     _dev(block_table, "block_table", torch.int32), block_table.shape[1],
                                     int(max_q_len), int(max_seq_len), ws_ptr, ws_bytes, _stream(stream)),
            "pa_prefill_chunk")
    return out


class BlockManager:
    """Host block manager of libpa (pa_bm_*): allocate / fork / copy on write."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        self._l = L.lib()
        fo = None
        if free_order is not None:
            self._fo = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            fo = self._fo.ctypes.data_as(C.POINTER(C.c_int32))
        self._h = self._l.pa_bm_create(int(num_blocks), int(block_size), fo)
        if not self._h:
            raise L.PaError(L.PA_ERR_SHAPE, "pa_bm_create")
        self.num_blocks, self.block_size = int(num_blocks), int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._l.pa_bm_destroy(h)
            self._h = None

    def seq_new(self) -> int:
        s = self._l.pa_bm_seq_new(self._h)
        if s < 0:
            raise L.PaError(s, "pa_bm_seq_new")
        return s

    def append(self, seq: int, n: int) -> np.ndarray:
        out = np.zeros(max(n, 1), dtype=np.int32)
        got = self._l.pa_bm_append(self._h, seq, n, out.ctypes.data_as(C.POINTER(C.c_int32)))
        if got < 0:
            raise L.PaError(got, "pa_bm_append")
        if got < n:
            raise MemoryError(self._l.pa_last_error().decode())
        return out[:n]

    def fork(self, seq: int) -> int:
        s = self._l.pa_bm_fork(self._h, seq)
        if s < 0:
            raise L.PaError(s, "pa_bm_fork")
        return s

    def release(self, seq: int) -> None:
        L.check(self._l.pa_bm_release(self._h, seq), "pa_bm_release")

    def take_copies(self) -> np.ndarray:
        pairs = []
        buf = np.zeros((64, 2), dtype=np.int32)
        while True:
            n = self._l.pa_bm_take_copies(self._h, buf.ctypes.data_as(C.POINTER(C.c_int32)), 64)
            if n < 0:
                raise L.PaError(n, "pa_bm_take_copies")
            pairs.append(buf[:n].copy())
            if n < 64:
                break
        return np.concatenate(pairs).reshape(-1, 2)

    def seq_len(self, seq: int) -> int:
        return int(self._l.pa_bm_seq_len(self._h, seq))

    def block_table(self, seq: int) -> list:
        n = self._l.pa_bm_block_table(self._h, seq, None, 0)
        if n < 0:
            raise L.PaError(n, "pa_bm_block_table")
        out = np.zeros(max(n, 1), dtype=np.int32)
        self._l.pa_bm_block_table(self._h, seq, out.ctypes.data_as(C.POINTER(C.c_int32)), n)
        return out[:n].tolist()

    def block_tables(self, seqs, pad: int, min_width: int = 1) -> np.ndarray:
        rows = [self.block_table(s) for s in seqs]
        width = max([min_width] + [len(r) for r in rows])
        out = np.full((len(rows), width), pad, dtype=np.int32)
        for i, r in enumerate(rows):
            out[i, :len(r)] = r
        return out

    @property
    def used_blocks(self) -> int:
        return int(self._l.pa_bm_used_blocks(self._h))

    def ref_count(self, block: int) -> int:
        r = self._l.pa_bm_ref_count(self._h, block)
        if r < 0:
            raise L.PaError(r, "pa_bm_ref_count")
        return int(r)

    # -- prefix cache (pa_bm_prefix_*) ----------------------------------------
    @staticmethod
    def _ids(token_ids):
        a = np.ascontiguousarray(np.asarray(token_ids, dtype=np.int32).reshape(-1))
        return a, a.ctypes.data_as(C.POINTER(C.c_int32))

    def set_prefix_capacity(self, capacity_blocks: int) -> None:
        L.check(self._l.pa_bm_prefix_cache_set_capacity(self._h, int(capacity_blocks)),
                "pa_bm_prefix_cache_set_capacity")

    def prefix_lookup(self, token_ids):
        """(hit tokens, physical blocks of the hit)."""
        a, p = self._ids(token_ids)
        out = np.zeros(max(len(a) // self.block_size, 1), dtype=np.int32)
        hit = self._l.pa_bm_prefix_lookup(self._h, p, len(a),
                                          out.ctypes.data_as(C.POINTER(C.c_int32)), len(out))
        if hit < 0:
            raise L.PaError(hit, "pa_bm_prefix_lookup")
        return int(hit), out[:hit // self.block_size].tolist()

    def seq_new_prefixed(self, token_ids) -> int:
        a, p = self._ids(token_ids)
        s = self._l.pa_bm_seq_new_prefixed(self._h, p, len(a))
        if s < 0:
            raise L.PaError(s, "pa_bm_seq_new_prefixed")
        return s

    def prefix_insert(self, seq: int, token_ids) -> int:
        a, p = self._ids(token_ids)
        n = self._l.pa_bm_prefix_insert(self._h, seq, p, len(a))
        if n < 0:
            raise L.PaError(n, "pa_bm_prefix_insert")
        return int(n)

    def prefix_stats(self) -> dict:
        out = (C.c_int64 * 4)()
        L.check(self._l.pa_bm_prefix_stats(self._h, out), "pa_bm_prefix_stats")
        return {"hits": out[0], "misses": out[1], "cached_blocks": out[2], "capacity": out[3]}

    def unused_block(self) -> int:
        for b in range(self.num_blocks):
            if self._l.pa_bm_ref_count(self._h, b) == 0:
                return b
        return 0
