"""pa_decode_noalloc (the library's own per-device scratch in place of a
caller workspace) against pa_decode with a workspace (needs an MI355X).

Calls in a row on shrinking batches (the Qwen3-8B decode layer, five
long-context sequences, the tiny fp32 batch), at 64-token partitions and
with no split: each output is
bit-identical to pa_decode's on the same inputs (same kernels, same launch,
so the same arithmetic), and within the bf16 tolerance of the oracle.
"""
import sys

import numpy as np
import pytest
import torch

import workloads as W
from tests import oracle_setup as OS

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from paged_kv_attention_26_amd import _lib
    _lib.lib()


def _subset(batch, n):
    """The first n sequences of a decode batch, with its own pool."""
    rng = np.random.default_rng(batch.seed + 500)
    return W.paged_batch(batch.name + f"-first{n}", batch.seed + 500, kv_dtype=batch.kv_dtype,
                         io_dtype=batch.io_dtype, Hq=batch.num_q_heads, Hkv=batch.num_kv_heads, d=batch.head_dim,
                         B=batch.block_size, prior_lens=batch.prior_lens[:n], new_lens=batch.new_lens[:n],
                         is_chunk=batch.is_chunk[:n], rng=rng)


def test_decode_noalloc_matches_decode_twice():
    from paged_kv_attention_26_amd import binding as pa, runner
    big = W.config2()
    small = _subset(W.config3(16, small=True), 5)
    tiny = W.config1()                                   # fp32 cache, head_dim 64
    tol = {"bf16": 2e-2, "f32": 1e-4}
    for part in (64, 0):
        for batch in (big, small, tiny):
            say(f"[gpu] decode_noalloc {batch.name} ({batch.num_seqs} seqs) partition {part}")
            g = runner.prepare(batch)
            runner.store_step(g)
            d = g.dec
            ws = pa.decode_workspace(1, 1, batch.head_dim, 1, part)
            want = pa.decode(g.cache, d["q"], d["table"], d["lens"], d["max_len"], batch.scale,
                             partition_tokens=part, workspace=ws)
            got = pa.decode_noalloc(g.cache, d["q"], d["table"], d["lens"], d["max_len"], batch.scale,
                                    partition_tokens=part)
            torch.cuda.synchronize()
            assert torch.equal(got.view(torch.int16), want.view(torch.int16))       # bit-identical
            err = np.max(np.abs(got.float().cpu().numpy().astype(np.float64) -
                                OS.decode_ref(batch, OS.build(batch))))
            say(f"      bit-identical to pa_decode; max abs err {err:.3e}")
            assert err < tol[batch.kv_dtype]
            del g
