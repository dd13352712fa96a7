"""CPU oracle for paged attention over a block-table-indexed KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and never imports it.

What it computes, in plain slow fp64 numpy, and what each part follows:

* ``block_manager``  -- host block manager (allocate / incref / free / CoW /
  fork / append), written from the page "LLM 推理服务引擎深度拆解"
  (chenxutan.com), section 2.3 (手写一个 Block Manager) and section 2.2
  (分页思想: block table, one indirection per KV read).
* ``fp8_e4m3``       -- OCP E4M3FN codec (round-to-nearest-even, saturate to
  +-448).  The PD-engineering page (ybb.press), section 6.2 (KV 缓存的精度压缩),
  names FP8 E4M3 KV caches; the bit format is the OCP 8-bit float format.
* ``paged``          -- store into / copy between paged blocks, and fp64
  attention that walks the block table (decode: one query per sequence;
  chunked prefill: a causal chunk over its paged prefix plus itself).
* ``byte_model``     -- KV bytes per token, after the PD-engineering page,
  section 3 (KV Cache 传输协议) and the serving-stack page, section 1.3.

Pins (tests marked ``not gpu``): every function here is checked against
something other than itself -- torch's float8_e4m3fn cast, torch's fp64
``scaled_dot_product_attention`` over contiguous K/V, closed forms, the
fork demo traced from section 2.3, the printed byte counts of the
PD-engineering page and the cost-model ratios of the nanoPD page.  No
function in this package is "parity unpinned".
"""
