"""CPU oracle for paged decode attention — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and its
Python binding) never imports, links or calls anything here, and this package
shares no code, header, table or helper with it.  Inputs come from the seeded
generators in ``synth``; nothing here ever reads a value produced by the GPU
path.

What it computes, in float64 from the same fp16/bf16 values the GPU reads:

* ``BlockManager`` — the paged KV bookkeeping: fixed-size token blocks, a
  per-sequence block table mapping logical to physical blocks, blocks allocated
  on demand, per-block reference counts and copy-on-write when parallel samples
  share prompt blocks (page "vLLM 部署与 PagedAttention 原理 · 检索整理", item 2,
  the 2023 vLLM blog; page "vLLM：从 PagedAttention 长出来的开源服务栈", section
  "把显存当虚拟内存管").
* ``scatter_ref`` / ``copy_ref`` / ``swap_ref`` — the slot-mapped cache write,
  the copy-on-write block copy and the block swap between two caches, on a
  plain ``[num_blocks, block_size, Hkv, D]`` cache.
* ``attention_ref`` / ``paged_decode_ref`` — decode attention: QK dot products,
  softmax normalisation and the weighted sum of V (page "vLLM 深度解析：以
  PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §2.1), read through the block
  table.
* ``brute_force_ref`` — the textbook formula in explicit loops on contiguous
  per-sequence K/V, independent of everything above.
* ``partition_partials_ref`` / ``lse_merge_ref`` — the same softmax split into
  token partitions and recombined by the log-sum-exp identity.
* ``prefill_ref`` — multi-token-query (chunked prefill) attention over the
  paged cache, causal by absolute position (readings in ``oracle/prefill.py``).
* ``fp8`` — the fp8 (E4M3) KV cache variant: the E4M3 codec written from its
  definition, the quantising slot-mapped write and decode attention over the
  dequantised rows (readings stated in ``oracle/fp8.py``).

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, special cases, brute force and the facts the pages print (see the
tests' docstrings).  No function is "parity unpinned".
"""

from .numerics import to_f64
from .block_manager import BlockManager, OutOfBlocks
from .cache_ops import new_cache, scatter_ref, copy_ref, swap_ref
from .attention import (
    attention_ref,
    paged_decode_ref,
    brute_force_ref,
    partition_partials_ref,
    lse_merge_ref,
)
from .runner import OracleStep, run_decode_step
from . import fp8
from .prefill import prefill_ref

__all__ = [
    "to_f64",
    "BlockManager",
    "OutOfBlocks",
    "new_cache",
    "scatter_ref",
    "copy_ref",
    "swap_ref",
    "attention_ref",
    "paged_decode_ref",
    "brute_force_ref",
    "partition_partials_ref",
    "lse_merge_ref",
    "OracleStep",
    "run_decode_step",
    "fp8",
    "prefill_ref",
]
