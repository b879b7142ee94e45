"""Run one synthetic decode step entirely on the oracle side.

Drives the oracle block manager through the workload's ops, writes every prior
token and the new tokens with ``scatter_ref``, applies the copy-on-write pairs
with ``copy_ref`` and evaluates ``paged_decode_ref``.  Test infrastructure only.
"""

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .attention import paged_decode_ref
from .block_manager import BlockManager
from .cache_ops import copy_ref, new_cache, scatter_ref
from .fp8 import new_fp8_cache, paged_decode_fp8_ref, scatter_fp8_ref

BLOCK_SIZE = 16


@dataclass
class OracleStep:
    block_manager: BlockManager
    k_cache: np.ndarray
    v_cache: np.ndarray
    k_cache_before_step: Optional[np.ndarray]
    v_cache_before_step: Optional[np.ndarray]
    slot_mapping: np.ndarray
    block_pairs: np.ndarray
    block_tables: np.ndarray
    context_lens: np.ndarray
    out: Optional[np.ndarray]  # float64 [S, Hq, D]


def run_decode_step(wl, *, max_blocks: Optional[int] = None, compute_out: bool = True,
                    keep_before: bool = False, seqs: Optional[Sequence[int]] = None,
                    initial_cache=None) -> OracleStep:
    """initial_cache: optional (K, V) [NB, 16, Hkv, 128] starting contents
    (e.g. garbage in never-written slots); copied, not modified.  An fp8
    workload (``wl.kv_dtype == "fp8e4m3"``) keeps uint8 E4M3 codes in the
    cache and attends over their dequantised values."""
    hkv = wl.num_kv_heads
    fp8 = wl.kv_dtype == "fp8e4m3"
    npdt = np.uint8 if fp8 else {"fp16": np.float16, "bf16": np.uint16}[wl.dtype]
    bm = BlockManager(wl.pool_blocks, BLOCK_SIZE, wl.free_order)
    if initial_cache is None:
        kc, vc = (new_fp8_cache if fp8 else lambda *a: new_cache(*a, npdt))(wl.pool_blocks, BLOCK_SIZE, hkv, 128)
    else:
        kc = np.array(initial_cache[0], dtype=npdt, copy=True)
        vc = np.array(initial_cache[1], dtype=npdt, copy=True)

    def scatter(k, v, slots):
        if fp8:
            scatter_fp8_ref(kc, vc, k, v, slots, wl.dtype, wl.k_scale, wl.v_scale)
        else:
            scatter_ref(kc, vc, k, v, slots)

    slot_mapping = pairs = None
    kb = vb = None
    for op in wl.ops:
        if op[0] == "add":
            _, s, n = op
            slots = bm.add(s, n)
            if n:
                k, v = wl.prior_kv_for_add(s)
                scatter(k, v, slots)
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        elif op[0] == "step":
            if keep_before:
                kb, vb = kc.copy(), vc.copy()
            slot_mapping, pairs = bm.step(op[1])
            copy_ref(kc, vc, pairs)
            k_new, v_new = wl.new_token_kv()
            scatter(k_new, v_new, slot_mapping)
        else:
            raise ValueError(op)
    S = wl.num_seqs
    ctx = bm.context_lens(range(S))
    assert np.array_equal(ctx, wl.context_lens)
    if max_blocks is None:
        max_blocks = max(len(bm.blocks[s]) for s in range(S))
    tables = bm.block_table(range(S), max_blocks)
    out = None
    if compute_out and fp8:
        out = paged_decode_fp8_ref(wl.q, kc, vc, tables, ctx, wl.scale, hkv, wl.dtype, wl.k_scale, wl.v_scale,
                                   seqs=seqs)
    elif compute_out:
        out = paged_decode_ref(wl.q, kc, vc, tables, ctx, wl.scale, hkv, wl.dtype, seqs=seqs)
    return OracleStep(bm, kc, vc, kb, vb, slot_mapping, pairs, tables, ctx, out)
