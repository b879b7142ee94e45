"""Slot-mapped cache write and block copy on a plain cache (oracle side).

The oracle's cache is ``[num_blocks, block_size, Hkv, D]`` in the storage dtype
(numpy float16, or uint16 bf16 bit patterns): block ``b``, offset ``o`` holds
the K (or V) rows of every KV head for one token.  This layout is the oracle's
own and says nothing about how the GPU library lays out its pages.

The pages describe the block/slot model (page "vLLM 部署与 PagedAttention 原理 ·
检索整理", item 2: fixed-size blocks reached through a block table, shared
blocks copied on write).  The slot encoding ``slot = block * block_size +
offset`` and "negative slot = padding, skipped" are readings: the pages do not
name a slot mapping.
"""

import numpy as np


def new_cache(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int,
              np_dtype, fill=0):
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    return np.full(shape, fill, dtype=np_dtype), np.full(shape, fill, dtype=np_dtype)


def scatter_ref(k_cache, v_cache, k, v, slot_mapping):
    """For each token i with slot >= 0: write k[i], v[i] ([Hkv, D]) to
    block slot // bs, offset slot % bs."""
    bs = k_cache.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        k_cache[slot // bs, slot % bs] = k[i]
        v_cache[slot // bs, slot % bs] = v[i]


def copy_ref(k_cache, v_cache, block_pairs):
    """For each (src, dst): the whole block (all offsets, all heads) of src
    is copied to dst, for K and for V."""
    for src, dst in np.asarray(block_pairs).reshape(-1, 2).tolist():
        k_cache[dst] = k_cache[src]
        v_cache[dst] = v_cache[src]


def swap_ref(dst_k, dst_v, src_k, src_v, block_pairs):
    """Block swap between two caches of one shape (page "vLLM：从 PagedAttention
    长出来的开源服务栈", section "把显存当虚拟内存管": blocks can be swapped out of
    device memory and back in): for each (src, dst), block src of the source
    cache — every offset and head, K and V — becomes block dst of the
    destination cache.  Pairs naming a block outside its cache are skipped."""
    for src, dst in np.asarray(block_pairs).reshape(-1, 2).tolist():
        if 0 <= src < src_k.shape[0] and 0 <= dst < dst_k.shape[0]:
            dst_k[dst] = src_k[src]
            dst_v[dst] = src_v[src]
