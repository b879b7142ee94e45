"""Multi-token-query paged attention (chunked prefill), oracle side — TEST
INFRASTRUCTURE ONLY.

Page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §2.2
(continuous batching, chunked prefill and prefix caching): the prefill of a long
prompt is cut into chunks that run alongside decode requests.  The page gives no
formula for a chunk's attention; the plainest reading, taken here:

* sequence s has ``context_lens[s]`` tokens in the paged cache, the last
  ``C_s`` of which are the current chunk (written by the slot-mapped write before
  the attention call); ``C_s = query_start[s+1] - query_start[s]``;
* chunk query j of sequence s sits at absolute position
  ``p = context_lens[s] - C_s + j`` and attends causally to cache tokens
  ``0 .. p`` (itself included); its output row is ``query_start[s] + j``;
* each query is plain softmax attention (``attention_ref``) over those rows,
  float64, heads grouped as in decode (KV head ``h // (Hq / Hkv)``).

Pins (``tests/test_oracle_prefill.py``): a chunk of one token is decode
attention; the whole prompt as one chunk equals textbook causal attention in
explicit loops; the first position returns its own V row; splitting a chunk in
two changes nothing.  ``causal_chunk_ref`` (the same definition with the scores
of a block of queries taken as one matrix product) equals ``prefill_ref`` and
the explicit-loop brute force, and a causal bound one key too wide fails it.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import attention_ref, gather_seq
from .numerics import to_f64


def prefill_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_tables: np.ndarray,
                context_lens: Sequence[int], query_start: Sequence[int], scale: float, num_kv_heads: int,
                dtype: str, seqs: Sequence[int] = None) -> np.ndarray:
    """q: [Tq, Hq, D] storage dtype (Tq = query_start[-1]); caches [NB, bs, Hkv, D]
    storage dtype.  Returns float64 [Tq, Hq, D] (rows of unlisted sequences are
    left zero when ``seqs`` is given)."""
    tq, hq, d = q.shape
    S = len(context_lens)
    assert len(query_start) == S + 1 and int(query_start[-1]) == tq
    out = np.zeros((tq, hq, d), dtype=np.float64)
    for s in (range(S) if seqs is None else seqs):
        L = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        C = q1 - q0
        assert 0 <= C <= L
        k = to_f64(gather_seq(k_cache, block_tables[s], L), dtype)
        v = to_f64(gather_seq(v_cache, block_tables[s], L), dtype)
        for j in range(C):
            p = L - C + j
            out[q0 + j] = attention_ref(to_f64(q[q0 + j], dtype), k[:p + 1], v[:p + 1], scale)
    return out


def run_prefill(wl, *, compute_out: bool = True, seqs: Sequence[int] = None):
    """Oracle side of a prefill workload: the block manager places every token
    of every sequence, ``scatter_ref`` writes their rows, and ``prefill_ref``
    evaluates the chunks.  Returns (k_cache, v_cache, block_tables, out)."""
    from .block_manager import BlockManager
    from .cache_ops import new_cache, scatter_ref

    npdt = {"fp16": np.float16, "bf16": np.uint16}[wl.dtype]
    bm = BlockManager(wl.pool_blocks, 16, wl.free_order)
    kc, vc = new_cache(wl.pool_blocks, 16, wl.num_kv_heads, 128, npdt)
    for s in range(wl.num_seqs):
        slots = bm.add(s, int(wl.context_lens[s]))
        k, v = wl.seq_kv(s)
        scatter_ref(kc, vc, k, v, slots)
    max_blocks = max(len(bm.blocks[s]) for s in range(wl.num_seqs))
    tables = bm.block_table(range(wl.num_seqs), max_blocks)
    out = None
    if compute_out:
        out = prefill_ref(wl.q, kc, vc, tables, wl.context_lens, wl.query_start, wl.scale, wl.num_kv_heads,
                          wl.dtype, seqs=seqs)
    return kc, vc, tables, out


def causal_chunk_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float, first_pos: int,
                     row_block: int = 128) -> np.ndarray:
    """Every query of one sequence's chunk, by matrix products.

    q: float64 [C, Hq, D], chunk query j at absolute position first_pos + j;
    k, v: float64 [L, Hkv, D] with L >= first_pos + C (the sequence's rows in
    logical order).  The same definition as ``prefill_ref``: for each KV head,
    the scores of its query heads against the keys are one product over a
    block of queries, keys past a query's position get weight zero (the causal
    bound), then the softmax with its maximum shift and the weighted sum of V
    rows.  Returns float64 [C, Hq, D].
    """
    C, hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    assert first_pos >= 0 and first_pos + C <= L
    pos = first_pos + np.arange(C)
    out = np.empty((C, hq, d), dtype=np.float64)
    for j in range(hkv):
        kj = np.ascontiguousarray(k[:, j, :])
        vj = np.ascontiguousarray(v[:, j, :])
        heads = slice(j * g, (j + 1) * g)
        for r0 in range(0, C, row_block):
            r1 = min(C, r0 + row_block)
            n = int(pos[r1 - 1]) + 1  # keys any row of this block can see
            qq = q[r0:r1, heads, :]  # [R, g, D]
            logits = scale * (qq.reshape(-1, d) @ kj[:n].T).reshape(r1 - r0, g, n)
            visible = np.arange(n)[None, None, :] <= pos[r0:r1, None, None]
            logits = np.where(visible, logits, -np.inf)
            m = logits.max(axis=-1, keepdims=True)
            w = np.exp(logits - m)  # exactly 0 past the position
            out[r0:r1, heads] = (w @ vj[:n]) / w.sum(axis=-1, keepdims=True)
    return out
