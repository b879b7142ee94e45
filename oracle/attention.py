"""Decode attention, float64 (oracle side).

Page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §2.1
(PagedAttention), names the three steps of the kernel's work: QK dot products,
softmax normalisation and the accumulation of the V rows weighted by the
softmax ("LV 累加").  Paging only changes where K/V rows live, not the result
(page "vLLM 部署与 PagedAttention 原理 · 检索整理", item 2; page "vLLM：从
PagedAttention 长出来的开源服务栈", first section), so the oracle of paged decode
attention is the plain definition applied to the rows gathered through the
block table.

Readings where the pages are silent:

* one query token per sequence attends to all ``context_lens[s]`` tokens,
  including the one written in the same step; no mask, bias or soft-cap;
* logits are multiplied by ``scale`` before the softmax;
* query head ``h`` reads KV head ``h // (Hq // Hkv)`` (contiguous groups);
* results are float64 and unrounded: the comparison with a GPU output in
  fp16/bf16 happens in the tests.
"""

import math
from typing import List, Sequence

import numpy as np

from .numerics import to_f64


def attention_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                  return_weights: bool = False):
    """Softmax attention of one query token per head over L tokens.

    q: float64 [Hq, D]; k, v: float64 [L, Hkv, D].  Returns float64 [Hq, D]
    (and the normalised weights [Hq, L] if asked).
    """
    hq, d = q.shape
    L, hkv, _ = k.shape
    if L == 0:
        raise ValueError("softmax over an empty context")
    g = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    weights = np.empty((hq, L), dtype=np.float64)
    for h in range(hq):
        kvh = h // g
        logits = scale * (k[:, kvh, :] @ q[h])  # QK dot products, [L]
        m = logits.max()
        w = np.exp(logits - m)  # softmax numerator (any shift gives the same ratio)
        z = w.sum()
        weights[h] = w / z
        out[h] = (w @ v[:, kvh, :]) / z  # weighted sum of V rows
    if return_weights:
        return out, weights
    return out


def gather_seq(cache: np.ndarray, block_table_row: np.ndarray, length: int) -> np.ndarray:
    """Rows of tokens 0..length-1 of one sequence, in logical order, read
    through its block table: token t lives in block table[t // bs], offset t % bs."""
    bs = cache.shape[1]
    t = np.arange(length)
    blocks = np.asarray(block_table_row)[t // bs]
    return cache[blocks, t % bs]


def paged_decode_ref(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                     block_tables: np.ndarray, context_lens: Sequence[int], scale: float,
                     num_kv_heads: int, dtype: str, seqs: Sequence[int] = None) -> np.ndarray:
    """Paged decode attention for every (or every listed) sequence.

    q: [S, Hq, D] storage dtype; caches: [NB, bs, Hkv, D] storage dtype;
    block_tables: int [S, max_blocks].  Returns float64 [len(seqs), Hq, D].
    """
    S, hq, d = q.shape
    assert k_cache.shape[2] == num_kv_heads and hq % num_kv_heads == 0
    if seqs is None:
        seqs = range(S)
    out = []
    for s in seqs:
        L = int(context_lens[s])
        kt = to_f64(gather_seq(k_cache, block_tables[s], L), dtype)
        vt = to_f64(gather_seq(v_cache, block_tables[s], L), dtype)
        out.append(attention_ref(to_f64(q[s], dtype), kt, vt, scale))
    return np.stack(out) if out else np.zeros((0, hq, d))


def brute_force_ref(q: List[List[float]], k: List[List[List[float]]],
                    v: List[List[List[float]]], scale: float) -> List[List[float]]:
    """Textbook attention with explicit loops, for tiny inputs.

    q: [Hq][D]; k, v: [L][Hkv][D] nested lists of floats (contiguous, never
    paged).  out[h][d] = sum_t exp(s_t) v[t][h//g][d] / sum_t exp(s_t), with
    s_t = scale * sum_d q[h][d] k[t][h//g][d].  No max shift: inputs are small.
    """
    hq = len(q)
    L = len(k)
    hkv = len(k[0])
    D = len(q[0])
    g = hq // hkv
    out = []
    for h in range(hq):
        j = h // g
        e = []
        for t in range(L):
            dot = 0.0
            for dd in range(D):
                dot += q[h][dd] * k[t][j][dd]
            e.append(math.exp(scale * dot))
        den = math.fsum(e)
        row = []
        for dd in range(D):
            row.append(math.fsum(e[t] * v[t][j][dd] for t in range(L)) / den)
        out.append(row)
    return out


def partition_partials_ref(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                           partition_tokens: int):
    """Softmax statistics of each token partition of one sequence.

    For partition p = tokens [p*P, min((p+1)*P, L)):
      m_p = max logit, Z_p = sum exp(l - m_p), o_p = sum exp(l - m_p) v / Z_p.
    q: float64 [Hq, D]; k, v: float64 [L, Hkv, D].
    Returns m [Hq, np], z [Hq, np], o [Hq, np, D].
    """
    hq, d = q.shape
    L, hkv, _ = k.shape
    g = hq // hkv
    n = -(-L // partition_tokens)
    m = np.empty((hq, n))
    z = np.empty((hq, n))
    o = np.empty((hq, n, d))
    for p in range(n):
        lo, hi = p * partition_tokens, min((p + 1) * partition_tokens, L)
        for h in range(hq):
            logits = scale * (k[lo:hi, h // g, :] @ q[h])
            m[h, p] = logits.max()
            w = np.exp(logits - m[h, p])
            z[h, p] = w.sum()
            o[h, p] = (w @ v[lo:hi, h // g, :]) / z[h, p]
    return m, z, o


def lse_merge_ref(m: np.ndarray, z: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Recombine partition results.  With M = max_p m_p and
    c_p = Z_p exp(m_p - M): out = sum_p c_p o_p / sum_p c_p.  This follows
    from writing the full softmax sum as a sum over partitions."""
    M = m.max(axis=-1, keepdims=True)
    c = z * np.exp(m - M)
    return (c[..., None] * o).sum(axis=-2) / c.sum(axis=-1)[..., None]
