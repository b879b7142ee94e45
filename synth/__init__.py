"""Seeded synthetic workloads for paged decode attention.

This module only draws random numbers and describes workloads. It holds none of
the method's arithmetic: no attention, no paging, no slot or block-table math.
Both the oracle side (``oracle/``) and the HIP side (the package binding) take
their inputs from here, and nothing else is shared between them.

Workload shapes follow the five decode batches the paged-attention pages are
measured on (LLaMA-7B/13B-shaped serving batches, a GQA batch, a long-context
split batch, and a tiny case).  The pages' own workload draws prompt and output
lengths from ShareGPT, which is not available; the lognormal and uniform length
recipes below stand in for it.

Recipe (all streams are ``numpy.random.default_rng``):

* main stream ``default_rng(seed)``: context lengths first, then a permutation
  of the block pool (the free-list order), then per-KV-head key scales (GQA
  batch only), then the query ``[S, Hq, D]``;
* per-sequence stream ``default_rng([seed, 1, s])``: K then V rows of the tokens
  that belong to sequence ``s`` alone (all its tokens for a singleton, only the
  new token for a member of a sampling group);
* per-group stream ``default_rng([seed, 2, g])``: K then V rows of the shared
  prompt of sampling group ``g``.

Values are drawn N(0, 1) in float32 and rounded once, round-to-nearest-even, to
the storage dtype; both sides receive the rounded values.  bfloat16 values are
kept as their uint16 bit patterns because numpy has no bfloat16 type.
"""

from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional, Sequence, Tuple, Union

import numpy as np

HEAD_SIZE = 128
BLOCK_SIZE = 16

__all__ = [
    "HEAD_SIZE",
    "BLOCK_SIZE",
    "ConfigSpec",
    "CONFIGS",
    "Workload",
    "make_workload",
    "make_random_workload",
    "round_fp16",
    "round_bf16_bits",
    "storage_dtype",
    "thread_map",
    "PrefillWorkload",
    "make_prefill_workload",
    "PREFILL_CONFIGS",
    "make_prefill",
]


def thread_map(fn, items, max_workers: Optional[int] = None):
    """map() over a thread pool; numpy's generators release the GIL while
    filling large arrays, so per-sequence draws run in parallel."""
    items = list(items)
    if max_workers is None:
        max_workers = min(16, len(os.sched_getaffinity(0)))
    if max_workers <= 1 or len(items) <= 1:
        return [fn(i) for i in items]
    with ThreadPoolExecutor(max_workers) as ex:
        return list(ex.map(fn, items))


# --------------------------------------------------------------------------
# rounding of float32 draws to the storage dtype (input encoding only)
# --------------------------------------------------------------------------

def round_fp16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def round_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs are finite by construction, so no NaN special case is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    # finite inputs: u + 0x8000 cannot wrap past 0xFFFFFFFF
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def storage_dtype(dtype: str):
    if dtype == "fp16":
        return np.float16
    if dtype == "bf16":
        return np.uint16
    raise ValueError(f"unknown dtype {dtype!r}")


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_fp16(x) if dtype == "fp16" else round_bf16_bits(x)


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class ConfigSpec:
    name: str
    seed: int
    num_seqs: int
    num_heads: int
    num_kv_heads: int
    dtype: str
    lengths: Tuple  # ("fixed", [...]) | ("lognormal", median, sigma, cap) | ("uniform", lo, hi)
    pool_blocks: int  # physical pool size (1.1x the blocks the batch needs; C1: 64)
    group_fraction: float = 0.0  # fraction of sequences in sampling groups of 3
    key_scale: Optional[Tuple[float, float]] = None  # per-KV-head U[lo, hi] key scale
    partition_tokens: int = 0  # 0: library default
    description: str = ""
    kv_dtype: Optional[str] = None  # "fp8e4m3": the cache stores E4M3 codes of the rows
    # fp8 cache: dequantised K = code value * k_scale, one float per cache or a
    # tuple of one float per KV head (likewise V)
    k_scale: Union[float, Tuple[float, ...]] = 1.0
    v_scale: Union[float, Tuple[float, ...]] = 1.0
    # > 0: the K scale of KV head h is this times the batch's key scale of
    # head h (per-head scales that follow the heads' key magnitudes)
    k_scale_per_key_scale: float = 0.0

    @property
    def group_size(self) -> int:
        return self.num_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_SIZE)


CONFIGS: Dict[str, ConfigSpec] = {
    "tiny": ConfigSpec(
        name="tiny", seed=1, num_seqs=4, num_heads=8, num_kv_heads=8, dtype="fp16",
        lengths=("fixed", (17, 33, 100, 250)), pool_blocks=64,
        description="4 sequences, contexts {17,33,100,250}, 8/8 heads, fp16, 64-block pool"),
    "llama7b": ConfigSpec(
        name="llama7b", seed=2, num_seqs=64, num_heads=32, num_kv_heads=32, dtype="fp16",
        lengths=("lognormal", 400.0, 1.0, 2048), pool_blocks=2731,
        description="LLaMA-7B-shaped decode batch: 64 seqs, 32 MHA heads, fp16, "
                    "lognormal contexts (median 400, cap 2048), pool 1.1x"),
    "llama13b": ConfigSpec(
        name="llama13b", seed=3, num_seqs=128, num_heads=40, num_kv_heads=40, dtype="fp16",
        lengths=("lognormal", 600.0, 1.0, 2048), pool_blocks=5548, group_fraction=0.3,
        description="LLaMA-13B-shaped decode batch: 128 seqs, 40 MHA heads, fp16, "
                    "lognormal contexts (median 600, cap 2048), 13 groups of 3 "
                    "parallel samples sharing prompt blocks, copy-on-write"),
    "gqa": ConfigSpec(
        name="gqa", seed=4, num_seqs=256, num_heads=64, num_kv_heads=8, dtype="bf16",
        lengths=("uniform", 1024, 8192), pool_blocks=83223, key_scale=(0.5, 2.0),
        description="GQA decode batch: 256 seqs, 64 query / 8 KV heads, bf16, "
                    "contexts U[1024,8192], per-KV-head key scale U[0.5,2]"),
    # 512-token partitions: each wave of a decode work-group streams one
    # 512-token partition of a 2048-token segment; the 4 partitions are merged
    # in the work-group and the segments by the log-sum-exp reduce kernel
    "long": ConfigSpec(
        name="long", seed=5, num_seqs=8, num_heads=32, num_kv_heads=8, dtype="bf16",
        lengths=("uniform", 32768, 131072), pool_blocks=46457, partition_tokens=2048,
        description="long-context split decode: 8 seqs, 32 query / 8 KV heads, bf16, "
                    "contexts U[32768,131072], 512-token partitions (4 per 2048-token segment)"),
}

# fp8 (E4M3) cache variants of two batches: same lengths, pools and values;
# the cache holds E4M3 codes of the rows under one float32 scale per cache
# (max |row| / scale stays near the E4M3 limit of 448 for N(0,1) rows)
CONFIGS["llama13b_fp8"] = replace(
    CONFIGS["llama13b"], name="llama13b_fp8", kv_dtype="fp8e4m3", k_scale=0.0125, v_scale=0.0125,
    description="LLaMA-13B-shaped decode batch over an fp8 (E4M3) cache: 128 seqs, 40 MHA heads, "
                "fp16 queries, lognormal contexts (median 600, cap 2048), 13 groups of 3 parallel "
                "samples, K/V scales 0.0125")
CONFIGS["gqa_fp8"] = replace(
    CONFIGS["gqa"], name="gqa_fp8", kv_dtype="fp8e4m3", k_scale_per_key_scale=0.0125, v_scale=0.0125,
    description="GQA decode batch over an fp8 (E4M3) cache: 256 seqs, 64 query / 8 KV heads, bf16 "
                "queries, contexts U[1024,8192], per-KV-head key scale U[0.5,2]; per-KV-head K scales "
                "0.0125 x the head's key scale, one V scale 0.0125")


# --------------------------------------------------------------------------
# workload
# --------------------------------------------------------------------------

@dataclass
class Workload:
    """A decode step: each sequence has ``context_lens[s] - 1`` tokens already in
    the cache and appends one new token, whose K/V is written through the slot
    mapping before attention reads all ``context_lens[s]`` tokens.

    ``ops`` describes the block-manager calls that build this state, in order:
      ("add", seq, n_tokens)   a new sequence with n_tokens prior tokens
      ("fork", parent, child)  child shares all of parent's blocks
      ("step", [seq, ...])     append one token to each listed sequence
    """

    spec: ConfigSpec
    context_lens: np.ndarray  # int64 [S]
    free_order: np.ndarray  # int32 [pool]
    q: np.ndarray  # storage dtype [S, Hq, D]
    key_scales: Optional[np.ndarray]  # float32 [Hkv] or None
    groups: List[Tuple[int, int, int]]  # (first_seq, n_samples, prompt_len)
    ops: List[tuple] = field(default_factory=list)

    # ---- shape helpers -------------------------------------------------
    @property
    def num_seqs(self) -> int:
        return self.spec.num_seqs

    @property
    def num_heads(self) -> int:
        return self.spec.num_heads

    @property
    def num_kv_heads(self) -> int:
        return self.spec.num_kv_heads

    @property
    def dtype(self) -> str:
        return self.spec.dtype

    @property
    def kv_dtype(self) -> str:
        """Storage type of the cache: the activation dtype, or "fp8e4m3"."""
        return self.spec.kv_dtype or self.spec.dtype

    @property
    def k_scale(self):
        """fp8 cache: the K scale, a float (one per cache) or float32 [Hkv]."""
        if self.spec.k_scale_per_key_scale > 0:
            return (np.float32(self.spec.k_scale_per_key_scale) * self.key_scales).astype(np.float32)
        return _scale_value(self.spec.k_scale)

    @property
    def v_scale(self):
        return _scale_value(self.spec.v_scale)

    @property
    def pool_blocks(self) -> int:
        return int(self.free_order.shape[0])

    @property
    def scale(self) -> float:
        return self.spec.scale

    def group_of(self, s: int) -> Optional[int]:
        for g, (first, n, _p) in enumerate(self.groups):
            if first <= s < first + n:
                return g
        return None

    # ---- value streams ---------------------------------------------------
    def _draw_kv(self, rng: np.random.Generator, n: int):
        hkv = self.num_kv_heads
        k = rng.standard_normal((n, hkv, HEAD_SIZE), dtype=np.float32)
        if self.key_scales is not None:
            k *= self.key_scales[None, :, None]
        v = rng.standard_normal((n, hkv, HEAD_SIZE), dtype=np.float32)
        return _to_storage(k, self.dtype), _to_storage(v, self.dtype)

    def group_prompt_kv(self, g: int):
        _first, _n, plen = self.groups[g]
        rng = np.random.default_rng([self.spec.seed, 2, g])
        return self._draw_kv(rng, plen)

    def own_kv(self, s: int):
        """K/V rows that belong to sequence s alone (all of them for a
        singleton, only the newly decoded token for a group member)."""
        g = self.group_of(s)
        n = 1 if g is not None else int(self.context_lens[s])
        rng = np.random.default_rng([self.spec.seed, 1, s])
        return self._draw_kv(rng, n)

    def seq_kv(self, s: int):
        """Contiguous K/V of all context_lens[s] tokens of sequence s, in
        logical order: [L_s, Hkv, D] each (storage dtype)."""
        g = self.group_of(s)
        k_own, v_own = self.own_kv(s)
        if g is None:
            return k_own, v_own
        k_p, v_p = self.group_prompt_kv(g)
        return np.concatenate([k_p, k_own]), np.concatenate([v_p, v_own])

    def new_token_kv(self):
        """K/V of the token each sequence appends in the step: [S, Hkv, D]."""
        ks, vs = [], []
        for s in range(self.num_seqs):
            k, v = self.own_kv(s)
            ks.append(k[-1])
            vs.append(v[-1])
        return np.stack(ks), np.stack(vs)

    def prior_kv_for_add(self, seq: int):
        """K/V of the prior tokens created by the ("add", seq, n) op."""
        g = self.group_of(seq)
        if g is not None:
            return self.group_prompt_kv(g)
        k, v = self.own_kv(seq)
        n = int(self.context_lens[seq]) - 1
        return k[:n], v[:n]

    @property
    def total_context(self) -> int:
        return int(self.context_lens.sum())


def _scale_value(x):
    """A float stays a float; a tuple of per-head scales becomes float32 [Hkv]."""
    return np.asarray(x, dtype=np.float32) if isinstance(x, (tuple, list, np.ndarray)) else float(x)


def _as_spec_scale(x):
    return tuple(float(v) for v in x) if isinstance(x, (tuple, list, np.ndarray)) else float(x)


def _draw_lengths(spec: ConfigSpec, rng: np.random.Generator):
    kind = spec.lengths[0]
    S = spec.num_seqs
    groups: List[Tuple[int, int, int]] = []
    if kind == "fixed":
        lens = np.asarray(spec.lengths[1], dtype=np.int64)
        assert lens.shape[0] == S
        return lens, groups
    if kind == "lognormal":
        _, median, sigma, cap = spec.lengths
        n_groups = int(round(spec.group_fraction * S / 3))
        if n_groups:
            plen = rng.lognormal(math.log(median), sigma, n_groups)
            plen = np.clip(np.rint(plen), 1, cap - 1).astype(np.int64)
        n_single = S - 3 * n_groups
        x = rng.lognormal(math.log(median), sigma, n_single)
        single = np.clip(np.rint(x), 1, cap).astype(np.int64)
        lens = []
        for g in range(n_groups):
            groups.append((3 * g, 3, int(plen[g])))
            lens += [int(plen[g]) + 1] * 3
        lens += [int(v) for v in single]
        return np.asarray(lens, dtype=np.int64), groups
    if kind == "uniform":
        _, lo, hi = spec.lengths
        return rng.integers(lo, hi, S, endpoint=True).astype(np.int64), groups
    raise ValueError(kind)


def _ops_for(lens: np.ndarray, groups: Sequence[Tuple[int, int, int]]) -> List[tuple]:
    ops: List[tuple] = []
    S = int(lens.shape[0])
    member = {}
    for first, n, plen in groups:
        for i in range(n):
            member[first + i] = (first, plen)
    for s in range(S):
        if s in member:
            first, plen = member[s]
            if s == first:
                ops.append(("add", s, plen))
            else:
                ops.append(("fork", first, s))
        else:
            ops.append(("add", s, int(lens[s]) - 1))
    ops.append(("step", list(range(S))))
    return ops


def make_workload(name_or_spec, *, with_q: bool = True) -> Workload:
    spec = CONFIGS[name_or_spec] if isinstance(name_or_spec, str) else name_or_spec
    rng = np.random.default_rng(spec.seed)
    lens, groups = _draw_lengths(spec, rng)
    free_order = rng.permutation(spec.pool_blocks).astype(np.int32)
    key_scales = None
    if spec.key_scale is not None:
        lo, hi = spec.key_scale
        key_scales = rng.uniform(lo, hi, spec.num_kv_heads).astype(np.float32)
    q = None
    if with_q:
        q = _to_storage(
            rng.standard_normal((spec.num_seqs, spec.num_heads, HEAD_SIZE), dtype=np.float32),
            spec.dtype)
    return Workload(spec=spec, context_lens=lens, free_order=free_order, q=q,
                    key_scales=key_scales, groups=groups, ops=_ops_for(lens, groups))


def make_random_workload(seed: int, *, num_seqs: int, num_heads: int, num_kv_heads: int,
                         dtype: str, max_len: int, pool_slack: int = 4,
                         min_len: int = 1, groups: int = 0, group_size: int = 3,
                         key_scale=None, kv_dtype: Optional[str] = None, k_scale=1.0,
                         v_scale=1.0) -> Workload:
    """Small random workload for property tests: lengths U[min_len, max_len],
    optionally the first group_size*groups sequences in sampling groups of
    group_size."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(min_len, max_len, num_seqs, endpoint=True).astype(np.int64)
    grp = []
    n = group_size
    for g in range(groups):
        plen = int(max(1, min(lens[n * g], max_len) - 1))
        grp.append((n * g, n, plen))
        lens[n * g:n * g + n] = plen + 1
    # generous pool: every token its own block would still fit
    pool = int(sum(-(-int(v) // BLOCK_SIZE) + 1 for v in lens)) + n * groups + pool_slack
    spec = ConfigSpec(name=f"random{seed}", seed=seed, num_seqs=num_seqs, num_heads=num_heads,
                      num_kv_heads=num_kv_heads, dtype=dtype,
                      lengths=("fixed", tuple(int(v) for v in lens)), pool_blocks=pool,
                      key_scale=key_scale, kv_dtype=kv_dtype, k_scale=_as_spec_scale(k_scale),
                      v_scale=_as_spec_scale(v_scale))
    free_order = rng.permutation(pool).astype(np.int32)
    key_scales = None
    if key_scale is not None:
        key_scales = rng.uniform(key_scale[0], key_scale[1], num_kv_heads).astype(np.float32)
    q = _to_storage(rng.standard_normal((num_seqs, num_heads, HEAD_SIZE), dtype=np.float32), dtype)
    return Workload(spec=spec, context_lens=lens, free_order=free_order, q=q,
                    key_scales=key_scales, groups=grp, ops=_ops_for(lens, grp))


# --------------------------------------------------------------------------
# chunked prefill (multi-token queries over the paged cache)
# --------------------------------------------------------------------------

@dataclass
class PrefillWorkload:
    """Sequence s holds ``context_lens[s]`` tokens in the cache (all written by
    the slot-mapped write); its last ``chunk_lens[s]`` tokens are the chunk whose
    queries attend causally to the cache.  ``q`` is ``[sum(chunk_lens), Hq, D]``,
    sequence-major.  Streams: main ``default_rng(seed)`` (lengths, chunk lengths,
    pool permutation, q), per-sequence ``default_rng([seed, 3, s])`` (K then V
    rows of all its tokens)."""

    name: str
    seed: int
    num_heads: int
    num_kv_heads: int
    dtype: str
    context_lens: np.ndarray  # int64 [S]
    chunk_lens: np.ndarray  # int64 [S]
    free_order: np.ndarray  # int32 [pool]
    q: np.ndarray  # storage dtype [Tq, Hq, D]
    key_scales: Optional[np.ndarray] = None
    description: str = ""
    kv_dtype: Optional[str] = None  # "fp8e4m3": the cache holds E4M3 codes of the rows
    k_scale: Union[float, np.ndarray] = 1.0  # a float (one per cache) or float32 [Hkv]
    v_scale: Union[float, np.ndarray] = 1.0

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def pool_blocks(self) -> int:
        return int(self.free_order.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_SIZE)

    @property
    def query_start(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.chunk_lens)]).astype(np.int64)

    @property
    def num_query_tokens(self) -> int:
        return int(self.chunk_lens.sum())

    def seq_kv(self, s: int):
        """K, V rows of all context_lens[s] tokens of sequence s: [L_s, Hkv, D]."""
        rng = np.random.default_rng([self.seed, 3, s])
        n, hkv = int(self.context_lens[s]), self.num_kv_heads
        k = rng.standard_normal((n, hkv, HEAD_SIZE), dtype=np.float32)
        if self.key_scales is not None:
            k *= self.key_scales[None, :, None]
        v = rng.standard_normal((n, hkv, HEAD_SIZE), dtype=np.float32)
        return _to_storage(k, self.dtype), _to_storage(v, self.dtype)


def make_prefill_workload(seed: int, *, num_seqs: int, num_heads: int, num_kv_heads: int, dtype: str,
                          context: Tuple[int, int], chunk: Tuple[int, int], key_scale=None, pool_slack: int = 4,
                          name: str = "", description: str = "", kv_dtype: Optional[str] = None,
                          k_scale=1.0, v_scale=1.0) -> PrefillWorkload:
    """Contexts U[context], chunk lengths U[chunk] clipped to the context.  fp8
    scales: a float, or one float per KV head."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(context[0], context[1], num_seqs, endpoint=True).astype(np.int64)
    chunks = np.minimum(rng.integers(chunk[0], chunk[1], num_seqs, endpoint=True), lens).astype(np.int64)
    pool = int(sum(-(-int(L) // BLOCK_SIZE) for L in lens)) + pool_slack
    free_order = rng.permutation(pool).astype(np.int32)
    key_scales = None
    if key_scale is not None:
        key_scales = rng.uniform(key_scale[0], key_scale[1], num_kv_heads).astype(np.float32)
    q = _to_storage(rng.standard_normal((int(chunks.sum()), num_heads, HEAD_SIZE), dtype=np.float32), dtype)
    return PrefillWorkload(name=name or f"prefill{seed}", seed=seed, num_heads=num_heads, num_kv_heads=num_kv_heads,
                           dtype=dtype, context_lens=lens, chunk_lens=chunks, free_order=free_order, q=q,
                           key_scales=key_scales, description=description, kv_dtype=kv_dtype,
                           k_scale=_scale_value(k_scale), v_scale=_scale_value(v_scale))


PREFILL_CONFIGS = {
    "prefill_llama13b": dict(seed=21, num_seqs=16, num_heads=40, num_kv_heads=40, dtype="fp16",
                             context=(1024, 4096), chunk=(512, 512),
                             description="chunked prefill, LLaMA-13B-shaped: 16 seqs, 40 MHA heads, fp16, "
                                         "contexts U[1024,4096], the last 512 tokens of each as the chunk"),
    "prefill_llama13b_fp8": dict(seed=21, num_seqs=16, num_heads=40, num_kv_heads=40, dtype="fp16",
                                 context=(1024, 4096), chunk=(512, 512), kv_dtype="fp8e4m3", k_scale=0.0125,
                                 v_scale=0.0125,
                                 description="chunked prefill, LLaMA-13B-shaped, over an fp8 (E4M3) cache: 16 seqs, "
                                             "40 MHA heads, fp16 queries, contexts U[1024,4096], 512-token chunks"),
    "prefill_gqa": dict(seed=22, num_seqs=16, num_heads=64, num_kv_heads=8, dtype="bf16",
                        context=(1024, 8192), chunk=(512, 512), key_scale=(0.5, 2.0),
                        description="chunked prefill, GQA: 16 seqs, 64 query / 8 KV heads, bf16, "
                                    "contexts U[1024,8192], the last 512 tokens of each as the chunk"),
}


def make_prefill(name: str) -> PrefillWorkload:
    cfg = dict(PREFILL_CONFIGS[name])
    return make_prefill_workload(cfg.pop("seed"), name=name, **cfg)


# --------------------------------------------------------------------------
# prefix caching: requests that share system prompts, in two phases
# --------------------------------------------------------------------------

@dataclass
class PrefixCacheWorkload:
    """Requests built as (a prefix of one of a few system prompts) + (their own
    tokens), served in two phases: phase 1 adds ``phase1`` requests; then the
    requests in ``freed`` finish; phase 2 adds the remaining requests while
    every phase-1 survivor decodes one token.  A phase-2 request with
    ``req_parent[r] >= 0`` is the next turn of a finished request: its prompt
    is that request's prompt followed by its own tokens.  Token ids and K/V
    rows of a shared prefix are the same in every request that holds it (K/V of
    a token is a function of its whole prefix, and these prefixes are equal).

    Streams: main ``default_rng(seed)`` (prompt lengths, request shapes, freed
    set, pool permutation); system prompt j: ids ``default_rng([seed, 4, j])``,
    K then V ``default_rng([seed, 5, j])``; request r: ids then K then V
    ``default_rng([seed, 6, r])``; the decode token of r: id then K then V
    ``default_rng([seed, 7, r])``; q rows of r's positions 0 .. L_r
    ``default_rng([seed, 8, r])``."""

    seed: int
    num_heads: int
    num_kv_heads: int
    dtype: str
    sys_lens: np.ndarray    # int64 [P]
    req_sys: np.ndarray     # int64 [R]: which system prompt
    req_keep: np.ndarray    # int64 [R]: how many of its tokens the request starts with
    req_own: np.ndarray     # int64 [R]: own tokens after them (>= 1)
    req_parent: np.ndarray  # int64 [R]: the finished request this one continues, or -1
    phase1: int
    freed: np.ndarray       # int64: phase-1 requests that finish before phase 2
    free_order: np.ndarray  # int32 [pool]
    kv_dtype: Optional[str] = None
    k_scale: float = 1.0
    v_scale: float = 1.0
    vocab: int = 32000

    @property
    def num_requests(self) -> int:
        return int(self.req_sys.shape[0])

    @property
    def pool_blocks(self) -> int:
        return int(self.free_order.shape[0])

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(HEAD_SIZE)

    def prompt_len(self, r: int) -> int:
        p = int(self.req_parent[r])
        base = self.prompt_len(p) if p >= 0 else int(self.req_keep[r])
        return base + int(self.req_own[r])

    def _sys(self, j: int):
        n = int(self.sys_lens[j])
        ids = np.random.default_rng([self.seed, 4, j]).integers(0, self.vocab, n)
        rng = np.random.default_rng([self.seed, 5, j])
        k = rng.standard_normal((n, self.num_kv_heads, HEAD_SIZE), dtype=np.float32)
        v = rng.standard_normal((n, self.num_kv_heads, HEAD_SIZE), dtype=np.float32)
        return ids, k, v

    def prompt(self, r: int):
        """(token ids int64 [L], K, V storage dtype [L, Hkv, D]) of request r's prompt."""
        own = int(self.req_own[r])
        rng = np.random.default_rng([self.seed, 6, r])
        oid = rng.integers(0, self.vocab, own)
        ok = _to_storage(rng.standard_normal((own, self.num_kv_heads, HEAD_SIZE), dtype=np.float32), self.dtype)
        ov = _to_storage(rng.standard_normal((own, self.num_kv_heads, HEAD_SIZE), dtype=np.float32), self.dtype)
        p = int(self.req_parent[r])
        if p >= 0:
            ids, k, v = self.prompt(p)
        else:
            keep = int(self.req_keep[r])
            ids, k, v = self._sys(int(self.req_sys[r]))
            ids, k, v = ids[:keep], _to_storage(k[:keep], self.dtype), _to_storage(v[:keep], self.dtype)
        return np.concatenate([ids, oid]), np.concatenate([k, ok]), np.concatenate([v, ov])

    def decode_token(self, r: int):
        """(id, K [Hkv, D], V [Hkv, D]) of the token request r decodes in phase 2."""
        rng = np.random.default_rng([self.seed, 7, r])
        tid = int(rng.integers(0, self.vocab))
        k = rng.standard_normal((self.num_kv_heads, HEAD_SIZE), dtype=np.float32)
        v = rng.standard_normal((self.num_kv_heads, HEAD_SIZE), dtype=np.float32)
        return tid, _to_storage(k, self.dtype), _to_storage(v, self.dtype)

    def q_rows(self, r: int):
        """q of request r at positions 0 .. prompt_len(r) (the last: its decode token)."""
        rng = np.random.default_rng([self.seed, 8, r])
        q = rng.standard_normal((self.prompt_len(r) + 1, self.num_heads, HEAD_SIZE), dtype=np.float32)
        return _to_storage(q, self.dtype)


def make_prefix_cache_workload(seed: int, *, num_heads: int = 8, num_kv_heads: int = 2, dtype: str = "fp16",
                               sys_lens=(40, 150, 300), phase1: int = 12, phase2: int = 12,
                               own: Tuple[int, int] = (1, 120), kv_dtype: Optional[str] = None,
                               k_scale: float = 1.0, v_scale: float = 1.0,
                               pool_blocks: Optional[int] = None, keep_prob: float = 0.7) -> PrefixCacheWorkload:
    """Each request takes a system prompt (uniformly), keeps all of it with
    probability ``keep_prob`` (else a uniform cut), and adds U[own] own tokens; half the
    phase-1 requests finish, and each phase-2 request continues one of them
    with probability 0.3.  The pool is the largest number of blocks the live
    requests hold without any sharing, so the run always fits and the freed,
    registered blocks must be evicted once the free list runs out.  Given
    ``pool_blocks``, the pool has that many blocks instead (everything else is
    drawn the same)."""
    rng = np.random.default_rng(seed)
    sys_lens = np.asarray(sys_lens, dtype=np.int64)
    R = phase1 + phase2
    req_sys = rng.integers(0, len(sys_lens), R)
    full = rng.random(R) < keep_prob
    cut = np.array([rng.integers(0, sys_lens[j] + 1) for j in req_sys], dtype=np.int64)
    req_keep = np.where(full, sys_lens[req_sys], cut).astype(np.int64)
    req_own = rng.integers(own[0], own[1], R, endpoint=True).astype(np.int64)
    freed = np.sort(rng.choice(phase1, phase1 // 2, replace=False)).astype(np.int64)
    follow = rng.random(R) < 0.3
    pick = rng.integers(0, max(1, freed.shape[0]), R)
    req_parent = np.full(R, -1, dtype=np.int64)
    if freed.shape[0]:
        req_parent[phase1:] = np.where(follow[phase1:], freed[pick[phase1:]], -1)
    blocks = lambda n: -(-int(n) // BLOCK_SIZE)  # noqa: E731
    L = np.array([req_keep[r] + req_own[r] if req_parent[r] < 0 else req_keep[req_parent[r]]
                  + req_own[req_parent[r]] + req_own[r] for r in range(R)], dtype=np.int64)
    peak1 = sum(blocks(L[r]) for r in range(phase1))
    peak2 = (sum(blocks(L[r] + 1) for r in range(phase1) if r not in set(freed.tolist()))
             + sum(blocks(L[r]) for r in range(phase1, R)))
    pool = max(peak1, peak2) if pool_blocks is None else int(pool_blocks)
    free_order = rng.permutation(pool).astype(np.int32)
    return PrefixCacheWorkload(seed=seed, num_heads=num_heads, num_kv_heads=num_kv_heads, dtype=dtype,
                               sys_lens=sys_lens, req_sys=req_sys, req_keep=req_keep, req_own=req_own,
                               req_parent=req_parent, phase1=phase1, freed=freed, free_order=free_order, kv_dtype=kv_dtype,
                               k_scale=k_scale, v_scale=v_scale)


PREFIX_CONFIGS = {
    "prefix_llama13b": dict(seed=31, num_heads=40, num_kv_heads=40, dtype="fp16", sys_lens=(1024,), phase1=1,
                            phase2=64, own=(128, 512), keep_prob=1.0,
                            description="prefix-cached prompt admission, LLaMA-13B-shaped: 40 MHA heads, fp16; "
                                        "64 new prompts = one shared 1024-token system prompt (already served "
                                        "once) + U[128,512] own tokens"),
}


def make_prefix(name: str):
    cfg = dict(PREFIX_CONFIGS[name])
    desc = cfg.pop("description")
    return make_prefix_cache_workload(cfg.pop("seed"), **cfg), desc
