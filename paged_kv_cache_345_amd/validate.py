"""Host checks of the device-array contracts in include/pagedkv.h, run on host
copies before a call when the environment sets PKV_VALIDATE=1 (a debug aid;
the library itself never reads device contents on the host).  Each check
raises ValueError naming the first violation.  They check only what the
header states as the caller's contract; none of them computes anything of
the calls themselves."""

from __future__ import annotations

import os

import numpy as np

BLOCK_SIZE = 16


def enabled() -> bool:
    return os.environ.get("PKV_VALIDATE", "") == "1"


def _host(a) -> np.ndarray:
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.asarray(a)


def check_tables(block_tables, context_lens, num_blocks: int) -> None:
    """1 <= context_lens[s] <= 16 * max_blocks_per_seq, and the block ids of
    the first ceil(context_lens[s] / 16) table entries in [0, num_blocks)."""
    bt = _host(block_tables).astype(np.int64)
    lens = _host(context_lens).astype(np.int64)
    if bt.ndim != 2 or lens.shape != (bt.shape[0],):
        raise ValueError("block_tables must be [num_seqs, max_blocks] and context_lens [num_seqs]")
    cap = BLOCK_SIZE * bt.shape[1]
    bad = np.nonzero((lens < 1) | (lens > cap))[0]
    if bad.size:
        s = int(bad[0])
        raise ValueError(f"context_lens[{s}] = {int(lens[s])} outside [1, {cap}]")
    need = -(-lens // BLOCK_SIZE)
    live = np.arange(bt.shape[1])[None, :] < need[:, None]
    wrong = live & ((bt < 0) | (bt >= num_blocks))
    if wrong.any():
        s, j = (int(x) for x in np.argwhere(wrong)[0])
        raise ValueError(f"block_tables[{s}][{j}] = {int(bt[s, j])} outside [0, {num_blocks})")


def check_lengths(context_lens, max_blocks_per_seq: int) -> None:
    lens = _host(context_lens).astype(np.int64)
    cap = BLOCK_SIZE * max_blocks_per_seq
    bad = np.nonzero((lens < 1) | (lens > cap))[0]
    if bad.size:
        s = int(bad[0])
        raise ValueError(f"context_lens[{s}] = {int(lens[s])} outside [1, {cap}]")


def check_query_start(query_start, context_lens, num_query_tokens: int, max_query_len: int) -> None:
    """query_start non-decreasing from 0 to num_query_tokens, C_s <= context_lens[s],
    and every C_s <= max_query_len."""
    qs = _host(query_start).astype(np.int64)
    lens = _host(context_lens).astype(np.int64)
    if qs.shape != (lens.shape[0] + 1,):
        raise ValueError("query_start must be [num_seqs + 1]")
    if qs[0] != 0 or qs[-1] != num_query_tokens:
        raise ValueError(f"query_start must run from 0 to {num_query_tokens}, not {int(qs[0])} .. {int(qs[-1])}")
    c = np.diff(qs)
    for what, bad in (("decreases", c < 0), ("exceeds context_lens", c > lens), ("exceeds max_query_len",
                                                                                 c > max_query_len)):
        idx = np.nonzero(bad)[0]
        if idx.size:
            s = int(idx[0])
            raise ValueError(f"chunk {s} ({int(c[s])} queries) {what}")


def check_slots(slot_mapping, num_blocks: int) -> None:
    """Non-negative slots below num_blocks * 16 and pairwise distinct."""
    sm = _host(slot_mapping).astype(np.int64)
    live = sm[sm >= 0]
    over = live[live >= num_blocks * BLOCK_SIZE]
    if over.size:
        raise ValueError(f"slot {int(over[0])} outside the pool of {num_blocks} blocks")
    u, counts = np.unique(live, return_counts=True)
    if (counts > 1).any():
        raise ValueError(f"slot {int(u[np.argmax(counts > 1)])} written twice")


def check_copy_pairs(block_pairs, num_blocks: int) -> None:
    """Ids in [0, num_blocks), every dst distinct, no dst equal to any src."""
    bp = _host(block_pairs).astype(np.int64).reshape(-1, 2)
    if ((bp < 0) | (bp >= num_blocks)).any():
        r = int(np.argwhere((bp < 0) | (bp >= num_blocks))[0][0])
        raise ValueError(f"block_pairs[{r}] = {bp[r].tolist()} outside [0, {num_blocks})")
    _distinct_dsts(bp)
    clash = np.intersect1d(bp[:, 0], bp[:, 1])
    if clash.size:
        raise ValueError(f"block {int(clash[0])} is both a source and a destination")


def check_swap_pairs(block_pairs, src_blocks: int, dst_blocks: int) -> None:
    """Ids inside their pools (a pair outside is skipped by the call: flagged
    here as a likely mistake) and every dst distinct."""
    bp = _host(block_pairs).astype(np.int64).reshape(-1, 2)
    bad = (bp[:, 0] < 0) | (bp[:, 0] >= src_blocks) | (bp[:, 1] < 0) | (bp[:, 1] >= dst_blocks)
    if bad.any():
        r = int(np.nonzero(bad)[0][0])
        raise ValueError(f"block_pairs[{r}] = {bp[r].tolist()} outside the pools ({src_blocks}, {dst_blocks})")
    _distinct_dsts(bp)


def _distinct_dsts(bp: np.ndarray) -> None:
    u, counts = np.unique(bp[:, 1], return_counts=True)
    if (counts > 1).any():
        raise ValueError(f"destination block {int(u[np.argmax(counts > 1)])} appears twice")


def check_prologue_sources(block_pairs, slot_mapping) -> None:
    """decode_step_prologue's extra condition: a token written into the source
    block of a pair lies at an offset that is also written in the pair's
    destination."""
    bp = _host(block_pairs).astype(np.int64).reshape(-1, 2)
    slots = _host(slot_mapping).astype(np.int64)
    slots = slots[slots >= 0]
    by_block = {}
    for sl in slots.tolist():
        by_block.setdefault(sl // BLOCK_SIZE, set()).add(sl % BLOCK_SIZE)
    for src, dst in bp.tolist():
        extra = by_block.get(src, set()) - by_block.get(dst, set())
        if extra:
            raise ValueError(f"block_pairs ({src}, {dst}): tokens are written into the source block at offsets "
                             f"{sorted(extra)} that the destination does not receive")


def check_head_scales(scales, name: str) -> None:
    """Per-KV-head fp8 scales: finite and > 0."""
    x = _host(scales).astype(np.float64)
    bad = np.nonzero(~np.isfinite(x) | (x <= 0))[0]
    if bad.size:
        raise ValueError(f"{name}[{int(bad[0])}] = {x[bad[0]]} is not a finite positive scale")
