"""Block manager for a paged KV cache (oracle side, plain Python).

Follows the mechanism described on page "vLLM 部署与 PagedAttention 原理 ·
检索整理（CSDN 频道批次）", item 2 (the 2023 vLLM blog), and page "vLLM：从
PagedAttention 长出来的开源服务栈，200+ 模型架构与五维并行", section
"把显存当虚拟内存管：PagedAttention 之后的一整套服务栈":

* the KV cache is cut into blocks of a fixed number of tokens;
* each sequence's logical blocks map to physical blocks through a block table,
  and those physical blocks need not be contiguous;
* physical blocks are taken only when needed, so only a sequence's last block
  can be partly empty;
* reference counts let parallel samples share prompt blocks, and a shared
  block is copied before it is written (copy-on-write).

Readings where the pages are silent:

* the free list starts in a given order (a permutation of the pool) and blocks
  are taken from its front; freed blocks go to its back, in block-table order;
* a new token at a block boundary takes a fresh block; otherwise, if the
  sequence's last block is shared (ref > 1), the appending sequence takes a
  fresh block, the pair (old, new) is recorded for a whole-block copy, and the
  old block's count drops by one — so the last of the sharing samples to append
  keeps the original block and writes into it in place;
* a slot is ``physical_block * block_size + offset``.
"""

from collections import deque
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np


class OutOfBlocks(RuntimeError):
    """The free list cannot supply the blocks a call needs."""


class BlockManager:
    def __init__(self, num_blocks: int, block_size: int = 16,
                 free_order: Optional[Sequence[int]] = None):
        if free_order is None:
            free_order = range(num_blocks)
        order = [int(b) for b in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.blocks: Dict[int, List[int]] = {}
        self.length: Dict[int, int] = {}

    # ------------------------------------------------------------------
    def _take(self) -> int:
        b = self.free.popleft()
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _slot(self, seq: int, pos: int) -> int:
        bs = self.block_size
        return self.blocks[seq][pos // bs] * bs + pos % bs

    # ------------------------------------------------------------------
    def add(self, seq: int, num_tokens: int) -> List[int]:
        """New sequence holding ``num_tokens`` tokens; returns their slots."""
        if seq in self.blocks:
            raise ValueError(f"sequence {seq} exists")
        if num_tokens < 0:
            raise ValueError("negative token count")
        need = -(-num_tokens // self.block_size)
        if need > len(self.free):
            raise OutOfBlocks(f"need {need} blocks, {len(self.free)} free")
        self.blocks[seq] = [self._take() for _ in range(need)]
        self.length[seq] = num_tokens
        return [self._slot(seq, t) for t in range(num_tokens)]

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (reference count +1)."""
        if child in self.blocks:
            raise ValueError(f"sequence {child} exists")
        blocks = self.blocks[parent]
        for b in blocks:
            self.ref[b] += 1
        self.blocks[child] = list(blocks)
        self.length[child] = self.length[parent]

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Room for one more token; returns (slot, copy pair or None)."""
        bs = self.block_size
        pos = self.length[seq]
        blocks = self.blocks[seq]
        cow = None
        if pos % bs == 0:
            if not self.free:
                raise OutOfBlocks("no free block for a new token")
            blocks.append(self._take())
        else:
            old = blocks[pos // bs]
            if self.ref[old] > 1:
                if not self.free:
                    raise OutOfBlocks("no free block for copy-on-write")
                new = self._take()
                self.ref[old] -= 1
                blocks[pos // bs] = new
                cow = (old, new)
        self.length[seq] = pos + 1
        return self._slot(seq, pos), cow

    def step(self, seqs: Iterable[int]) -> Tuple[np.ndarray, np.ndarray]:
        """One decode step: append a token to each sequence, in order.
        Returns (slot_mapping int32 [n], copy pairs int32 [k, 2]).
        All or nothing: if the free list cannot cover every append, raises
        OutOfBlocks before changing any state."""
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs):
            raise ValueError("a sequence appears twice in one step")
        need = 0
        pending_ref = {}
        for s in seqs:
            pos = self.length[s]
            if pos % self.block_size == 0:
                need += 1
            else:
                b = self.blocks[s][pos // self.block_size]
                r = pending_ref.get(b, self.ref[b])
                if r > 1:
                    need += 1
                    pending_ref[b] = r - 1
        if need > len(self.free):
            raise OutOfBlocks(f"step needs {need} blocks, {len(self.free)} free")
        slots, pairs = [], []
        for s in seqs:
            slot, cow = self.append_slot(s)
            slots.append(slot)
            if cow is not None:
                pairs.append(cow)
        return (np.asarray(slots, dtype=np.int32),
                np.asarray(pairs, dtype=np.int32).reshape(-1, 2))

    def free_seq(self, seq: int) -> None:
        for b in self.blocks.pop(seq):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)
        del self.length[seq]

    # ------------------------------------------------------------------
    def block_table(self, seqs: Sequence[int], max_blocks: int) -> np.ndarray:
        """int32 [len(seqs), max_blocks]; unused entries are -1."""
        out = np.full((len(seqs), max_blocks), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            b = self.blocks[s]
            if len(b) > max_blocks:
                raise ValueError("max_blocks too small")
            out[i, :len(b)] = b
        return out

    def context_lens(self, seqs: Sequence[int]) -> np.ndarray:
        return np.asarray([self.length[s] for s in seqs], dtype=np.int32)

    def waste(self, seq: int) -> int:
        """Allocated but unused slots of one sequence."""
        return self.block_size * len(self.blocks[seq]) - self.length[seq]

    def num_free(self) -> int:
        return len(self.free)

    def num_used(self) -> int:
        return self.num_blocks - len(self.free)
