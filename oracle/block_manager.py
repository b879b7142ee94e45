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

Prefix caching (page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM
推理引擎", §2.2: the cache of an identical prefix, such as a shared system
prompt, is computed once and reused by later requests).  The page gives the
purpose, not the policy; the reading taken here:

* a full block whose token ids are known is registered in a table under the
  pair (node of the previous block of its chain, its token ids); node ids are
  drawn from a counter that never repeats, 0 standing for "no previous block",
  so a key names one whole token prefix;
* ``add_cached`` walks the new prompt's full blocks through that table and
  reuses the longest matching run (reference count + 1); the rest are fresh
  blocks, and fresh full blocks are registered;
* ``append_token`` is ``append_slot`` for a token whose id is known; the block
  it fills is registered, unless a block with that key exists already (then
  the chain follows the existing block's node and this block stays private);
  a token appended without an id (``append_slot``, ``step``) ends registration
  for the rest of that sequence;
* a registered block whose count drops to 0 is "evictable": it keeps its key,
  a later hit revives it, and allocation takes it (least recently freed first,
  dropping its key) only once the free list is empty.
"""

from collections import OrderedDict, deque
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
        # prefix cache
        self.table: Dict[Tuple[int, Tuple[int, ...]], int] = {}  # key -> block
        self.key: Dict[int, Tuple[int, Tuple[int, ...]]] = {}    # block -> its key
        self.node: Dict[int, int] = {}                           # block -> node id
        self.evictable: "OrderedDict[int, None]" = OrderedDict()  # least recently freed first
        self.chain: Dict[int, Optional[int]] = {}  # seq -> node of its last full block (None: ids unknown)
        self.pending: Dict[int, List[int]] = {}    # seq -> token ids of its partial last block
        self._next_node = 1

    # ------------------------------------------------------------------
    def _take(self) -> int:
        if self.free:
            b = self.free.popleft()
        else:  # evict the least recently freed registered block
            b, _ = self.evictable.popitem(last=False)
            del self.table[self.key.pop(b)]
            del self.node[b]
        assert self.ref[b] == 0
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            if b in self.key:
                self.evictable[b] = None
            else:
                self.free.append(b)

    def _filled(self, seq: int, b: int, tokens: Sequence[int]) -> None:
        """Block b of ``seq`` now holds ``tokens`` (a whole block): register it."""
        parent = self.chain[seq]
        if parent is None:
            return
        k = (parent, tuple(int(t) for t in tokens))
        if k in self.table:
            self.chain[seq] = self.node[self.table[k]]
            return
        self.table[k] = b
        self.key[b] = k
        self.node[b] = self._next_node
        self.chain[seq] = self._next_node
        self._next_node += 1

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
        if need > self.num_free():
            raise OutOfBlocks(f"need {need} blocks, {self.num_free()} free")
        self.blocks[seq] = [self._take() for _ in range(need)]
        self.length[seq] = num_tokens
        self.chain[seq] = None
        self.pending[seq] = []
        return [self._slot(seq, t) for t in range(num_tokens)]

    def add_cached(self, seq: int, token_ids: Sequence[int]) -> Tuple[List[int], int]:
        """New sequence with these token ids, reusing the registered blocks of
        its longest cached prefix.  Returns (slots, tokens already cached)."""
        if seq in self.blocks:
            raise ValueError(f"sequence {seq} exists")
        ids = [int(t) for t in token_ids]
        bs = self.block_size
        full = len(ids) // bs
        hits, parent = [], 0
        while len(hits) < full:
            j = len(hits)
            b = self.table.get((parent, tuple(ids[j * bs:(j + 1) * bs])))
            if b is None:
                break
            hits.append(b)
            parent = self.node[b]
        need = -(-len(ids) // bs) - len(hits)
        avail = self.num_free() - sum(1 for b in hits if b in self.evictable)
        if need > avail:
            raise OutOfBlocks(f"need {need} blocks, {avail} available")
        for b in hits:
            self.evictable.pop(b, None)
            self.ref[b] += 1
        self.blocks[seq] = list(hits)
        self.chain[seq] = parent
        for j in range(len(hits), len(hits) + need):
            b = self._take()
            self.blocks[seq].append(b)
            if j < full:
                self._filled(seq, b, ids[j * bs:(j + 1) * bs])
        self.length[seq] = len(ids)
        self.pending[seq] = ids[full * bs:]
        return [self._slot(seq, t) for t in range(len(ids))], len(hits) * bs

    def fork(self, parent: int, child: int) -> None:
        """``child`` shares every block of ``parent`` (reference count +1)."""
        if child in self.blocks:
            raise ValueError(f"sequence {child} exists")
        blocks = self.blocks[parent]
        for b in blocks:
            self.ref[b] += 1
        self.blocks[child] = list(blocks)
        self.length[child] = self.length[parent]
        self.chain[child] = self.chain[parent]
        self.pending[child] = list(self.pending[parent])

    def append_slot(self, seq: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """Room for one more token; returns (slot, copy pair or None)."""
        bs = self.block_size
        pos = self.length[seq]
        blocks = self.blocks[seq]
        cow = None
        if pos % bs == 0:
            if not self.num_free():
                raise OutOfBlocks("no free block for a new token")
            blocks.append(self._take())
        else:
            old = blocks[pos // bs]
            if self.ref[old] > 1:
                if not self.num_free():
                    raise OutOfBlocks("no free block for copy-on-write")
                new = self._take()
                self.ref[old] -= 1
                blocks[pos // bs] = new
                cow = (old, new)
        self.length[seq] = pos + 1
        self.chain[seq] = None  # a token without an id
        self.pending[seq] = []
        return self._slot(seq, pos), cow

    def append_token(self, seq: int, token_id: int) -> Tuple[int, Optional[Tuple[int, int]]]:
        """``append_slot`` for a token whose id is known (prefix caching)."""
        chain, pend = self.chain[seq], self.pending[seq]
        slot, cow = self.append_slot(seq)
        if chain is not None:
            self.chain[seq] = chain
            self.pending[seq] = pend + [int(token_id)]
            if len(self.pending[seq]) == self.block_size:
                self._filled(seq, self.blocks[seq][-1], self.pending[seq])
                self.pending[seq] = []
        return slot, cow

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
        if need > self.num_free():
            raise OutOfBlocks(f"step needs {need} blocks, {self.num_free()} free")
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
            self._release(b)
        del self.length[seq], self.chain[seq], self.pending[seq]

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
        """Blocks an allocation can take: the free list and the evictable blocks."""
        return len(self.free) + len(self.evictable)

    def num_evictable(self) -> int:
        return len(self.evictable)

    def num_used(self) -> int:
        return self.num_blocks - self.num_free()
