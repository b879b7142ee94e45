"""Pins of the oracle block manager and the cache write/copy references.

* semantic copy-on-write check: random add/fork/append/free sequences run
  against a flat cache; every live sequence, read through its block table,
  sees exactly the token values it was given (a write by one sample never
  changes another's view);
* reference counts equal the number of sequences holding each block, and
  used + free always covers the pool;
* waste is confined to the last block (at most block_size - 1 slots) and the
  aggregate waste on the LLaMA-shaped batches falls where the pages put it;
* the pool sizes of the synthetic batches are 1.1x the blocks they need.
"""

import json
import math
import os

import numpy as np
import pytest

import synth
from oracle import BlockManager, OutOfBlocks, copy_ref, new_cache, scatter_ref

BS = 16


def _check_refcounts(bm):
    count = [0] * bm.num_blocks
    for blocks in bm.blocks.values():
        for b in blocks:
            count[b] += 1
    assert count == bm.ref
    free = set(bm.free)
    assert len(free) == len(bm.free)
    for b in range(bm.num_blocks):
        assert (b in free) == (count[b] == 0)


@pytest.mark.parametrize("seed", range(25))
def test_random_ops_keep_every_view(seed):
    rng = np.random.default_rng(seed)
    nb = 40
    bm = BlockManager(nb, BS, rng.permutation(nb))
    cache = np.full(nb * BS, -1, dtype=np.int64)  # one value per slot
    truth = {}
    next_val = [0]

    def fresh():
        next_val[0] += 1
        return next_val[0]

    next_seq = 0
    for _ in range(300):
        op = rng.integers(0, 10)
        live = sorted(truth)
        try:
            if op == 0 or not live:
                n = int(rng.integers(0, 40))
                slots = bm.add(next_seq, n)
                vals = [fresh() for _ in range(n)]
                for sl, v in zip(slots, vals):
                    cache[sl] = v
                truth[next_seq] = vals
                next_seq += 1
            elif op == 1:
                p = int(rng.choice(live))
                bm.fork(p, next_seq)
                truth[next_seq] = list(truth[p])
                next_seq += 1
            elif op == 2 and len(live) > 1:
                s = int(rng.choice(live))
                bm.free_seq(s)
                del truth[s]
            else:
                seqs = [int(x) for x in rng.choice(live, size=min(len(live), 3), replace=False)]
                slots, pairs = bm.step(seqs)
                for src, dst in pairs:
                    cache[dst * BS:(dst + 1) * BS] = cache[src * BS:(src + 1) * BS]
                for s, sl in zip(seqs, slots):
                    v = fresh()
                    cache[sl] = v
                    truth[s].append(v)
        except OutOfBlocks:
            pass
        _check_refcounts(bm)
        for s, vals in truth.items():
            table = bm.block_table([s], max(1, len(bm.blocks[s])))[0]
            seen = [int(cache[table[t // BS] * BS + t % BS]) for t in range(len(vals))]
            assert seen == vals
            assert 0 <= bm.waste(s) <= BS - 1 or len(vals) == 0


def test_out_of_blocks_leaves_state_unchanged():
    bm = BlockManager(3, BS, [2, 0, 1])
    bm.add(0, 40)  # 3 blocks
    before = (list(bm.free), list(bm.ref), {k: list(v) for k, v in bm.blocks.items()})
    with pytest.raises(OutOfBlocks):
        bm.add(1, 1)
    bm.fork(0, 2)
    with pytest.raises(OutOfBlocks):
        bm.append_slot(2)  # shared partial block needs a copy, pool is empty
    assert bm.length[2] == 40
    bm.free_seq(2)
    assert (list(bm.free), list(bm.ref)) == before[:2]


def test_append_slot_cases():
    bm = BlockManager(8, BS, [5, 3, 7, 1, 0, 2, 4, 6])
    assert bm.add(0, 16) == list(range(5 * BS, 6 * BS))
    slot, cow = bm.append_slot(0)  # block boundary: fresh block 3
    assert (slot, cow) == (3 * BS, None)
    bm.fork(0, 1)
    bm.fork(0, 2)
    slot, cow = bm.append_slot(1)  # shared partial block: copy 3 -> 7
    assert (slot, cow) == (7 * BS + 1, (3, 7))
    slot, cow = bm.append_slot(2)  # still shared by 0 and 2: copy 3 -> 1
    assert (slot, cow) == (1 * BS + 1, (3, 1))
    slot, cow = bm.append_slot(0)  # last holder writes in place
    assert (slot, cow) == (3 * BS + 1, None)
    assert bm.ref[5] == 3 and bm.ref[3] == 1
    bm.free_seq(1)
    assert list(bm.free)[-1] == 7 and bm.ref[5] == 2


def test_scatter_and_copy_refs():
    kc, vc = new_cache(4, BS, 2, 3, np.float16)
    k = np.arange(2 * 2 * 3, dtype=np.float16).reshape(2, 2, 3)
    v = -k
    scatter_ref(kc, vc, k, v, np.array([2 * BS + 5, -1], dtype=np.int32))
    assert np.array_equal(kc[2, 5], k[0]) and np.array_equal(vc[2, 5], v[0])
    assert np.count_nonzero(kc) == np.count_nonzero(k[0])  # padding slot skipped
    copy_ref(kc, vc, np.array([[2, 0]], dtype=np.int32))
    assert np.array_equal(kc[0], kc[2]) and np.array_equal(vc[0], vc[2])


def _bm_for(wl):
    bm = BlockManager(wl.pool_blocks, BS, wl.free_order)
    pairs = None
    for op in wl.ops:
        if op[0] == "add":
            bm.add(op[1], op[2])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        else:
            _, pairs = bm.step(op[1])
    return bm, pairs


def test_waste_matches_pages(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))
    lo, hi = facts["memory_waste"]["reserved_waste_range_pct"]
    below = facts["memory_waste"]["paged_waste_below_pct"]
    assert facts["last_block_only"]["max_wasted_slots_per_sequence"] == BS - 1
    for name, cap in (("llama7b", 2048), ("llama13b", 2048)):
        wl = synth.make_workload(name, with_q=False)
        bm, _ = _bm_for(wl)
        S = wl.num_seqs
        for s in range(S):
            assert 0 <= bm.waste(s) <= BS - 1
        logical_slots = sum(BS * len(bm.blocks[s]) for s in range(S))
        paged = 100.0 * sum(bm.waste(s) for s in range(S)) / logical_slots
        reserved = 100.0 * (1 - wl.total_context / (S * cap))
        assert paged < below
        assert lo <= reserved <= hi


def test_block_elements_fact(golden_dir):
    facts = json.load(open(os.path.join(golden_dir, "page_facts.json")))["block_elements"]
    assert facts["block_size"] * facts["head_size"] == facts["elements_per_block_per_head"]
    assert (facts["block_size"], facts["head_size"]) == (synth.BLOCK_SIZE, synth.HEAD_SIZE)


def test_llama13b_copy_on_write_shape():
    wl = synth.make_workload("llama13b", with_q=False)
    bm, pairs = _bm_for(wl)
    assert len(wl.groups) == 13
    assert pairs.shape == (22, 2)
    assert sum(1 for (_f, _n, p) in wl.groups if p % BS == 0) == 2
    shared = 0
    for (first, _n, plen) in wl.groups:
        for b in bm.blocks[first][: plen // BS]:
            assert bm.ref[b] == 3
            shared += 1
    assert shared == 536
    assert bm.num_used() == 5043
    assert sum(len(bm.blocks[s]) for s in range(wl.num_seqs)) == 6115
    assert wl.pool_blocks == math.ceil(1.1 * bm.num_used())
    _check_refcounts(bm)


@pytest.mark.parametrize("name", ["llama7b", "gqa", "long"])
def test_pool_is_1p1x_needed(name):
    wl = synth.make_workload(name, with_q=False)
    bm, pairs = _bm_for(wl)
    assert pairs.shape == (0, 2)
    assert wl.pool_blocks == math.ceil(1.1 * bm.num_used())
