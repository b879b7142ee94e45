"""Pins of the oracle's prefix caching (oracle/block_manager.py: add_cached,
append_token, evictable blocks).

Page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎",
§2.2 states the purpose: the cache of an identical prefix is computed once and
reused.  What that fixes, whatever the policy:

* semantic check (the property prefix caching must keep): the K/V of a token
  depends on the token and every token before it, so a flat stand-in cache
  stores at each written slot the whole token prefix it belongs to; after
  random add_cached / append_token / append_slot / fork / free sequences, every
  live sequence read through its block table sees exactly its own prefixes,
  although only the tokens add_cached reports as uncached were written;
* structure: a shared prompt's full blocks are shared (same block ids,
  refcount = sharers); equal block content after a different prefix is not a
  hit; a prompt shorter than one block caches nothing; used + free + evictable
  covers the pool;
* worked cases of the stated policy: revival of evictable blocks, least
  recently freed evicted first, registration by append_token, no registration
  after a token without an id.
"""

import numpy as np
import pytest

from oracle import BlockManager, OutOfBlocks

BS = 16


def _check_pool(bm):
    count = [0] * bm.num_blocks
    for blocks in bm.blocks.values():
        for b in blocks:
            count[b] += 1
    assert count == bm.ref
    free, ev = list(bm.free), list(bm.evictable)
    assert len(set(free)) == len(free) and not set(free) & set(ev)
    for b in range(bm.num_blocks):
        assert (b in free or b in ev) == (count[b] == 0)
    assert all(b in bm.key for b in ev)  # evictable blocks keep their key
    assert bm.num_used() + bm.num_free() == bm.num_blocks


def _prompt(rng, base, n):
    """A prompt that starts with a prefix of one of a few shared 'system prompts'."""
    k = int(rng.integers(0, min(n, len(base)) + 1))
    return list(base[:k]) + [int(x) for x in rng.integers(0, 5, n - k)]


@pytest.mark.parametrize("seed", range(30))
def test_every_sequence_reads_its_own_prefixes(seed):
    rng = np.random.default_rng(seed)
    nb = int(rng.integers(6, 40))
    bm = BlockManager(nb, BS, rng.permutation(nb))
    cache = {}  # slot -> token prefix written there
    toks = {}   # seq -> token ids
    bases = [[int(x) for x in rng.integers(0, 3, 80)] for _ in range(3)]
    live, nxt, hits = [], 0, 0
    for _ in range(300):
        op = int(rng.integers(0, 8))
        if op <= 1 or not live:
            ids = _prompt(rng, bases[int(rng.integers(0, 3))], int(rng.integers(0, 70)))
            try:
                slots, cached = bm.add_cached(nxt, ids)
            except OutOfBlocks:
                continue
            assert cached % BS == 0 and 0 <= cached <= len(ids)
            hits += cached
            for t in range(cached, len(ids)):  # only the uncached tokens are written
                cache[slots[t]] = tuple(ids[:t + 1])
            toks[nxt] = ids
            live.append(nxt)
            nxt += 1
        elif op == 2:
            p = int(rng.choice(live))
            bm.fork(p, nxt)
            toks[nxt] = list(toks[p])
            live.append(nxt)
            nxt += 1
        elif op == 3 and len(live) > 1:
            s = int(rng.choice(live))
            bm.free_seq(s)
            live.remove(s)
            del toks[s]
        else:
            s = int(rng.choice(live))
            t = int(rng.integers(0, 3))
            try:
                slot, cow = bm.append_slot(s) if op == 7 else bm.append_token(s, t)
            except OutOfBlocks:
                continue
            if cow is not None:
                for o in range(BS):
                    if cow[0] * BS + o in cache:
                        cache[cow[1] * BS + o] = cache[cow[0] * BS + o]
            toks[s].append(t)
            cache[slot] = tuple(toks[s])
        _check_pool(bm)
        for s in live:
            for t in range(len(toks[s])):
                slot = bm.blocks[s][t // BS] * BS + t % BS
                assert cache.get(slot) == tuple(toks[s][:t + 1]), (s, t)
    assert seed > 3 or hits > 0  # the streams do exercise hits


def test_shared_prompt_blocks_are_shared():
    bm = BlockManager(20, BS)
    sys_prompt = list(range(100, 140))  # 40 tokens: two full blocks + 8
    a, ca = bm.add_cached(0, sys_prompt + [1, 2, 3])
    b, cb = bm.add_cached(1, sys_prompt + [7] * 30)
    assert ca == 0 and cb == 32
    assert bm.blocks[0][:2] == bm.blocks[1][:2]
    assert bm.ref[bm.blocks[0][0]] == 2 and bm.ref[bm.blocks[0][1]] == 2
    assert bm.blocks[0][2] != bm.blocks[1][2]  # the partly shared third block is not
    assert b[:32] == a[:32]
    assert bm.num_used() == 3 + 2 + 1


def test_same_block_after_another_prefix_is_not_a_hit():
    bm = BlockManager(10, BS)
    x, y, z = [1] * 16, [2] * 16, [3] * 16
    bm.add_cached(0, x + y)
    _, c = bm.add_cached(1, z + y)
    assert c == 0 and not set(bm.blocks[0]) & set(bm.blocks[1])
    _, c = bm.add_cached(2, x + z)
    assert c == 16 and bm.blocks[2][0] == bm.blocks[0][0] and bm.blocks[2][1] != bm.blocks[0][1]


def test_short_prompts_cache_nothing():
    bm = BlockManager(4, BS)
    bm.add_cached(0, list(range(15)))
    _, c = bm.add_cached(1, list(range(15)))
    assert c == 0 and bm.blocks[0] != bm.blocks[1]
    b0 = bm.blocks[0][0]
    bm.free_seq(0)
    assert bm.num_evictable() == 0 and list(bm.free)[-1] == b0
    _, c = bm.add_cached(2, [])
    assert c == 0 and bm.blocks[2] == []


def test_freed_prompt_is_revived():
    bm = BlockManager(8, BS, [5, 2, 7, 0, 1, 3, 4, 6])
    ids = list(range(40))
    bm.add_cached(0, ids)
    blocks = list(bm.blocks[0])
    assert blocks == [5, 2, 7]
    bm.free_seq(0)
    # full blocks evictable, the partial third block back on the free list
    assert list(bm.evictable) == [5, 2] and list(bm.free)[-1] == 7
    assert bm.num_free() == 8 and bm.num_evictable() == 2
    _, c = bm.add_cached(1, ids)
    assert c == 32 and bm.blocks[1][:2] == [5, 2] and bm.num_evictable() == 0
    assert bm.ref[5] == 1 and bm.ref[2] == 1


def test_least_recently_freed_is_evicted_first():
    bm = BlockManager(4, BS, [0, 1, 2, 3])
    bm.add_cached(0, [1] * 32)  # blocks 0, 1
    bm.add_cached(1, [2] * 32)  # blocks 2, 3
    bm.free_seq(1)
    bm.free_seq(0)
    assert list(bm.evictable) == [2, 3, 0, 1] and not bm.free
    bm.add(2, 17)  # two blocks: the two least recently freed
    assert bm.blocks[2] == [2, 3]
    _, c = bm.add_cached(3, [2] * 32)  # its prefix was evicted
    assert c == 0 and bm.blocks[3] == [0, 1]
    with pytest.raises(OutOfBlocks):
        bm.add_cached(4, [1] * 32)  # pool full; nothing evictable
    _check_pool(bm)


def test_hits_on_evictable_blocks_do_not_count_as_available():
    bm = BlockManager(3, BS)
    bm.add_cached(0, [4] * 32)  # blocks 0, 1
    bm.free_seq(0)
    assert bm.num_free() == 3
    # reusing both cached blocks leaves one block for the rest
    _, c = bm.add_cached(1, [4] * 32 + [5] * 16)
    assert c == 32 and bm.num_free() == 0
    bm.free_seq(1)
    with pytest.raises(OutOfBlocks):
        bm.add_cached(2, [4] * 32 + [6] * 32)  # needs 2 fresh + 2 revived of 3
    _check_pool(bm)


def test_generated_blocks_are_registered():
    bm = BlockManager(8, BS)
    bm.add_cached(0, list(range(10)))
    for t in range(10, 40):
        bm.append_token(0, t)
    _, c = bm.add_cached(1, list(range(45)))
    assert c == 32 and bm.blocks[1][:2] == bm.blocks[0][:2]


def test_a_token_without_an_id_stops_registration():
    bm = BlockManager(8, BS)
    bm.add_cached(0, list(range(10)))
    bm.append_slot(0)
    for t in range(11, 40):
        bm.append_token(0, t)
    _, c = bm.add_cached(1, list(range(10)) + [0] + list(range(11, 40)))
    assert c == 0


def test_duplicate_content_follows_the_registered_chain():
    """Two sequences generate the same tokens: the second's block stays private
    (the first is registered), yet its later blocks chain on from the first's,
    so a third prompt finds the whole run."""
    bm = BlockManager(12, BS)
    bm.add_cached(0, [])
    bm.add_cached(1, [])
    for t in range(32):
        bm.append_token(0, t % 5)
    for t in range(48):
        bm.append_token(1, t % 5)
    assert bm.blocks[0][:2] != bm.blocks[1][:2]
    _, c = bm.add_cached(2, [t % 5 for t in range(50)])
    assert c == 48
    assert bm.blocks[2][:2] == bm.blocks[0][:2] and bm.blocks[2][2] == bm.blocks[1][2]
    bm.free_seq(1)  # its first two blocks were never registered: back to the free list
    assert bm.num_evictable() == 0 and bm.ref[bm.blocks[2][2]] == 1


def test_fork_then_generate_shares_and_registers():
    bm = BlockManager(10, BS)
    bm.add_cached(0, list(range(20)))
    bm.fork(0, 1)
    s0, cow0 = bm.append_token(0, 99)
    s1, cow1 = bm.append_token(1, 98)
    assert cow0 is not None and cow1 is None  # the first to append copies
    for t in range(11):
        bm.append_token(0, 200 + t)
        bm.append_token(1, 300 + t)
    _, c = bm.add_cached(2, list(range(20)) + [98] + list(range(300, 311)))
    assert c == 32 and bm.blocks[2][1] == bm.blocks[1][1]


def _serve(wl):
    """The host side of the two-phase request mix the GPU test serves, on the
    oracle block manager with the token-prefix stand-in cache."""
    bm = BlockManager(wl.pool_blocks, BS, wl.free_order)
    cache, toks = {}, {}
    st = dict(hits=0, revived=0, min_free=wl.pool_blocks, peak_used=0)

    def add(r):
        ids = wl.prompt(r)[0].tolist()
        ev = bm.num_evictable()
        slots, c = bm.add_cached(r, ids)
        st["hits"] += c
        st["revived"] += ev - bm.num_evictable() > 0
        for t in range(c, len(ids)):
            cache[slots[t]] = tuple(ids[:t + 1])
        toks[r] = ids
        st["min_free"] = min(st["min_free"], len(bm.free))
        st["peak_used"] = max(st["peak_used"], bm.num_used())

    for r in range(wl.phase1):
        add(r)
    for r in wl.freed.tolist():
        bm.free_seq(r)
        del toks[r]
    assert bm.num_evictable() > 0
    for r in list(toks):
        tid = wl.decode_token(r)[0]
        slot, cow = bm.append_token(r, tid)
        assert cow is None
        toks[r].append(tid)
        cache[slot] = tuple(toks[r])
        st["peak_used"] = max(st["peak_used"], bm.num_used())
    for r in range(wl.phase1, wl.num_requests):
        add(r)
    _check_pool(bm)
    for r, ids in toks.items():
        for t in range(len(ids)):
            assert cache[bm.blocks[r][t // BS] * BS + t % BS] == tuple(ids[:t + 1])
    return st


@pytest.mark.parametrize("seed", [901, 906, 907, 908, 918])  # the GPU test's mixes
def test_prefix_workload_reuses_revives_and_evicts(seed):
    """Run on the pool without sharing, the mix reuses and revives blocks; run
    again on a pool of just its peak of blocks in use (eviction takes only
    blocks no live request holds, so that peak does not change), it fits,
    exhausts the free list and so evicts, and every request still reads its
    own prefixes."""
    import synth
    loose = _serve(synth.make_prefix_cache_workload(seed))
    assert loose["min_free"] > 0  # nothing evicted: every drop of the evictable count is a revival
    assert loose["hits"] > 0 and loose["revived"] > 0
    tight = _serve(synth.make_prefix_cache_workload(seed, pool_blocks=loose["peak_used"]))
    assert tight["min_free"] == 0 and tight["peak_used"] == loose["peak_used"]
    assert 0 < tight["hits"] <= loose["hits"]
