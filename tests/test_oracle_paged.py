"""Pins of the oracle's paged decode: paging changes storage, not the result.

* paged decode == explicit-loop brute force on the contiguous per-sequence K/V
  (the tiny batch, and random tiny shapes including GQA and bf16);
* any permutation of physical block ids gives a bit-identical result;
* block-table entries past a sequence's last block and stale cache slots are
  never read;
* copy-on-write keeps shared prompt blocks unchanged and each sample still sees
  its own prompt + new token.
"""

import numpy as np
import pytest

import oracle
import synth
from oracle import attention_ref, brute_force_ref, paged_decode_ref, run_decode_step, to_f64

BS = 16


def _contiguous_ref(wl, s):
    k, v = wl.seq_kv(s)
    return attention_ref(to_f64(wl.q[s], wl.dtype), to_f64(k, wl.dtype), to_f64(v, wl.dtype), wl.scale)


def test_tiny_batch_matches_brute_force():
    wl = synth.make_workload("tiny")
    st = run_decode_step(wl)
    assert list(st.context_lens) == [17, 33, 100, 250]
    for s in range(wl.num_seqs):
        k, v = wl.seq_kv(s)
        bf = brute_force_ref(to_f64(wl.q[s], "fp16").tolist(), to_f64(k, "fp16").tolist(),
                             to_f64(v, "fp16").tolist(), wl.scale)
        assert np.abs(st.out[s] - np.asarray(bf)).max() <= 1e-12


@pytest.mark.parametrize("seed", range(60))
def test_random_tiny_paged_equals_contiguous(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.integers(1, 5))
    g = int(rng.choice([1, 2, 4]))
    dtype = "bf16" if seed % 2 else "fp16"
    groups = 1 if seed % 3 == 0 else 0
    wl = synth.make_random_workload(1000 + seed, num_seqs=int(rng.integers(3, 5)),
                                    num_heads=hkv * g, num_kv_heads=hkv, dtype=dtype,
                                    max_len=70, groups=groups)
    st = run_decode_step(wl)
    for s in range(wl.num_seqs):
        ref = _contiguous_ref(wl, s)
        assert np.abs(st.out[s] - ref).max() <= 1e-12
    if seed < 6:  # explicit loops on a few of them
        s = 0
        k, v = wl.seq_kv(s)
        bf = brute_force_ref(to_f64(wl.q[s], dtype).tolist(), to_f64(k, dtype).tolist(),
                             to_f64(v, dtype).tolist(), wl.scale)
        assert np.abs(st.out[s] - np.asarray(bf)).max() <= 1e-12


def test_block_permutation_invariance():
    wl = synth.make_workload("tiny")
    st = run_decode_step(wl)
    rng = np.random.default_rng(11)
    perm = rng.permutation(wl.pool_blocks)
    kc2 = np.empty_like(st.k_cache); vc2 = np.empty_like(st.v_cache)
    kc2[perm] = st.k_cache; vc2[perm] = st.v_cache
    tables = np.where(st.block_tables >= 0, perm[np.maximum(st.block_tables, 0)], -1)
    out2 = paged_decode_ref(wl.q, kc2, vc2, tables, st.context_lens, wl.scale, wl.num_kv_heads, wl.dtype)
    assert np.array_equal(out2, st.out)


def test_stale_slots_and_table_tail_are_never_read():
    wl = synth.make_workload("tiny")
    st = run_decode_step(wl)
    kc = st.k_cache.copy(); vc = st.v_cache.copy()
    live = np.zeros(kc.shape[:2], dtype=bool)
    for s in range(wl.num_seqs):
        for t in range(int(st.context_lens[s])):
            live[st.block_tables[s, t // BS], t % BS] = True
    kc[~live] = np.float16(np.nan); vc[~live] = np.float16(np.inf)
    tables = st.block_tables.copy()
    tables[tables < 0] = 10 ** 6  # would raise IndexError if read
    tables = np.concatenate([tables, np.full((tables.shape[0], 3), 10 ** 6, np.int32)], axis=1)
    out = paged_decode_ref(wl.q, kc, vc, tables, st.context_lens, wl.scale, wl.num_kv_heads, wl.dtype)
    assert np.array_equal(out, st.out)


def test_copy_on_write_step_values():
    """Sampling groups at their first decode step: shared full prompt blocks are
    untouched and keep ref = 3; each sample equals attention over its own
    contiguous prompt + new token."""
    for seed in range(6):
        wl = synth.make_random_workload(500 + seed, num_seqs=7, num_heads=4, num_kv_heads=2,
                                        dtype="fp16", max_len=60, min_len=20, groups=2)
        st = run_decode_step(wl, keep_before=True)
        bm = st.block_manager
        n_pairs_expected = sum(2 for (_f, _n, p) in wl.groups if p % BS)
        assert st.block_pairs.shape == (n_pairs_expected, 2)
        for (first, n, plen) in wl.groups:
            shared = bm.blocks[first][: plen // BS]  # full prompt blocks
            for b in shared:
                assert bm.ref[b] == 3
                assert np.array_equal(st.k_cache[b], st.k_cache_before_step[b])
                assert np.array_equal(st.v_cache[b], st.v_cache_before_step[b])
            for s in range(first, first + n):
                assert bm.blocks[s][: plen // BS] == shared
        written = set(int(x) // BS for x in st.slot_mapping)
        for b in range(wl.pool_blocks):
            if b not in written and b not in set(st.block_pairs[:, 1].tolist()):
                assert np.array_equal(st.k_cache[b], st.k_cache_before_step[b])
        for s in range(wl.num_seqs):
            assert np.abs(st.out[s] - _contiguous_ref(wl, s)).max() <= 1e-12


def test_swap_ref_round_trip_and_copy_special_case():
    """Swapping blocks out to a second cache and back with the inverse pairs
    restores them; swapping within one cache is the block copy."""
    rng = np.random.default_rng(77)
    a_k = rng.integers(0, 1 << 16, (6, 16, 2, 8)).astype(np.uint16)
    a_v = rng.integers(0, 1 << 16, (6, 16, 2, 8)).astype(np.uint16)
    b_k, b_v = np.zeros((4, 16, 2, 8), np.uint16), np.zeros((4, 16, 2, 8), np.uint16)
    out_pairs = np.array([[5, 0], [1, 3], [2, 1]])
    oracle.swap_ref(b_k, b_v, a_k, a_v, out_pairs)
    back_k, back_v = np.zeros_like(a_k), np.zeros_like(a_v)
    oracle.swap_ref(back_k, back_v, b_k, b_v, out_pairs[:, ::-1])
    for src, _dst in out_pairs:
        assert np.array_equal(back_k[src], a_k[src]) and np.array_equal(back_v[src], a_v[src])
    assert not back_k[0].any() and not back_k[3].any()  # untouched
    c_k, c_v = a_k.copy(), a_v.copy()
    d_k, d_v = a_k.copy(), a_v.copy()
    pairs = np.array([[0, 4], [2, 3]])
    oracle.swap_ref(c_k, c_v, c_k, c_v, pairs)
    oracle.copy_ref(d_k, d_v, pairs)
    assert np.array_equal(c_k, d_k) and np.array_equal(c_v, d_v)
    oracle.swap_ref(b_k, b_v, a_k, a_v, np.array([[9, 0], [0, 7]]))  # out-of-range pairs skipped
