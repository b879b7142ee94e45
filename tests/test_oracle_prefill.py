"""Pins of the oracle's chunked-prefill attention (oracle/prefill.py).

Reading (page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎",
§2.2, chunked prefill): the chunk's query at absolute position p attends to
cache tokens 0..p.  Pins: a one-token chunk is decode attention; a whole prompt
as one chunk is textbook causal attention in explicit loops; position 0
returns its own V row; a chunk split in two gives the same rows; a planted
off-by-one in the causal bound fails the pins.
"""

import numpy as np
import pytest

import oracle
import synth
from oracle import prefill


def _wl(seed, *, ctx=(1, 70), chunk=(1, 70), hkv=2, g=2, dtype="fp16"):
    return synth.make_prefill_workload(seed, num_seqs=4, num_heads=hkv * g, num_kv_heads=hkv, dtype=dtype,
                                       context=ctx, chunk=chunk)


def test_one_token_chunks_are_decode_attention():
    wl = _wl(1, chunk=(1, 1))
    kc, vc, tables, out = prefill.run_prefill(wl)
    dec = oracle.paged_decode_ref(wl.q, kc, vc, tables, wl.context_lens, wl.scale, wl.num_kv_heads, wl.dtype)
    assert np.array_equal(out, dec)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_whole_prompt_is_textbook_causal_attention(dtype):
    wl = synth.make_prefill_workload(2, num_seqs=2, num_heads=4, num_kv_heads=2, dtype=dtype,
                                     context=(5, 24), chunk=(24, 24))
    assert np.array_equal(wl.chunk_lens, wl.context_lens)
    _, _, _, out = prefill.run_prefill(wl)
    qs = wl.query_start
    for s in range(wl.num_seqs):
        k, v = wl.seq_kv(s)
        kf, vf = oracle.to_f64(k, dtype), oracle.to_f64(v, dtype)
        for p in range(int(wl.context_lens[s])):
            q = oracle.to_f64(wl.q[qs[s] + p], dtype)
            ref = oracle.brute_force_ref(q.tolist(), kf[:p + 1].tolist(), vf[:p + 1].tolist(), wl.scale)
            np.testing.assert_allclose(out[qs[s] + p], np.array(ref), rtol=0, atol=1e-12)


def test_first_position_returns_its_value_row():
    wl = synth.make_prefill_workload(3, num_seqs=3, num_heads=2, num_kv_heads=2, dtype="fp16",
                                     context=(3, 40), chunk=(40, 40))
    _, _, _, out = prefill.run_prefill(wl)
    for s in range(wl.num_seqs):
        _, v = wl.seq_kv(s)
        assert np.array_equal(out[wl.query_start[s]], oracle.to_f64(v[0], "fp16"))


def test_splitting_a_chunk_changes_nothing():
    """The first part of a chunk, run as its own chunk (a call whose context
    ends where that part ends), gives the same rows."""
    wl = _wl(4, ctx=(40, 90), chunk=(20, 30))
    kc, vc, tables, out = prefill.run_prefill(wl)
    half = wl.chunk_lens // 2
    lens2 = wl.context_lens - wl.chunk_lens + half
    qs2 = np.concatenate([[0], np.cumsum(half)])
    q2 = np.concatenate([wl.q[wl.query_start[s]:wl.query_start[s] + half[s]] for s in range(wl.num_seqs)])
    out2 = prefill.prefill_ref(q2, kc, vc, tables, lens2, qs2, wl.scale, wl.num_kv_heads, wl.dtype)
    for s in range(wl.num_seqs):
        assert np.array_equal(out2[qs2[s]:qs2[s + 1]], out[wl.query_start[s]:wl.query_start[s] + half[s]])


def test_planted_off_by_one_fails():
    """A causal bound one token too wide (keys 0..p+1) changes every row but
    the last, so the pins above would catch it."""
    wl = synth.make_prefill_workload(5, num_seqs=1, num_heads=2, num_kv_heads=2, dtype="fp16",
                                     context=(20, 20), chunk=(20, 20))
    kc, vc, tables, good = prefill.run_prefill(wl)
    L = int(wl.context_lens[0])
    k = oracle.to_f64(oracle.attention.gather_seq(kc, tables[0], L), "fp16")
    v = oracle.to_f64(oracle.attention.gather_seq(vc, tables[0], L), "fp16")
    bad = np.stack([oracle.attention_ref(oracle.to_f64(wl.q[p], "fp16"), k[:min(p + 2, L)], v[:min(p + 2, L)],
                                         wl.scale) for p in range(L)])
    for p in range(L - 1):
        assert not np.allclose(bad[p], good[p])
    assert np.array_equal(bad[-1], good[-1])


@pytest.mark.parametrize("seed,g,dtype", [(11, 1, "fp16"), (12, 4, "bf16"), (13, 3, "fp16")])
def test_causal_chunk_ref_equals_prefill_ref(seed, g, dtype):
    """The by-products form of the chunk attention gives the per-query rows of
    prefill_ref, for chunks that start mid-context and whole prompts, with
    query blocks smaller than the chunk."""
    wl = synth.make_prefill_workload(seed, num_seqs=4, num_heads=2 * g, num_kv_heads=2, dtype=dtype,
                                     context=(1, 150), chunk=(1, 120))
    _, _, _, out = prefill.run_prefill(wl)
    qs = wl.query_start
    for s in range(wl.num_seqs):
        k, v = wl.seq_kv(s)
        L, C = int(wl.context_lens[s]), int(wl.chunk_lens[s])
        q = oracle.to_f64(wl.q[qs[s]:qs[s] + C], dtype)
        got = prefill.causal_chunk_ref(q, oracle.to_f64(k, dtype), oracle.to_f64(v, dtype), wl.scale, L - C,
                                       row_block=16)
        np.testing.assert_allclose(got, out[qs[s]:qs[s] + C], rtol=0, atol=1e-12)


def test_causal_chunk_ref_brute_force_and_planted_bound():
    """Against textbook attention in explicit loops on a whole prompt; a mask
    one key too wide (keys 0..p+1) fails."""
    wl = synth.make_prefill_workload(14, num_seqs=1, num_heads=4, num_kv_heads=2, dtype="bf16",
                                     context=(21, 21), chunk=(21, 21))
    k, v = wl.seq_kv(0)
    kf, vf = oracle.to_f64(k, "bf16"), oracle.to_f64(v, "bf16")
    q = oracle.to_f64(wl.q, "bf16")
    got = prefill.causal_chunk_ref(q, kf, vf, wl.scale, 0, row_block=8)
    for p in range(21):
        ref = oracle.brute_force_ref(q[p].tolist(), kf[:p + 1].tolist(), vf[:p + 1].tolist(), wl.scale)
        np.testing.assert_allclose(got[p], np.array(ref), rtol=0, atol=1e-12)
    # planted: every query sees one key more (the last row has none to add)
    wide = np.stack([prefill.causal_chunk_ref(q[p:p + 1], kf, vf, wl.scale, min(p + 1, 20))[0] for p in range(21)])
    for p in range(20):
        assert not np.allclose(wide[p], got[p])
