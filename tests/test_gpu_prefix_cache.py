"""Prefix caching end to end on the GPU: requests that share system prompts
are served in two phases through the library's block manager (add_cached /
append_token), reshape_and_cache of only the rows not cached yet, and one
paged_attn_prefill call per phase (page "vLLM 深度解析：以 PagedAttention 与
内核生态构建高吞吐 LLM 推理引擎", §2.2: an identical prefix is computed once and
reused).  Marked gpu.

Checks: every query row against the float64 oracle on the request's contiguous
rows (tolerances as for decode: 2e-3 fp16, 1e-2 bf16); the outputs bit for bit
against the same queries served without prefix caching (every row written,
no sharing); and that the run did reuse, revive and evict blocks.
"""

import numpy as np
import pytest

import harness
import oracle
import synth
from oracle import fp8 as ofp8

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"fp16": 2e-3, "bf16": 1e-2}


def _rows_f64(wl, k, v):
    if wl.kv_dtype == "fp8e4m3":
        return (ofp8.dequantize_ref(ofp8.quantize_ref(k, wl.dtype, wl.k_scale), wl.k_scale),
                ofp8.dequantize_ref(ofp8.quantize_ref(v, wl.dtype, wl.v_scale), wl.v_scale))
    return oracle.to_f64(k, wl.dtype), oracle.to_f64(v, wl.dtype)


def _seq_rows(wl, r, n):
    """Contiguous K, V of request r's first n tokens (prompt, then its decode token)."""
    _, k, v = wl.prompt(r)
    if n > k.shape[0]:
        _, kt, vt = wl.decode_token(r)
        k, v = np.concatenate([k, kt[None]]), np.concatenate([v, vt[None]])
    return _rows_f64(wl, k[:n], v[:n])


def _peak_in_use(wl):
    """Most blocks live requests hold at once when served with prefix caching
    (oracle block manager, host only).  Eviction takes only blocks no live
    request holds, so a pool of exactly this size still fits the mix and
    forces evictions."""
    bm = oracle.BlockManager(wl.pool_blocks, 16, wl.free_order)
    peak = 0
    for r in range(wl.phase1):
        bm.add_cached(r, wl.prompt(r)[0].tolist())
        peak = max(peak, bm.num_used())
    for r in wl.freed.tolist():
        bm.free_seq(r)
    for r in range(wl.phase1):
        if r not in set(wl.freed.tolist()):
            bm.append_token(r, wl.decode_token(r)[0])
            peak = max(peak, bm.num_used())
    for r in range(wl.phase1, wl.num_requests):
        bm.add_cached(r, wl.prompt(r)[0].tolist())
        peak = max(peak, bm.num_used())
    return peak


CASES = [("fp16", 1, None, 901), ("bf16", 4, None, 906), ("fp16", 4, "fp8e4m3", 907), ("bf16", 16, None, 918)]


@pytest.mark.parametrize("dtype,g,kv,seed", CASES)
def test_prefix_cache_end_to_end(dtype, g, kv, seed):
    hkv = 2
    kw = dict(num_heads=hkv * g, num_kv_heads=hkv, dtype=dtype, kv_dtype=kv, k_scale=0.0125, v_scale=0.02)
    wl = synth.make_prefix_cache_workload(seed, pool_blocks=_peak_in_use(synth.make_prefix_cache_workload(seed, **kw)),
                                          **kw)
    run = harness.run_prefix_cache(wl)
    assert sum(run.cached.values()) > 0
    assert run.min_free_list == 0 and min(run.evictable_seen) < max(run.evictable_seen)
    for ph in run.phases:
        got = oracle.to_f64(harness.to_host_bits(ph.out).view(np.float16) if dtype == "fp16"
                            else harness.to_host_bits(ph.out), dtype)
        assert np.isfinite(got).all()
        for i, r in enumerate(ph.seqs):
            L = int(ph.context_lens[i])
            k, v = _seq_rows(wl, r, L)
            qr = wl.q_rows(r)
            for j, p in enumerate(range(int(ph.first_pos[i]), L)):
                ref = oracle.attention_ref(oracle.to_f64(qr[p], dtype), k[:p + 1], v[:p + 1], wl.scale)
                err = np.abs(got[ph.query_start[i] + j] - ref).max()
                assert err <= TOL[dtype], (r, p, err)
    fps = [{r: int(f) for r, f in zip(ph.seqs, ph.first_pos)} for ph in run.phases]
    # without sharing the tight pool is too small: same mix on the loose pool
    plain = harness.run_prefix_cache(synth.make_prefix_cache_workload(seed, **kw), cached=False, first_pos=fps)
    assert plain.written > run.written
    for a, b in zip(run.phases, plain.phases):
        assert a.seqs == b.seqs and np.array_equal(a.query_start, b.query_start)
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
