"""GPU parity of the data-movement path (slot-mapped write, copy-on-write block
copy, gather): bit-exact against the oracle.  Marked gpu."""

import numpy as np
import pytest

import fullsize
import harness
import oracle
import synth
from layout import decode_pages, encode_pages
from oracle import fp8 as ofp8

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import paged_kv_cache_345_amd as pkv  # noqa: E402


def _garbage(wl, seed):
    rng = np.random.default_rng(seed)
    shape = (wl.pool_blocks, 16, wl.num_kv_heads, 128)
    return (rng.integers(0, 1 << 16, size=shape, dtype=np.uint16),
            rng.integers(0, 1 << 16, size=shape, dtype=np.uint16))


def _as_storage(bits, dtype):
    return bits.view(np.float16) if dtype == "fp16" else bits


def _full_cache_check(wl, seed=7):
    """Start both sides from the same garbage, run the step, compare every
    byte of both caches."""
    gk, gv = _garbage(wl, seed)
    step = harness.build_step(wl, garbage="pages",
                              initial_pages=(encode_pages(gk, "k"), encode_pages(gv, "v")))
    torch.cuda.synchronize()
    ref = oracle.run_decode_step(wl, compute_out=False,
                                 initial_cache=(_as_storage(gk, wl.dtype), _as_storage(gv, wl.dtype)))
    kb = harness.to_host_bits(step.k_cache)
    vb = harness.to_host_bits(step.v_cache)
    assert np.array_equal(decode_pages(kb, "k"), ref.k_cache.view(np.uint16))
    assert np.array_equal(decode_pages(vb, "v"), ref.v_cache.view(np.uint16))
    assert np.array_equal(step.slot_mapping_host, ref.slot_mapping)
    assert np.array_equal(step.block_pairs_host, ref.block_pairs)
    assert np.array_equal(step.block_tables_host, ref.block_tables)
    return step


def test_tiny_step_cache_bit_exact():
    _full_cache_check(synth.make_workload("tiny"))


@pytest.mark.parametrize("seed", range(6))
def test_random_step_with_copy_on_write_bit_exact(seed):
    dtype = "bf16" if seed % 2 else "fp16"
    wl = synth.make_random_workload(3000 + seed, num_seqs=9, num_heads=6, num_kv_heads=3, dtype=dtype,
                                    max_len=90, min_len=1, groups=2)
    step = _full_cache_check(wl, seed)
    assert step.block_pairs_host.shape[0] == sum(2 for (_f, _n, p) in wl.groups if p % 16)


def test_gather_matches_generator_values():
    wl = synth.make_random_workload(41, num_seqs=5, num_heads=4, num_kv_heads=4, dtype="fp16", max_len=200,
                                    groups=1)
    step = harness.build_step(wl)
    lens = wl.context_lens.astype(np.int32)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
    total = int(lens.sum())
    ko = torch.empty((total, 4, 128), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(ko)
    pkv.gather_cache(ko, vo, step.k_cache, step.v_cache, step.block_tables, step.context_lens,
                     torch.from_numpy(offs).cuda())
    kh, vh = harness.to_host_bits(ko), harness.to_host_bits(vo)
    for s in range(wl.num_seqs):
        k, v = wl.seq_kv(s)
        assert np.array_equal(kh[offs[s]:offs[s] + lens[s]], k.view(np.uint16))
        assert np.array_equal(vh[offs[s]:offs[s] + lens[s]], v.view(np.uint16))


def test_copy_blocks_and_padding_slots():
    rng = np.random.default_rng(5)
    nb, hkv = 50, 5
    gk, gv = (rng.integers(0, 1 << 16, size=(nb, 16, hkv, 128), dtype=np.uint16) for _ in range(2))
    kc = torch.from_numpy(encode_pages(gk, "k").view(np.int16)).cuda().view(torch.bfloat16)
    vc = torch.from_numpy(encode_pages(gv, "v").view(np.int16)).cuda().view(torch.bfloat16)
    blocks = rng.permutation(nb)
    pairs = np.stack([blocks[:12], blocks[12:24]], axis=1).astype(np.int32)
    pkv.copy_blocks(kc, vc, torch.from_numpy(pairs).cuda())
    # slot mapping with padding entries
    k = rng.integers(0, 1 << 16, size=(7, hkv, 128), dtype=np.uint16)
    v = rng.integers(0, 1 << 16, size=(7, hkv, 128), dtype=np.uint16)
    slots = np.array([5, -1, 16 * 49 + 15, -7, 16 * 3, 16 * 3 + 1, 0], dtype=np.int32)
    pkv.reshape_and_cache(harness.to_device(k, "bf16", "cuda"), harness.to_device(v, "bf16", "cuda"), kc, vc,
                          torch.from_numpy(slots).cuda())
    ok, ov = gk.copy(), gv.copy()
    oracle.copy_ref(ok, ov, pairs)
    oracle.scatter_ref(ok, ov, k, v, slots)
    assert np.array_equal(decode_pages(harness.to_host_bits(kc), "k"), ok)
    assert np.array_equal(decode_pages(harness.to_host_bits(vc), "v"), ov)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama7b", "llama13b"])
def test_full_size_step_caches_bit_exact(name):
    """The LLaMA-shaped batches at full size, in the configuration the bench
    times: both whole caches after the decode step (every prior token, the
    copy-on-write copies, the new tokens, and garbage everywhere else), the
    slot mapping, the copy pairs and the block tables, bit for bit against the
    oracle's step from the same garbage."""
    wl = synth.make_workload(name)
    step = _full_cache_check(wl)
    if name == "llama13b":
        assert step.block_pairs_host.shape == (22, 2)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["gqa", "long", "llama13b_fp8", "gqa_fp8"])
def test_full_size_live_rows_bit_exact(name):
    """The other full-size batches: every live row of every sequence, read
    back through its block table with gather_cache, equals the generator's
    value (16-bit) or the oracle's E4M3 code of it (fp8), bit for bit."""
    wl = synth.make_workload(name)
    step = harness.build_step(wl)
    fp8 = wl.kv_dtype == "fp8e4m3"
    cdt = torch.uint8 if fp8 else harness.torch_dtype(wl.dtype)
    hkv = wl.num_kv_heads
    for lo in range(0, wl.num_seqs, 32):
        seqs = list(range(lo, min(lo + 32, wl.num_seqs)))
        lens = wl.context_lens[seqs].astype(np.int32)
        offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int32)
        ko = torch.empty((int(lens.sum()), hkv, 128), dtype=cdt, device="cuda")
        vo = torch.empty_like(ko)
        idx = torch.tensor(seqs, device="cuda")
        pkv.gather_cache(ko, vo, step.k_cache, step.v_cache, step.block_tables[idx].contiguous(),
                         step.context_lens[idx].contiguous(), torch.from_numpy(offs).cuda())
        if fp8:
            kh, vh = ko.cpu().numpy(), vo.cpu().numpy()
        else:
            kh, vh = harness.to_host_bits(ko), harness.to_host_bits(vo)

        def one(i):
            k, v = wl.seq_kv(seqs[i])
            if fp8:
                k = ofp8.quantize_ref(k, wl.dtype, wl.k_scale)
                v = ofp8.quantize_ref(v, wl.dtype, wl.v_scale)
            else:
                k, v = k.view(np.uint16), v.view(np.uint16)
            a, b = offs[i], offs[i] + lens[i]
            return bool(np.array_equal(kh[a:b], k) and np.array_equal(vh[a:b], v))

        ok = fullsize.host_map(one, range(len(seqs)))
        assert all(ok), [seqs[i] for i, o in enumerate(ok) if not o]


def test_validate_mode_catches_contract_violations(monkeypatch):
    """With PKV_VALIDATE=1 the binding checks device-array contents on host
    copies and raises before launching; valid calls run unchanged."""
    monkeypatch.setenv("PKV_VALIDATE", "1")
    wl = synth.make_workload("tiny")
    step = harness.build_step(wl, run=False)
    step.copy()
    step.write()
    out = step.decode()
    torch.cuda.synchronize()
    ref = harness.to_host_bits(out).copy()
    bad = step.block_tables.clone()
    bad[0, 0] = wl.pool_blocks  # outside the pool
    with pytest.raises(ValueError, match="block_tables"):
        step.decode(out=torch.empty_like(out), block_tables=bad)
    lens = step.context_lens.clone()
    lens[1] = 0
    with pytest.raises(ValueError, match="context_lens"):
        pkv.paged_attn_decode(torch.empty_like(out), step.q, step.k_cache, step.v_cache, step.block_tables, lens,
                              wl.scale, wl.num_kv_heads)
    dup = step.slot_mapping.clone()
    dup[1] = dup[0]
    with pytest.raises(ValueError, match="twice"):
        pkv.reshape_and_cache(step.k_new, step.v_new, step.k_cache, step.v_cache, dup)
    with pytest.raises(ValueError, match="source and a destination"):
        pkv.copy_blocks(step.k_cache, step.v_cache, torch.tensor([[0, 1], [1, 2]], dtype=torch.int32).cuda())
    out2 = step.decode(out=torch.empty_like(out))  # the caches were not touched by the refused calls
    torch.cuda.synchronize()
    assert np.array_equal(harness.to_host_bits(out2), ref)
