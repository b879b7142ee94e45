"""The synthetic batches: lengths, totals and value recipe (CPU only)."""

import numpy as np
import pytest

import synth

# (sum of contexts, min, median, max, logical blocks) of each batch
EXPECTED = {
    "tiny": (400, 17, 66.5, 250, 28),
    "llama7b": (39242, 35, 460.5, 2048, 2482),
    "llama13b": (96953, 35, 485.0, 2048, 6115),
    "gqa": (1208549, 1053, 4769.5, 8167, 75657),
    "long": (675670, 34994, 89075.0, 112192, 42233),
}


@pytest.mark.parametrize("name", list(EXPECTED))
def test_lengths(name):
    wl = synth.make_workload(name, with_q=False)
    L = wl.context_lens
    total, lo, med, hi, blocks = EXPECTED[name]
    assert (int(L.sum()), int(L.min()), float(np.median(L)), int(L.max())) == (total, lo, med, hi)
    assert int(sum(-(-int(x) // 16) for x in L)) == blocks
    assert sorted(wl.free_order.tolist()) == list(range(wl.pool_blocks))


def test_long_lengths_listed():
    wl = synth.make_workload("long", with_q=False)
    assert wl.context_lens.tolist() == [98710, 111903, 34994, 112192, 78858, 83427, 94723, 60863]


def test_gqa_key_scales_and_values():
    wl = synth.make_workload("gqa")
    assert wl.key_scales.shape == (8,)
    assert ((wl.key_scales >= 0.5) & (wl.key_scales <= 2.0)).all()
    assert wl.q.dtype == np.uint16 and wl.q.shape == (256, 64, 128)
    k, v = wl.own_kv(0)
    assert k.shape == (wl.context_lens[0], 8, 128) and k.dtype == np.uint16
    kf = (k.astype(np.uint32) << 16).view(np.float32)
    vf = (v.astype(np.uint32) << 16).view(np.float32)
    ratio = kf.std(axis=(0, 2)) / vf.std(axis=(0, 2))
    np.testing.assert_allclose(ratio, wl.key_scales, rtol=0.05)


def test_streams_are_deterministic_and_independent():
    a = synth.make_workload("tiny")
    b = synth.make_workload("tiny")
    assert np.array_equal(a.q, b.q)
    k0, _ = a.own_kv(2)
    k1, _ = b.own_kv(2)
    assert np.array_equal(k0, k1)
    assert not np.array_equal(a.own_kv(1)[0][:17], a.own_kv(0)[0][:17])


def test_group_members_share_prompt():
    wl = synth.make_workload("llama13b", with_q=False)
    first, n, plen = wl.groups[0]
    ks = [wl.seq_kv(s)[0] for s in range(first, first + n)]
    for k in ks:
        assert k.shape[0] == plen + 1
        assert np.array_equal(k[:plen], ks[0][:plen])
    assert not np.array_equal(ks[0][plen], ks[1][plen])


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    bits = synth.round_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert back.tolist() == [1.0, 1.0, 1.0 + 4 * 2 ** -8, -2.5, 1.0 + 2 ** -7]
