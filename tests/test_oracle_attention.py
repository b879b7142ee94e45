"""Pins of the oracle's attention functions against closed forms, special
cases and explicit-loop brute force (CPU only)."""

import math

import numpy as np
import pytest

import oracle
from oracle import attention_ref, brute_force_ref, lse_merge_ref, partition_partials_ref

D = 128
SCALE = 1 / math.sqrt(D)


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def test_two_tokens_closed_form():
    """Two tokens: weight of token 0 is the logistic function of the logit
    difference.  q = a e_0, k_t = b_t e_0, so the logits are scale*a*b_t."""
    a, b0, b1 = 1.5, 2.0, -0.5
    q = np.zeros((1, D)); q[0, 0] = a
    k = np.zeros((2, 1, D)); k[0, 0, 0] = b0; k[1, 0, 0] = b1
    rng = np.random.default_rng(0)
    v = _rand(rng, 2, 1, D)
    w0 = 1.0 / (1.0 + math.exp(SCALE * a * (b1 - b0)))
    expect = w0 * v[0, 0] + (1 - w0) * v[1, 0]
    np.testing.assert_allclose(attention_ref(q, k, v, SCALE)[0], expect, rtol=0, atol=1e-14)
    bf = brute_force_ref(q.tolist(), k.tolist(), v.tolist(), SCALE)
    np.testing.assert_allclose(np.asarray(bf)[0], expect, rtol=0, atol=1e-14)


def test_scale_enters_logits():
    """Same two tokens with scale doubled: the logit difference doubles."""
    q = np.zeros((1, D)); q[0, 3] = 1.0
    k = np.zeros((2, 1, D)); k[0, 0, 3] = 1.0
    v = np.zeros((2, 1, D)); v[0, 0, 0] = 1.0
    for scale in (0.5, 1.0, 2.0):
        w0 = 1.0 / (1.0 + math.exp(-scale))
        assert abs(attention_ref(q, k, v, scale)[0, 0] - w0) < 1e-15


def test_single_token_is_exact_copy():
    rng = np.random.default_rng(1)
    q = _rand(rng, 4, D); k = _rand(rng, 1, 2, D); v = _rand(rng, 1, 2, D)
    out = attention_ref(q, k, v, SCALE)
    for h in range(4):
        assert np.array_equal(out[h], v[0, h // 2])


def test_zero_query_gives_mean_of_values():
    rng = np.random.default_rng(2)
    L = 37
    q = np.zeros((2, D)); k = _rand(rng, L, 2, D); v = _rand(rng, L, 2, D)
    out = attention_ref(q, k, v, SCALE)
    for h in range(2):
        np.testing.assert_allclose(out[h], v[:, h].mean(axis=0), rtol=0, atol=1e-14)


def test_constant_keys_give_mean_of_values():
    rng = np.random.default_rng(3)
    L = 20
    q = _rand(rng, 1, D)
    k = np.repeat(_rand(rng, 1, 1, D), L, axis=0)
    v = _rand(rng, L, 1, D)
    np.testing.assert_allclose(attention_ref(q, k, v, SCALE)[0], v[:, 0].mean(axis=0), atol=1e-14)


def test_unit_values_and_weight_sum():
    """Softmax weights sum to one: with V == 1 the output is exactly 1 up to
    rounding, and the returned weights sum to 1."""
    rng = np.random.default_rng(4)
    L = 300
    q = _rand(rng, 3, D) * 3; k = _rand(rng, L, 3, D); v = np.ones((L, 3, D))
    out, w = attention_ref(q, k, v, SCALE, return_weights=True)
    assert np.abs(out - 1).max() < 1e-13
    assert np.abs(w.sum(axis=1) - 1).max() < 1e-13
    assert (w > 0).all()


def test_large_logits_are_stable():
    """Logits near 1000 would overflow exp without the max shift."""
    q = np.zeros((1, D)); q[0, 0] = 1000.0
    k = np.zeros((2, 1, D)); k[0, 0, 0] = 1.0; k[1, 0, 0] = 1.0
    v = np.zeros((2, 1, D)); v[0, 0, 0] = 2.0; v[1, 0, 0] = 4.0
    out = attention_ref(q, k, v, 1.0)
    assert out[0, 0] == 3.0


def test_gqa_mapping_equals_repeated_heads():
    """Query head h reads KV head h // g: identical to MHA on K/V whose heads
    were repeated g times (numpy.repeat lays out contiguous groups)."""
    rng = np.random.default_rng(5)
    L, hkv, g = 45, 3, 4
    q = _rand(rng, hkv * g, D); k = _rand(rng, L, hkv, D); v = _rand(rng, L, hkv, D)
    gqa = attention_ref(q, k, v, SCALE)
    mha = attention_ref(q, np.repeat(k, g, axis=1), np.repeat(v, g, axis=1), SCALE)
    assert np.array_equal(gqa, mha)


@pytest.mark.parametrize("seed", range(40))
def test_attention_ref_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(1, 71))
    hkv = int(rng.integers(1, 4))
    g = int(rng.choice([1, 2, 4]))
    q = _rand(rng, hkv * g, D); k = _rand(rng, L, hkv, D); v = _rand(rng, L, hkv, D)
    ref = attention_ref(q, k, v, SCALE)
    bf = np.asarray(brute_force_ref(q.tolist(), k.tolist(), v.tolist(), SCALE))
    assert np.abs(ref - bf).max() <= 1e-12


@pytest.mark.parametrize("P", [1, 16, 32, 100, 512, 4096])
def test_partition_merge_equals_full_softmax(P):
    rng = np.random.default_rng(7)
    L = 1000
    q = _rand(rng, 4, D) * 2; k = _rand(rng, L, 2, D); v = _rand(rng, L, 2, D)
    m, z, o = partition_partials_ref(q, k, v, SCALE, P)
    assert m.shape == (4, -(-L // P))
    merged = lse_merge_ref(m, z, o)
    assert np.abs(merged - attention_ref(q, k, v, SCALE)).max() <= 1e-12


def test_single_partition_is_identity():
    rng = np.random.default_rng(8)
    q = _rand(rng, 2, D); k = _rand(rng, 50, 1, D); v = _rand(rng, 50, 1, D)
    m, z, o = partition_partials_ref(q, k, v, SCALE, 64)
    np.testing.assert_allclose(lse_merge_ref(m, z, o), o[:, 0], atol=1e-15)


def test_merge_weights_by_partition_mass():
    """Two partitions with equal max: the merge weights their outputs by Z."""
    m = np.array([[0.0, 0.0]]); z = np.array([[1.0, 3.0]])
    o = np.array([[[1.0] * D, [5.0] * D]])
    np.testing.assert_allclose(lse_merge_ref(m, z, o)[0], [4.0] * D, atol=1e-15)
    # a partition whose max is ln(3) lower carries a third of its Z
    m = np.array([[math.log(3.0), 0.0]]); z = np.array([[1.0, 3.0]])
    np.testing.assert_allclose(lse_merge_ref(m, z, o)[0], [3.0] * D, atol=1e-14)


def test_empty_context_rejected():
    with pytest.raises(ValueError):
        attention_ref(np.zeros((1, D)), np.zeros((0, 1, D)), np.zeros((0, 1, D)), SCALE)


def test_oracle_catches_planted_mistakes():
    """Plausible slips in the formula change the result detectably."""
    rng = np.random.default_rng(9)
    L = 40
    q = _rand(rng, 2, D); k = _rand(rng, L, 2, D); v = _rand(rng, L, 2, D)
    bf = np.asarray(brute_force_ref(q.tolist(), k.tolist(), v.tolist(), SCALE))
    good = attention_ref(q, k, v, SCALE)
    assert np.abs(good - bf).max() < 1e-12
    # dropped scale, flipped sign, transposed head mapping, missing normalisation
    assert np.abs(attention_ref(q, k, v, 1.0) - bf).max() > 1e-3
    assert np.abs(attention_ref(-q, k, v, SCALE) - bf).max() > 1e-3
    assert np.abs(attention_ref(q, k[:, ::-1], v[:, ::-1], SCALE) - bf).max() > 1e-3
    _, w = attention_ref(q, k, v, SCALE, return_weights=True)
    assert np.abs((w * 2).sum(axis=1) - 1).max() > 0.5
