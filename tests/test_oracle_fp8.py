"""Pins of the oracle's FP8 (E4M3) KV-cache functions (oracle/fp8.py).

The format is the OCP 8-bit floating-point E4M3 encoding (the reading taken
for page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎",
§三, which says the KV cache can be quantised but fixes no format).  The pins:

* values the definition fixes in closed form (1, 448, 2^-6, 2^-9, -0, NaN, the
  count of finite codes, monotonic order);
* torch's own float8_e4m3fn conversion, an independent implementation of the
  same format: every decode, and every encode below the saturation bound;
* brute-force nearest-value search over all codes with ties to the even code;
* structure: doubling a normal value adds one to the exponent field;
* the fp8 attention reference equals the 16-bit one when the dequantised values
  are exactly representable in fp16, and a one-token context returns the
  dequantised V row.
"""

import numpy as np
import pytest

import oracle
from oracle import fp8

torch = pytest.importorskip("torch")


def test_closed_form_values():
    assert fp8.e4m3_value(0x38) == 1.0
    assert fp8.e4m3_value(0x7E) == 448.0 == fp8.E4M3_MAX
    assert fp8.e4m3_value(0x08) == 2.0 ** -6  # smallest normal
    assert fp8.e4m3_value(0x01) == 2.0 ** -9  # smallest subnormal
    assert fp8.e4m3_value(0x07) == 7 * 2.0 ** -9  # largest subnormal
    assert fp8.e4m3_value(0x00) == 0.0 and not np.signbit(fp8.e4m3_value(0x00))
    assert fp8.e4m3_value(0x80) == 0.0 and np.signbit(fp8.e4m3_value(0x80))
    assert fp8.e4m3_value(0xFE) == -448.0
    t = fp8.e4m3_table()
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = fp8.e4m3_table()
    both_nan = np.isnan(ref) & np.isnan(mine)
    assert np.array_equal(both_nan, np.isnan(ref) | np.isnan(mine))
    assert np.array_equal(ref[~both_nan], mine[~both_nan])
    assert np.array_equal(np.signbit(ref[~both_nan]), np.signbit(mine[~both_nan]))


def _samples(seed=0, n=20000):
    rng = np.random.default_rng(seed)
    mags = np.exp(rng.uniform(np.log(2.0 ** -12), np.log(440.0), n))
    x = (mags * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    t = fp8.e4m3_table()
    pos = t[:0x7F]
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact ties (dyadic)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)
    return np.concatenate([x, mids, -mids, pos.astype(np.float32), -pos.astype(np.float32),
                           np.float32([0.0, -0.0, 448.0, -448.0])])


def test_encode_matches_torch_below_saturation():
    x = _samples()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8.e4m3_encode(x), ref)


def test_encode_brute_force_nearest_ties_to_even():
    x = np.concatenate([_samples(1, 3000), np.float32([449.0, 463.9, 464.0, 500.0, 1e6, -470.0, -3e38])])
    t = fp8.e4m3_table()
    codes = fp8.e4m3_encode(x)
    for xi, ci in zip(x.astype(np.float64), codes):
        neg = np.signbit(xi)
        cand = np.arange(0x80, 0xFF) if neg else np.arange(0x00, 0x7F)
        if abs(xi) >= 448.0:
            want = 0xFE if neg else 0x7E
        else:
            d = np.abs(t[cand] - xi)  # exact in float64 for these magnitudes
            best = cand[d == d.min()]
            want = best[best % 2 == 0][0] if len(best) > 1 else best[0]
        assert ci == want, (xi, hex(ci), hex(want))


def test_round_trip_and_ties():
    finite = [c for c in range(256) if c not in fp8.E4M3_NAN_CODES]
    vals = np.array([fp8.e4m3_value(c) for c in finite], dtype=np.float32)
    assert np.array_equal(fp8.e4m3_encode(vals), np.array(finite, dtype=np.uint8))
    # midpoints go to the even code
    assert fp8.e4m3_encode(np.float32(1.0625)) == 0x38
    assert fp8.e4m3_encode(np.float32(1.1875)) == 0x3A
    assert fp8.e4m3_encode(np.float32(2.0 ** -10)) == 0x00
    assert fp8.e4m3_encode(np.float32(7.5 * 2.0 ** -9)) == 0x08
    assert fp8.e4m3_encode(np.float32(-(2.0 ** -11))) == 0x80
    assert fp8.e4m3_encode(np.float32(np.nan)) == 0x7F


def test_doubling_adds_one_to_the_exponent_field():
    pos = np.array([fp8.e4m3_value(c) for c in range(0x08, 0x76)], dtype=np.float32)  # normals < 256
    c1 = fp8.e4m3_encode(pos).astype(np.int64)
    c2 = fp8.e4m3_encode(pos * np.float32(2)).astype(np.int64)
    assert np.array_equal(c2, c1 + 8)


def test_quantize_rounds_the_float32_quotient():
    # 0.1 is not a float32; x / 0.1 in float32 differs from the float64 quotient
    # for some x: the code follows the float32 quotient (the stated reading)
    rng = np.random.default_rng(3)
    x = synth_round_fp16(rng.standard_normal(4096).astype(np.float32))
    q32 = x.astype(np.float32) / np.float32(0.1)
    assert np.array_equal(fp8.quantize_ref(x, "fp16", 0.1), fp8.e4m3_encode(q32))
    # with scale 1 the codes are the nearest E4M3 values of the inputs themselves
    assert np.array_equal(fp8.quantize_ref(x, "fp16", 1.0), fp8.e4m3_encode(x.astype(np.float32)))


def synth_round_fp16(x):
    return x.astype(np.float16)


def test_fp8_attention_equals_16bit_attention_on_exact_values():
    """With a power-of-two scale the dequantised values are exact in fp16, so
    the fp8 reference must equal the (pinned) 16-bit reference on a cache that
    stores those fp16 values."""
    rng = np.random.default_rng(11)
    NB, hkv, hq, S = 12, 2, 4, 3
    kc8 = rng.integers(0, 256, (NB, 16, hkv, 128)).astype(np.uint8)
    vc8 = rng.integers(0, 256, (NB, 16, hkv, 128)).astype(np.uint8)
    for c in (kc8, vc8):  # no NaN codes in the live rows
        c[np.isin(c, fp8.E4M3_NAN_CODES)] = 0x38
    ks, vs = 2.0 ** -5, 2.0 ** -3
    kc16 = (fp8.e4m3_decode(kc8) * ks).astype(np.float16)
    vc16 = (fp8.e4m3_decode(vc8) * vs).astype(np.float16)
    assert np.array_equal(kc16.astype(np.float64), fp8.e4m3_decode(kc8) * ks)
    q = rng.standard_normal((S, hq, 128)).astype(np.float16)
    tables = np.array([rng.permutation(NB)[:4] for _ in range(S)], dtype=np.int32)
    lens = np.array([1, 37, 64])
    a = fp8.paged_decode_fp8_ref(q, kc8, vc8, tables, lens, 0.0884, hkv, "fp16", ks, vs)
    b = oracle.paged_decode_ref(q, kc16, vc16, tables, lens, 0.0884, hkv, "fp16")
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)


def test_fp8_single_token_returns_dequantised_v():
    rng = np.random.default_rng(12)
    kc8 = rng.integers(0, 0x7F, (4, 16, 1, 128)).astype(np.uint8)
    vc8 = rng.integers(0, 0x7F, (4, 16, 1, 128)).astype(np.uint8)
    q = rng.standard_normal((1, 2, 128)).astype(np.float16)
    out = fp8.paged_decode_fp8_ref(q, kc8, vc8, np.array([[2, 0]]), [1], 0.1, 1, "fp16", 0.5, 0.025)
    want = fp8.e4m3_decode(vc8[2, 0, 0]) * np.float64(np.float32(0.025))
    assert np.array_equal(out[0, 0], want) and np.array_equal(out[0, 1], want)


def test_fp8_scatter_writes_the_codes_of_each_row():
    rng = np.random.default_rng(13)
    k = rng.standard_normal((5, 2, 128)).astype(np.float16)
    v = rng.standard_normal((5, 2, 128)).astype(np.float16)
    kc8, vc8 = fp8.new_fp8_cache(4, 16, 2, 128, fill=0xFF)
    slots = np.array([3, -1, 17, 63, 0])
    fp8.scatter_fp8_ref(kc8, vc8, k, v, slots, "fp16", 0.03, 0.05)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(kc8[s // 16, s % 16], fp8.quantize_ref(k[i], "fp16", 0.03))
        assert np.array_equal(vc8[s // 16, s % 16], fp8.quantize_ref(v[i], "fp16", 0.05))
    untouched = np.ones((4, 16), dtype=bool)
    for s in slots[slots >= 0]:
        untouched[s // 16, s % 16] = False
    assert np.all(kc8[untouched] == 0xFF)


@pytest.mark.parametrize("dtype,groups", [("fp16", 1), ("bf16", 0)])
def test_fp8_step_equals_brute_force_on_dequantised_rows(dtype, groups):
    """A whole oracle decode step over an fp8 cache (block manager, quantising
    write, copy-on-write, paged read) equals the explicit-loop formula on each
    sequence's contiguous rows, quantised and dequantised token by token:
    paging changes where the codes live, not the result."""
    import synth
    wl = synth.make_random_workload(40 + groups, num_seqs=5, num_heads=4, num_kv_heads=2, dtype=dtype,
                                    max_len=60, groups=groups, kv_dtype="fp8e4m3", k_scale=0.02, v_scale=0.03)
    st = oracle.run_decode_step(wl)
    for s in range(wl.num_seqs):
        k, v = wl.seq_kv(s)
        kd = fp8.e4m3_decode(fp8.quantize_ref(k, dtype, wl.k_scale)) * np.float64(np.float32(wl.k_scale))
        vd = fp8.e4m3_decode(fp8.quantize_ref(v, dtype, wl.v_scale)) * np.float64(np.float32(wl.v_scale))
        ref = oracle.brute_force_ref(oracle.to_f64(wl.q[s], dtype), kd, vd, wl.scale)
        np.testing.assert_allclose(st.out[s], ref, rtol=0, atol=1e-12)


# --- per-KV-head scales --------------------------------------------------


def _rows(seed, n=40, hkv=3, dtype="fp16", spread=(0.25, 4.0)):
    rng = np.random.default_rng(seed)
    s = rng.uniform(*spread, hkv).astype(np.float32)
    x = (rng.standard_normal((n, hkv, 128)) * s[None, :, None]).astype(np.float32)
    return (x.astype(np.float16) if dtype == "fp16" else synth_bf16(x)), s


def synth_bf16(x):
    import synth
    return synth.round_bf16_bits(x)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_per_head_codes_are_the_one_scale_codes_head_by_head(dtype):
    """Each head's codes under its own scale are exactly the codes of that
    head's rows quantised alone with that one scale (the pinned case)."""
    x, s = _rows(21, dtype=dtype)
    scales = (0.01 * s).astype(np.float32)
    codes = fp8.quantize_ref(x, dtype, scales)
    for h in range(x.shape[1]):
        assert np.array_equal(codes[:, h], fp8.quantize_ref(x[:, h], dtype, float(scales[h])))
    # and against torch's encoder on the float32 quotient of each head
    xf = oracle.to_f64(x, dtype).astype(np.float32) / scales[None, :, None]
    below = np.abs(xf) < fp8.E4M3_MAX
    ref = torch.from_numpy(xf).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[below], ref[below])


def test_equal_per_head_scales_equal_one_scale():
    x, _ = _rows(22)
    a = fp8.quantize_ref(x, "fp16", 0.03)
    b = fp8.quantize_ref(x, "fp16", np.full(3, 0.03, np.float32))
    assert np.array_equal(a, b)
    codes = a[:, None]  # [L, 1 token slot, ...] -> decode through the per-head path
    assert np.array_equal(fp8.dequantize_ref(a, 0.03), fp8.dequantize_ref(a, [0.03, 0.03, 0.03]))
    del codes


def test_per_head_scales_planted_mistakes():
    """Scales applied to the wrong heads, or one scale for all, change codes."""
    x, s = _rows(23)
    scales = (0.01 * s).astype(np.float32)
    good = fp8.quantize_ref(x, "fp16", scales)
    assert not np.array_equal(good, fp8.quantize_ref(x, "fp16", scales[::-1].copy()))
    assert not np.array_equal(good, fp8.quantize_ref(x, "fp16", float(scales.mean())))
    with pytest.raises(ValueError):
        fp8.quantize_ref(x, "fp16", scales[:2])


def test_per_head_dequantised_values():
    """decode(code) * the scale of the row's head, by explicit loops."""
    rng = np.random.default_rng(24)
    codes = rng.integers(0, 0x7F, (5, 4, 128)).astype(np.uint8)
    sc = np.float32([0.5, 0.125, 0.03, 2.0])
    got = fp8.dequantize_ref(codes, sc)
    for t in range(5):
        for h in range(4):
            for d in (0, 17, 127):
                assert got[t, h, d] == fp8.e4m3_value(codes[t, h, d]) * float(sc[h])


@pytest.mark.parametrize("dtype,groups", [("fp16", 1), ("bf16", 0)])
def test_fp8_step_with_per_head_scales_equals_brute_force(dtype, groups):
    """A whole oracle decode step over an fp8 cache with per-KV-head K and V
    scales equals the explicit-loop formula on each sequence's contiguous
    rows, quantised and dequantised head by head."""
    import synth
    ks = (0.012, 0.05, 0.02)
    vs = (0.03, 0.01, 0.02)
    wl = synth.make_random_workload(60 + groups, num_seqs=5, num_heads=6, num_kv_heads=3, dtype=dtype,
                                    max_len=60, groups=groups, key_scale=(0.5, 2.0), kv_dtype="fp8e4m3",
                                    k_scale=ks, v_scale=vs)
    assert wl.k_scale.shape == (3,)
    st = oracle.run_decode_step(wl)
    for s in range(wl.num_seqs):
        k, v = wl.seq_kv(s)
        kc, vc = fp8.quantize_ref(k, dtype, ks), fp8.quantize_ref(v, dtype, vs)
        kd = np.stack([[fp8.e4m3_decode(kc[t, h]) * float(np.float32(ks[h])) for h in range(3)]
                       for t in range(k.shape[0])])
        vd = np.stack([[fp8.e4m3_decode(vc[t, h]) * float(np.float32(vs[h])) for h in range(3)]
                       for t in range(v.shape[0])])
        ref = oracle.brute_force_ref(oracle.to_f64(wl.q[s], dtype), kd, vd, wl.scale)
        np.testing.assert_allclose(st.out[s], ref, rtol=0, atol=1e-12)
