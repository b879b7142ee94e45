"""Pins of the oracle's widening of stored 16-bit values (oracle/numerics.py).

Every attention reference reads the K, V and query values through
``oracle.to_f64``: these are the values the kernel reads (page "vLLM 深度解析：
以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §2.1, the QK dot products
and the weighted V sum act on the cached fp16/bf16 elements).  A wrong
widening would pass every other oracle test, because both sides of those
comparisons go through it, so it is pinned here against things that do not
use it:

* torch's own float16 and bfloat16 conversions to float64, an independent
  implementation, on all 65,536 bit patterns;
* closed forms written from the IEEE-754 binary16 and bfloat16 definitions
  (sign, 5 or 8 exponent bits, 10 or 7 fraction bits);
* planted mistakes (a shift by 15, a lost sign bit, swapped bytes) fail the
  same checks.
"""

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")

ALL = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def _torch_bf16_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _torch_f16_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.float16)
    return t.to(torch.float64).numpy()


def _same(a: np.ndarray, b: np.ndarray) -> bool:
    """Equal as values, with the same sign of zero and NaN in the same places."""
    na, nb = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb):
        return False
    return bool(np.array_equal(a[~na], b[~na]) and np.array_equal(np.signbit(a[~na]), np.signbit(b[~na])))


def _bf16_closed_forms_hold(widen) -> bool:
    """bfloat16 = 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits."""
    cases = {
        0x3F80: 1.0,  # exponent 127, fraction 0
        0xC020: -2.5,  # -(1 + 1/4) * 2^1
        0x0001: 2.0 ** -133,  # smallest subnormal: 2^-126 * 2^-7
        0x007F: 127 * 2.0 ** -133,  # largest subnormal
        0x0080: 2.0 ** -126,  # smallest normal
        0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
        0x7F80: np.inf,
        0xFF80: -np.inf,
        0x4049: 3.140625,  # (1 + 73/128) * 2
    }
    bits = np.array(list(cases), dtype=np.uint16)
    got = widen(bits)
    want = np.array(list(cases.values()), dtype=np.float64)
    if not np.array_equal(got, want):
        return False
    z = widen(np.array([0x0000, 0x8000], dtype=np.uint16))
    return bool(z[0] == 0 and z[1] == 0 and not np.signbit(z[0]) and np.signbit(z[1])
                and np.isnan(widen(np.array([0x7FC0], dtype=np.uint16))[0]))


def test_bf16_widening_matches_torch_on_every_pattern():
    got = oracle.to_f64(ALL, "bf16")
    assert got.dtype == np.float64
    assert _same(got, _torch_bf16_f64(ALL))
    # every non-NaN pattern is a distinct value except the two zeros
    finite = got[np.isfinite(got)]
    assert finite.size == 65536 - 256  # exponent field all ones: 2 infinities, 254 NaN patterns
    assert np.unique(finite).size == finite.size - 1


def test_bf16_widening_closed_forms():
    assert _bf16_closed_forms_hold(lambda b: oracle.to_f64(b, "bf16"))


def test_fp16_widening_matches_torch_on_every_pattern():
    x = ALL.view(np.float16)
    got = oracle.to_f64(x, "fp16")
    assert _same(got, _torch_f16_f64(ALL))
    cases = {0x3C00: 1.0, 0xC100: -2.5, 0x0001: 2.0 ** -24, 0x0400: 2.0 ** -14, 0x7BFF: 65504.0,
             0x7C00: np.inf}
    b = np.array(list(cases), dtype=np.uint16).view(np.float16)
    assert np.array_equal(oracle.to_f64(b, "fp16"), np.array(list(cases.values())))


def test_bf16_widening_is_the_upper_half_of_float32():
    """A bfloat16 is the upper 16 bits of the float32 of the same value, so
    torch's float32 -> bfloat16 conversion of a value with zero low bits is
    exact and the widening gives the value back."""
    rng = np.random.default_rng(3)
    f = rng.standard_normal(4096).astype(np.float32)
    f = (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)
    bits = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.to_f64(bits, "bf16"), f.astype(np.float64))


def test_planted_widening_mistakes_fail():
    """The checks above have teeth: each plausible slip fails them."""
    def shift15(b):
        return (b.astype(np.uint32) << np.uint32(15)).view(np.float32).astype(np.float64)

    def no_sign(b):
        return ((b.astype(np.uint32) & np.uint32(0x7FFF)) << np.uint32(16)).view(np.float32).astype(np.float64)

    def byteswap(b):
        return (b.byteswap().astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)

    def as_fp16(b):
        return b.view(np.float16).astype(np.float64)

    ref = _torch_bf16_f64(ALL)
    with np.errstate(invalid="ignore"):
        for wrong in (shift15, no_sign, byteswap, as_fp16):
            assert not _same(wrong(ALL), ref), wrong.__name__
            assert not _bf16_closed_forms_hold(wrong), wrong.__name__
