"""FP8 (E4M3) KV cache, oracle side — TEST INFRASTRUCTURE ONLY.

Page "vLLM 深度解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §三
(quantisation), says the KV cache itself can be stored quantised.  It names
neither the 8-bit format nor how values are scaled, so this module takes the
plainest readings, stated here and in the tests:

* format: the OCP 8-bit floating-point E4M3 encoding — 1 sign bit, 4 exponent
  bits with bias 7, 3 mantissa bits; exponent field 0 holds the subnormals
  (m / 8) * 2^-6; there are no infinities; S.1111.111 is NaN; the largest
  finite magnitude is 448;
* scaling: a float32 scale for K and one for V, either one per cache or one
  per KV head (``k_scale`` / ``v_scale`` given as a float, or as a sequence of
  ``num_kv_heads`` floats, element h applying to every row of KV head h); the
  stored code of a value x of head h is the E4M3 value nearest to the float32
  quotient x / scale_h (one IEEE float32 division), ties to the even mantissa,
  finite magnitudes beyond 448 saturated to 448, the sign of zero kept; the
  value a code stands for is decode(code) * scale_h;
* attention over an fp8 cache is the same softmax attention (``attention_ref``)
  over the dequantised rows, in float64; queries and outputs stay fp16/bf16.

Everything is written from the definition: the encoder picks the nearest
representable value by search over the sorted finite values, not by bit
manipulation.  Pins (``tests/test_oracle_fp8.py``): the closed-form values the
definition fixes (1, 448, 2^-6, 2^-9, -0, NaN), brute-force nearest-value
search over all codes, and torch's own float8_e4m3fn conversion where its
semantics coincide (every decode; encodes below the saturation bound).  Per-head
scales reduce, head by head, to the one-scale case (pinned the same way), and
equal per-head scales give exactly the one-scale results.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

from .attention import attention_ref, gather_seq
from .numerics import to_f64

E4M3_MAX = 448.0
E4M3_NAN_CODES = (0x7F, 0xFF)


def e4m3_value(code: int) -> float:
    """The value an E4M3 code stands for (float; NaN for the two NaN codes)."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_table() -> np.ndarray:
    """float64 [256]: the value of every code."""
    return np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


# non-negative finite values, increasing, and their codes (0x00 .. 0x7E)
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = np.array([e4m3_value(c) for c in range(0x7F)], dtype=np.float64)


def e4m3_encode(x) -> np.ndarray:
    """uint8 codes of float32 values x (any shape): nearest finite E4M3 value,
    ties to the even mantissa (even code), saturating beyond 448; NaN -> NaN
    code of the same sign."""
    xf = np.asarray(x, dtype=np.float32)
    a = np.abs(xf.astype(np.float64)).ravel()
    neg = np.signbit(xf).ravel()
    out = np.empty(a.shape, dtype=np.int64)
    nan = np.isnan(a)
    sat = ~nan & (a >= E4M3_MAX)
    mid = ~nan & ~sat
    # neighbours lo <= a < hi among the finite non-negative values
    hi_i = np.searchsorted(_POS_VALUES, a[mid], side="right")
    lo_i = hi_i - 1
    lo_v = _POS_VALUES[lo_i]
    hi_v = _POS_VALUES[hi_i]  # a < 448 so hi_i <= 0x7E
    d_lo = a[mid] - lo_v
    d_hi = hi_v - a[mid]
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi_i] % 2 == 0))
    out[mid] = np.where(take_hi, _POS_CODES[hi_i], _POS_CODES[lo_i])
    out[sat] = 0x7E
    out[nan] = 0x7F
    out = out | np.where(neg, 0x80, 0)
    return out.astype(np.uint8).reshape(xf.shape)


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of uint8 codes (any shape)."""
    return e4m3_table()[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def head_scales(scale, rows: np.ndarray) -> np.ndarray:
    """The float32 scale as an array that broadcasts over rows [..., Hkv, D]:
    a 0-d array for one scale per cache, [Hkv, 1] for one scale per KV head."""
    s = np.asarray(scale, dtype=np.float32)
    if s.ndim == 0:
        return s
    if rows.ndim < 2 or s.shape != (rows.shape[-2],):
        raise ValueError(f"per-head scales of shape {s.shape} do not match rows of shape {rows.shape}")
    return s[:, None]


def quantize_ref(x: np.ndarray, act_dtype: str, scale) -> np.ndarray:
    """E4M3 codes of stored fp16/bf16 rows x [..., Hkv, D] under a float32
    scale per cache or per KV head: the nearest code to float32(x) /
    float32(scale of the row's head)."""
    xf = to_f64(x, act_dtype).astype(np.float32)  # exact: fp16 and bf16 fit float32
    return e4m3_encode(xf / head_scales(scale, xf))


def dequantize_ref(codes: np.ndarray, scale) -> np.ndarray:
    """float64 values of codes [..., Hkv, D]: decode(code) * the row head's scale."""
    return e4m3_decode(codes) * head_scales(scale, np.asarray(codes)).astype(np.float64)


def new_fp8_cache(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int, fill: int = 0):
    shape = (num_blocks, block_size, num_kv_heads, head_size)
    return np.full(shape, fill, dtype=np.uint8), np.full(shape, fill, dtype=np.uint8)


def scatter_fp8_ref(k_cache8, v_cache8, k, v, slot_mapping, act_dtype: str, k_scale, v_scale):
    """The slot-mapped write into an fp8 cache: for each token i with slot >= 0,
    block slot // bs, offset slot % bs receives the codes of k[i], v[i]
    (scales per cache or per KV head)."""
    bs = k_cache8.shape[1]
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        k_cache8[slot // bs, slot % bs] = quantize_ref(k[i], act_dtype, k_scale)
        v_cache8[slot // bs, slot % bs] = quantize_ref(v[i], act_dtype, v_scale)


def paged_decode_fp8_ref(q: np.ndarray, k_cache8: np.ndarray, v_cache8: np.ndarray, block_tables: np.ndarray,
                         context_lens: Sequence[int], scale: float, num_kv_heads: int, act_dtype: str,
                         k_scale, v_scale, seqs: Sequence[int] = None) -> np.ndarray:
    """Paged decode attention over an fp8 cache: the rows gathered through the
    block table are dequantised (decode(code) * the scale of the row's head,
    float64) and attended to with the plain softmax definition.  Returns
    float64 [len(seqs), Hq, D]."""
    S, hq, d = q.shape
    assert k_cache8.dtype == np.uint8 and k_cache8.shape[2] == num_kv_heads
    if seqs is None:
        seqs = range(S)
    out = []
    for s in seqs:
        L = int(context_lens[s])
        k = dequantize_ref(gather_seq(k_cache8, block_tables[s], L), k_scale)
        v = dequantize_ref(gather_seq(v_cache8, block_tables[s], L), v_scale)
        out.append(attention_ref(to_f64(q[s], act_dtype), k, v, scale))
    return np.stack(out)
