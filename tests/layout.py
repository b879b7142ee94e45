"""Host decode/encode of the library's page layouts (16-bit and fp8), written
from the formulas documented in include/pagedkv.h (test helper; shares no code
with the kernels).  Canonical form: [num_blocks, 16, num_kv_heads, 128]."""

import numpy as np


def _offsets():
    t = np.arange(16)[:, None]
    d = np.arange(128)[None, :]
    k = (d // 8) * 128 + t * 8 + d % 8
    v = ((d // 16) // 2) * 512 + (16 * (t // 4) + d % 16) * 8 + ((d // 16) % 2) * 4 + t % 4
    return k, v


K_OFF, V_OFF = _offsets()


def _offsets_fp8():
    t = np.arange(16)[:, None]
    d = np.arange(128)[None, :]
    k = (d // 64) * 1024 + (16 * ((d // 8) % 4) + t) * 16 + ((d // 32) % 2) * 8 + d % 8
    v = (d // 64) * 1024 + (16 * (t // 4) + d % 16) * 16 + ((d // 32) % 2) * 8 + ((d // 16) % 2) * 4 + t % 4
    return k, v


K_OFF8, V_OFF8 = _offsets_fp8()


def _off(which: str, fp8: bool):
    if fp8:
        return K_OFF8 if which == "k" else V_OFF8
    return K_OFF if which == "k" else V_OFF


def decode_pages(pages: np.ndarray, which: str, fp8: bool = False) -> np.ndarray:
    """pages: [NB, Hkv, 2048] -> canonical [NB, 16, Hkv, 128]."""
    off = _off(which, fp8)
    x = pages[:, :, off]  # [NB, Hkv, 16, 128]
    return np.ascontiguousarray(x.transpose(0, 2, 1, 3))


def encode_pages(canon: np.ndarray, which: str, fp8: bool = False) -> np.ndarray:
    """canonical [NB, 16, Hkv, 128] -> pages [NB, Hkv, 2048]."""
    off = _off(which, fp8)
    nb, _, hkv, _ = canon.shape
    pages = np.empty((nb, hkv, 2048), dtype=canon.dtype)
    pages[:, :, off] = canon.transpose(0, 2, 1, 3)
    return pages
