"""Paged decode attention for MI355X (gfx950): Python binding of libpagedkv.so.

Thin ctypes wrappers with the names of the C ABI in ``include/pagedkv.h``.
They only marshal arguments — tensor pointers, shapes and the current HIP
stream — and every step of the computation runs in the library's kernels.
There is no fallback: if the library is not built or a tensor is not on the
GPU, the call raises.

Tensors (PyTorch is used for device memory and streams only):
  q, out          [num_seqs, num_heads, 128]          float16 / bfloat16, GPU
  k_cache, v_cache [num_blocks, num_kv_heads, 2048]   same dtype, GPU; the page
                   layout inside the last dimension is the library's own (see
                   pagedkv.h); use ``gather_cache`` or ``k_index``/``v_index`` to
                   read it.  An fp8 (E4M3) cache is a uint8 tensor of codes of
                   the same shape, used through the ``*_fp8`` calls, which take
                   the K and V scales
  block_tables    int32 [num_seqs, max_blocks_per_seq], GPU
  context_lens    int32 [num_seqs], GPU
  slot_mapping    int32 [num_tokens], GPU
  block_pairs     int32 [num_pairs, 2], GPU
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

BLOCK_SIZE = 16
HEAD_SIZE = 128
PAGE_ELEMS = BLOCK_SIZE * HEAD_SIZE

PKV_OK = 0
PKV_ERR_INVALID = 1
PKV_ERR_UNSUPPORTED = 2
PKV_ERR_DEVICE = 3
PKV_ERR_OUT_OF_BLOCKS = 4
PKV_F16 = 0
PKV_BF16 = 1
PKV_FP8_E4M3 = 2
NOALLOC_SCRATCH_BYTES = 32 << 20  # PKV_NOALLOC_SCRATCH_BYTES: the scratch of paged_attn_decode_noalloc

# Every symbol pagedkv.h declares, with (restype, argtypes).
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_fl = ctypes.c_float
_i32p = ctypes.POINTER(ctypes.c_int32)


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", _i32), ("block_size", _i32), ("num_kv_heads", _i32),
                ("head_size", _i32), ("dtype", _i32)]


class Fp8Scales(ctypes.Structure):
    _fields_ = [("act_dtype", _i32), ("k_scale", _fl), ("v_scale", _fl), ("k_head_scales", _vp),
                ("v_head_scales", _vp)]


_DP = ctypes.POINTER(CacheDesc)
_SP = ctypes.POINTER(Fp8Scales)

SIGNATURES = {
    "pkv_cache_bytes": (_sz, [_DP]),
    "pkv_k_index": (_i64, [_DP, _i32, _i32, _i32, _i32]),
    "pkv_v_index": (_i64, [_DP, _i32, _i32, _i32, _i32]),
    "paged_attn_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _DP, _i32,
                                 _vp, _sz, _vp]),
    "paged_attn_decode_plan": (_i32, [_vp, _i32, _i32, _i32, _DP, _i32, _vp, _sz, _vp]),
    "paged_attn_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _DP, _i32,
                                         _vp]),
    "paged_attn_decode_read_pages": (_i32, [_vp, _vp, _vp, _vp, _i32, _i32, _i32, _DP, _i32, _vp, _sz, _vp, _vp]),
    "paged_attn_decode_run": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _DP, _i32,
                                     _vp, _sz, _vp]),
    "paged_attn_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _DP]),
    "paged_attn_prefill_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _DP]),
    "paged_attn_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _i32, _i32, _DP,
                                  _i32, _vp, _sz, _vp]),
    "paged_attn_prefill_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _DP, _SP, _i32, _vp, _sz, _vp]),
    "paged_attn_decode_partition_tokens": (_i32, [_i32, _i32, _i32, _i32, _DP]),
    "reshape_and_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _DP, _vp]),
    "reshape_and_cache_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _DP, _SP, _vp]),
    "paged_attn_decode_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _DP, _SP,
                                     _i32, _vp, _sz, _vp]),
    "paged_attn_decode_run_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _fl, _i32, _i32, _i32, _i32, _DP, _SP,
                                         _i32, _vp, _sz, _vp]),
    "copy_blocks": (_i32, [_vp, _vp, _vp, _i32, _DP, _vp]),
    "decode_step_prologue": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _DP, _i32, _vp,
                                    _sz, _vp]),
    "decode_step_prologue_fp8": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _DP, _SP,
                                        _i32, _vp, _sz, _vp]),
    "swap_blocks": (_i32, [_vp, _vp, _DP, _vp, _vp, _DP, _vp, _i32, _vp]),
    "gather_cache": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _DP, _vp]),
    "pkv_status_string": (ctypes.c_char_p, [_i32]),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_bm_create": (_vp, [_i32, _i32, _i32p]),
    "pkv_bm_destroy": (None, [_vp]),
    "pkv_bm_add": (_i32, [_vp, _i32, _i32, _i32p]),
    "pkv_bm_fork": (_i32, [_vp, _i32, _i32]),
    "pkv_bm_append_slot": (_i32, [_vp, _i32, _i32p, _i32p]),
    "pkv_bm_step": (_i32, [_vp, _i32p, _i32, _i32p, _i32p, _i32p]),
    "pkv_bm_free": (_i32, [_vp, _i32]),
    "pkv_bm_block_table": (_i32, [_vp, _i32p, _i32, _i32, _i32p, _i32p]),
    "pkv_bm_num_free": (_i32, [_vp]),
    "pkv_bm_refcount": (_i32, [_vp, _i32]),
    "pkv_bm_length": (_i32, [_vp, _i32]),
    "pkv_bm_num_seq_blocks": (_i32, [_vp, _i32]),
    "pkv_bm_waste": (_i32, [_vp, _i32]),
    "pkv_bm_free_list": (_i32, [_vp, _i32p, _i32]),
    "pkv_bm_add_cached": (_i32, [_vp, _i32, _i32, _i32p, _i32p, _i32p]),
    "pkv_bm_append_token": (_i32, [_vp, _i32, _i32, _i32p, _i32p]),
    "pkv_bm_num_evictable": (_i32, [_vp]),
}

_LIB = None


from . import validate as _validate  # noqa: E402  (host contract checks under PKV_VALIDATE=1)


class PagedKVError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class OutOfBlocks(PagedKVError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built.

    PyTorch is imported first: its wheel ships its own HIP and HSA runtimes,
    and the library must bind to those (same soname) rather than load the
    system copies beside them, which would leave two runtimes in one process
    and device pointers from one used with the other."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_345_amd.build`")
        _torch()
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = handle
    return _LIB


def status_string(status: int) -> str:
    return lib().pkv_status_string(status).decode()


def version() -> str:
    return lib().pkv_version().decode()


def _check(status: int, what: str) -> None:
    if status == PKV_ERR_OUT_OF_BLOCKS:
        raise OutOfBlocks(status, what)
    if status != PKV_OK:
        raise PagedKVError(status, what)


# ---------------------------------------------------------------------------
# tensors and streams
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    return _code_of_dtype(t.dtype)


def _code_of_dtype(dtype) -> int:
    torch = _torch()
    if dtype == torch.float16:
        return PKV_F16
    if dtype == torch.bfloat16:
        return PKV_BF16
    if dtype == torch.uint8:  # a cache of E4M3 codes
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported dtype {dtype}; expected float16, bfloat16 or uint8 (fp8 E4M3 codes)")


def _gpu(t, name: str, dtype=None, ndim: Optional[int] = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    return t.data_ptr()


def _stream_handle(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def cache_desc(num_blocks: int, num_kv_heads: int, dtype) -> CacheDesc:
    """dtype: a PKV_* code, or torch.float16 / torch.bfloat16 / torch.uint8 (fp8 E4M3 codes)."""
    code = dtype if isinstance(dtype, int) else _code_of_dtype(dtype)
    return CacheDesc(int(num_blocks), BLOCK_SIZE, int(num_kv_heads), HEAD_SIZE, code)


def fp8_scales(act_dtype, k_scale, v_scale, num_kv_heads: Optional[int] = None) -> Fp8Scales:
    """act_dtype: torch.float16 / torch.bfloat16 (or a PKV_* code) of q, out and
    the new rows.  k_scale / v_scale: a float (one scale per cache), or a GPU
    float32 tensor [num_kv_heads] of per-head scales (its pointer is passed)."""
    code = act_dtype if isinstance(act_dtype, int) else _code_of_dtype(act_dtype)

    def one(x, name):
        if hasattr(x, "data_ptr"):
            torch = _torch()
            ptr = _gpu(x, name, torch.float32, 1)
            if num_kv_heads is not None and x.shape[0] != num_kv_heads:
                raise ValueError(f"{name} must have num_kv_heads = {num_kv_heads} entries")
            if _validate.enabled():
                _validate.check_head_scales(x, name)
            return 1.0, ptr
        return float(x), None

    ks, kp = one(k_scale, "k_scale")
    vs, vp = one(v_scale, "v_scale")
    return Fp8Scales(int(code), ks, vs, kp, vp)


def _desc_of(k_cache) -> CacheDesc:
    if k_cache.dim() != 3 or k_cache.shape[2] != PAGE_ELEMS:
        raise ValueError(f"cache must be [num_blocks, num_kv_heads, {PAGE_ELEMS}], got {tuple(k_cache.shape)}")
    return CacheDesc(int(k_cache.shape[0]), BLOCK_SIZE, int(k_cache.shape[1]), HEAD_SIZE, _dtype_code(k_cache))


def allocate_cache(num_blocks: int, num_kv_heads: int, dtype, device="cuda") -> Tuple[object, object]:
    """Uninitialised K and V caches of pkv_cache_bytes() each."""
    torch = _torch()
    desc = cache_desc(num_blocks, num_kv_heads, dtype)
    nbytes = lib().pkv_cache_bytes(ctypes.byref(desc))
    if nbytes == 0:
        raise ValueError("invalid cache shape")
    shape = (num_blocks, num_kv_heads, PAGE_ELEMS)
    return (torch.empty(shape, dtype=dtype, device=device), torch.empty(shape, dtype=dtype, device=device))


def k_index(desc: CacheDesc, block: int, head: int, token: int, dim: int) -> int:
    return int(lib().pkv_k_index(ctypes.byref(desc), block, head, token, dim))


def v_index(desc: CacheDesc, block: int, head: int, token: int, dim: int) -> int:
    return int(lib().pkv_v_index(ctypes.byref(desc), block, head, token, dim))


# ---------------------------------------------------------------------------
# the hot path
# ---------------------------------------------------------------------------

def workspace_size(num_seqs: int, num_heads: int, max_blocks_per_seq: int, desc: CacheDesc,
                   partition_tokens: int = 0) -> int:
    n = lib().paged_attn_decode_workspace_size(num_seqs, num_heads, max_blocks_per_seq, partition_tokens,
                                               ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID, "paged_attn_decode_workspace_size")
    return int(n)


def partition_tokens_for(num_seqs: int, num_heads: int, max_blocks_per_seq: int, desc: CacheDesc,
                         partition_tokens: int = 0) -> int:
    n = lib().paged_attn_decode_partition_tokens(num_seqs, num_heads, max_blocks_per_seq, partition_tokens,
                                                 ctypes.byref(desc))
    if n < 0:
        raise PagedKVError(PKV_ERR_INVALID, "paged_attn_decode_partition_tokens")
    return int(n)


def _decode_args(out, q, k_cache, v_cache, block_tables, context_lens, num_kv_heads, partition_tokens, workspace):
    torch = _torch()
    desc = _desc_of(k_cache)
    cache_dtype = torch.uint8 if desc.dtype == PKV_FP8_E4M3 else q.dtype
    if desc.num_kv_heads != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    num_seqs, num_heads, hs = q.shape
    if hs != HEAD_SIZE or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_seqs, num_heads, 128]")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    mbps = int(block_tables.shape[1])
    ptrs = [_gpu(out, "out", q.dtype, 3), _gpu(q, "q", None, 3), _gpu(k_cache, "k_cache", cache_dtype),
            _gpu(v_cache, "v_cache", cache_dtype), _gpu(block_tables, "block_tables", torch.int32, 2),
            _gpu(context_lens, "context_lens", torch.int32, 1)]
    if context_lens.shape[0] != num_seqs or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("context_lens / v_cache shape mismatch")
    if _validate.enabled():
        _validate.check_tables(block_tables, context_lens, desc.num_blocks)
    need = workspace_size(num_seqs, num_heads, mbps, desc, partition_tokens) if num_seqs else 0
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = _gpu(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return ptrs, desc, num_seqs, num_heads, mbps, ws_ptr, ws_bytes


def paged_attn_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                      num_kv_heads: int, *, partition_tokens: int = 0, workspace=None, stream=None):
    """out[s, h] = softmax(scale * q[s, h] . K[s, :ctx, h // g]) V[s, :ctx, h // g]."""
    ptrs, desc, S, Hq, mbps, ws_ptr, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                             num_kv_heads, partition_tokens, workspace)
    st = lib().paged_attn_decode(*ptrs, float(scale), int(num_kv_heads), int(S), int(Hq), mbps,
                                 ctypes.byref(desc), int(partition_tokens), ws_ptr, ws_bytes,
                                 _stream_handle(stream))
    _check(st, "paged_attn_decode")
    return out


def paged_attn_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                              num_kv_heads: int, *, partition_tokens: int = 0, stream=None):
    """paged_attn_decode with the library's per-GPU scratch as its workspace:
    nothing is allocated, here or in the library.  Calls that overlap on one
    GPU share that scratch and race; serialise them."""
    torch = _torch()
    desc = _desc_of(k_cache)
    cache_dtype = torch.uint8 if desc.dtype == PKV_FP8_E4M3 else q.dtype
    if desc.num_kv_heads != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    num_seqs, num_heads, hs = q.shape
    if hs != HEAD_SIZE or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_seqs, num_heads, 128]")
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError("block_tables must be [num_seqs, max_blocks_per_seq]")
    mbps = int(block_tables.shape[1])
    ptrs = [_gpu(out, "out", q.dtype, 3), _gpu(q, "q", None, 3), _gpu(k_cache, "k_cache", cache_dtype),
            _gpu(v_cache, "v_cache", cache_dtype), _gpu(block_tables, "block_tables", torch.int32, 2),
            _gpu(context_lens, "context_lens", torch.int32, 1)]
    if context_lens.shape[0] != num_seqs or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("context_lens / v_cache shape mismatch")
    if num_seqs:
        need = workspace_size(num_seqs, num_heads, mbps, desc, partition_tokens)
        if need > NOALLOC_SCRATCH_BYTES:
            raise ValueError(f"paged_attn_decode_noalloc: this batch needs a {need}-byte workspace, more than the "
                             f"library's {NOALLOC_SCRATCH_BYTES}-byte scratch; call paged_attn_decode with a workspace")
    if _validate.enabled():
        _validate.check_tables(block_tables, context_lens, desc.num_blocks)
    st = lib().paged_attn_decode_noalloc(*ptrs, float(scale), int(num_kv_heads), int(num_seqs), int(num_heads), mbps,
                                         ctypes.byref(desc), int(partition_tokens), _stream_handle(stream))
    _check(st, "paged_attn_decode_noalloc")
    return out


def paged_attn_decode_read_pages(k_cache, v_cache, block_tables, context_lens, num_heads: int, sink, *, workspace,
                                 partition_tokens: int = 0, stream=None):
    """Diagnostic: the page reads of paged_attn_decode_run alone, from the work
    list paged_attn_decode_plan wrote into `workspace`; `sink` is a GPU int32
    tensor of at least 4 elements."""
    torch = _torch()
    desc = _desc_of(k_cache)
    num_seqs, mbps = block_tables.shape
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr, ws_bytes = _gpu(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = lib().paged_attn_decode_read_pages(_gpu(k_cache, "k_cache"), _gpu(v_cache, "v_cache", k_cache.dtype),
                                            _gpu(block_tables, "block_tables", torch.int32, 2),
                                            _gpu(context_lens, "context_lens", torch.int32, 1), int(num_seqs),
                                            int(num_heads), int(mbps), ctypes.byref(desc), int(partition_tokens),
                                            ws_ptr, ws_bytes, _gpu(sink, "sink", torch.int32), _stream_handle(stream))
    _check(st, "paged_attn_decode_read_pages")


def paged_attn_decode_plan(context_lens, num_heads: int, max_blocks_per_seq: int, k_cache, workspace, *,
                           partition_tokens: int = 0, stream=None):
    """Write the work list of a batch into `workspace` (see paged_attn_decode_run)."""
    torch = _torch()
    desc = _desc_of(k_cache)
    n = int(context_lens.shape[0])
    if _validate.enabled():
        _validate.check_lengths(context_lens, max_blocks_per_seq)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:  # None: the call needs no workspace (a batch run without a plan)
        ws_ptr, ws_bytes = _gpu(workspace, "workspace"), workspace.numel() * workspace.element_size()
    st = lib().paged_attn_decode_plan(_gpu(context_lens, "context_lens", torch.int32, 1), n, int(num_heads),
                                      int(max_blocks_per_seq), ctypes.byref(desc), int(partition_tokens),
                                      ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "paged_attn_decode_plan")


def paged_attn_decode_run(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                          num_kv_heads: int, *, workspace, partition_tokens: int = 0, stream=None):
    """paged_attn_decode from a work list already written by paged_attn_decode_plan."""
    ptrs, desc, S, Hq, mbps, ws_ptr, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                             num_kv_heads, partition_tokens, workspace)
    st = lib().paged_attn_decode_run(*ptrs, float(scale), int(num_kv_heads), int(S), int(Hq), mbps,
                                     ctypes.byref(desc), int(partition_tokens), ws_ptr, ws_bytes,
                                     _stream_handle(stream))
    _check(st, "paged_attn_decode_run")
    return out


def paged_attn_decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                          num_kv_heads: int, k_scale, v_scale, *, partition_tokens: int = 0,
                          workspace=None, stream=None):
    """paged_attn_decode over an fp8 (E4M3, uint8) cache whose codes stand for
    code value * k_scale (K) and code value * v_scale (V); q, out fp16/bf16.
    A scale is a float (one per cache) or a GPU float32 tensor [num_kv_heads]
    (one per KV head)."""
    ptrs, desc, S, Hq, mbps, ws_ptr, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                             num_kv_heads, partition_tokens, workspace)
    sc = fp8_scales(q.dtype, k_scale, v_scale, desc.num_kv_heads)
    st = lib().paged_attn_decode_fp8(*ptrs, float(scale), int(num_kv_heads), int(S), int(Hq), mbps,
                                     ctypes.byref(desc), ctypes.byref(sc), int(partition_tokens), ws_ptr, ws_bytes,
                                     _stream_handle(stream))
    _check(st, "paged_attn_decode_fp8")
    return out


def paged_attn_decode_run_fp8(out, q, k_cache, v_cache, block_tables, context_lens, scale: float,
                              num_kv_heads: int, k_scale, v_scale, *, workspace,
                              partition_tokens: int = 0, stream=None):
    """paged_attn_decode_fp8 from a work list written by paged_attn_decode_plan."""
    ptrs, desc, S, Hq, mbps, ws_ptr, ws_bytes = _decode_args(out, q, k_cache, v_cache, block_tables, context_lens,
                                                             num_kv_heads, partition_tokens, workspace)
    sc = fp8_scales(q.dtype, k_scale, v_scale, desc.num_kv_heads)
    st = lib().paged_attn_decode_run_fp8(*ptrs, float(scale), int(num_kv_heads), int(S), int(Hq), mbps,
                                         ctypes.byref(desc), ctypes.byref(sc), int(partition_tokens), ws_ptr,
                                         ws_bytes, _stream_handle(stream))
    _check(st, "paged_attn_decode_run_fp8")
    return out


def prefill_workspace_size(num_seqs: int, num_heads: int, max_blocks_per_seq: int, num_query_tokens: int,
                           max_query_len: int, desc: CacheDesc, partition_tokens: int = 0) -> int:
    n = lib().paged_attn_prefill_workspace_size(num_seqs, num_heads, max_blocks_per_seq, num_query_tokens,
                                                max_query_len, partition_tokens, ctypes.byref(desc))
    if n == ctypes.c_size_t(-1).value:
        raise PagedKVError(PKV_ERR_INVALID, "paged_attn_prefill_workspace_size")
    return int(n)


def paged_attn_prefill(out, q, k_cache, v_cache, block_tables, context_lens, query_start, scale: float,
                       num_kv_heads: int, *, max_query_len: int, k_scale: Optional[float] = None,
                       v_scale: Optional[float] = None, partition_tokens: int = 0, workspace=None, stream=None):
    """Chunked-prefill attention: chunk query j of sequence s (row
    query_start[s] + j) attends to cache tokens 0 .. context_lens[s] - C_s + j.
    With k_scale / v_scale the cache is fp8 (uint8 E4M3 codes) and
    paged_attn_prefill_fp8 is called."""
    torch = _torch()
    desc = _desc_of(k_cache)
    if desc.num_kv_heads != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    tq, num_heads, hs = q.shape
    if hs != HEAD_SIZE or tuple(out.shape) != tuple(q.shape):
        raise ValueError("q and out must be [num_query_tokens, num_heads, 128]")
    num_seqs, mbps = block_tables.shape
    if tuple(query_start.shape) != (num_seqs + 1,) or tuple(context_lens.shape) != (num_seqs,):
        raise ValueError("query_start must be [num_seqs + 1] and context_lens [num_seqs]")
    fp8 = desc.dtype == PKV_FP8_E4M3
    if fp8 != (k_scale is not None and v_scale is not None):
        raise ValueError("an fp8 cache needs k_scale and v_scale, a 16-bit cache takes neither")
    cache_dtype = torch.uint8 if fp8 else q.dtype
    if _validate.enabled():
        _validate.check_tables(block_tables, context_lens, desc.num_blocks)
        _validate.check_query_start(query_start, context_lens, tq, max_query_len)
    need = prefill_workspace_size(num_seqs, num_heads, mbps, tq, max_query_len, desc, partition_tokens)
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = _gpu(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    args = [_gpu(out, "out", q.dtype, 3), _gpu(q, "q", None, 3), _gpu(k_cache, "k_cache", cache_dtype),
            _gpu(v_cache, "v_cache", cache_dtype), _gpu(block_tables, "block_tables", torch.int32, 2),
            _gpu(context_lens, "context_lens", torch.int32, 1), _gpu(query_start, "query_start", torch.int32, 1),
            float(scale), int(num_kv_heads), int(num_seqs), int(num_heads), int(mbps), int(tq), int(max_query_len),
            ctypes.byref(desc)]
    if fp8:
        sc = fp8_scales(q.dtype, k_scale, v_scale, desc.num_kv_heads)
        st = lib().paged_attn_prefill_fp8(*args, ctypes.byref(sc), int(partition_tokens), ws_ptr, ws_bytes,
                                          _stream_handle(stream))
    else:
        st = lib().paged_attn_prefill(*args, int(partition_tokens), ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "paged_attn_prefill" + ("_fp8" if fp8 else ""))
    return out


def reshape_and_cache(k, v, k_cache, v_cache, slot_mapping, *, stream=None):
    """Write k[i], v[i] ([num_kv_heads, 128]) of every token i to slot_mapping[i]."""
    torch = _torch()
    desc = _desc_of(k_cache)
    n = int(slot_mapping.shape[0])
    if tuple(k.shape) != (n, desc.num_kv_heads, HEAD_SIZE) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k, v must be [num_tokens, num_kv_heads, 128]")
    if _validate.enabled():
        _validate.check_slots(slot_mapping, desc.num_blocks)
    st = lib().reshape_and_cache(_gpu(k, "k", k_cache.dtype), _gpu(v, "v", k_cache.dtype),
                                 _gpu(k_cache, "k_cache"), _gpu(v_cache, "v_cache", k_cache.dtype),
                                 _gpu(slot_mapping, "slot_mapping", torch.int32, 1), n, ctypes.byref(desc),
                                 _stream_handle(stream))
    _check(st, "reshape_and_cache")


def reshape_and_cache_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale, *, stream=None):
    """Write the E4M3 codes of k[i] / k_scale and v[i] / v_scale (fp16/bf16 rows
    [num_kv_heads, 128]) of every token i to slot_mapping[i] of a uint8 cache.
    A scale is a float (one per cache) or a GPU float32 tensor [num_kv_heads]
    (one per KV head)."""
    torch = _torch()
    desc = _desc_of(k_cache)
    n = int(slot_mapping.shape[0])
    if tuple(k.shape) != (n, desc.num_kv_heads, HEAD_SIZE) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k, v must be [num_tokens, num_kv_heads, 128]")
    if _validate.enabled():
        _validate.check_slots(slot_mapping, desc.num_blocks)
    sc = fp8_scales(k.dtype, k_scale, v_scale, desc.num_kv_heads)
    st = lib().reshape_and_cache_fp8(_gpu(k, "k"), _gpu(v, "v", k.dtype), _gpu(k_cache, "k_cache", torch.uint8),
                                     _gpu(v_cache, "v_cache", torch.uint8),
                                     _gpu(slot_mapping, "slot_mapping", torch.int32, 1), n, ctypes.byref(desc),
                                     ctypes.byref(sc), _stream_handle(stream))
    _check(st, "reshape_and_cache_fp8")


def copy_blocks(k_cache, v_cache, block_pairs, *, stream=None):
    """Copy every (src, dst) block of block_pairs, K and V, all heads."""
    torch = _torch()
    desc = _desc_of(k_cache)
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    n = int(block_pairs.shape[0])
    if n == 0:
        return
    if _validate.enabled():
        _validate.check_copy_pairs(block_pairs, desc.num_blocks)
    st = lib().copy_blocks(_gpu(k_cache, "k_cache"), _gpu(v_cache, "v_cache", k_cache.dtype),
                           _gpu(block_pairs, "block_pairs", torch.int32, 2), n, ctypes.byref(desc),
                           _stream_handle(stream))
    _check(st, "copy_blocks")


def _prologue_args(k, v, k_cache, slot_mapping, block_pairs, context_lens, max_blocks_per_seq, workspace):
    desc = _desc_of(k_cache)
    n = int(slot_mapping.shape[0])
    if tuple(k.shape) != (n, desc.num_kv_heads, HEAD_SIZE) or tuple(v.shape) != tuple(k.shape):
        raise ValueError("k, v must be [num_tokens, num_kv_heads, 128]")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [num_pairs, 2]")
    npairs = int(block_pairs.shape[0])
    S = int(context_lens.shape[0])
    if _validate.enabled():
        _validate.check_slots(slot_mapping, desc.num_blocks)
        if npairs:
            _validate.check_copy_pairs(block_pairs, desc.num_blocks)
            _validate.check_prologue_sources(block_pairs, slot_mapping)
        if S:
            _validate.check_lengths(context_lens, max_blocks_per_seq)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _gpu(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    return desc, n, npairs, S, ws_ptr, ws_bytes


def decode_step_prologue(k, v, k_cache, v_cache, slot_mapping, block_pairs, context_lens, num_heads: int,
                         max_blocks_per_seq: int, workspace, *, partition_tokens: int = 0, stream=None):
    """copy_blocks(block_pairs), reshape_and_cache(k, v, slot_mapping) and
    paged_attn_decode_plan(context_lens, ...) into `workspace`, in one launch
    (16-bit caches; see pagedkv.h for the one extra condition)."""
    torch = _torch()
    desc, n, npairs, S, ws_ptr, ws_bytes = _prologue_args(k, v, k_cache, slot_mapping, block_pairs, context_lens,
                                                          max_blocks_per_seq, workspace)
    row_dtype = None if desc.dtype == PKV_FP8_E4M3 else k_cache.dtype  # fp8: the library refuses the cache
    st = lib().decode_step_prologue(_gpu(k, "k", row_dtype), _gpu(v, "v", row_dtype),
                                    _gpu(k_cache, "k_cache"), _gpu(v_cache, "v_cache", k_cache.dtype),
                                    _gpu(slot_mapping, "slot_mapping", torch.int32, 1), n,
                                    _gpu(block_pairs, "block_pairs", torch.int32, 2) if npairs else None, npairs,
                                    _gpu(context_lens, "context_lens", torch.int32, 1), S, int(num_heads),
                                    int(max_blocks_per_seq), ctypes.byref(desc), int(partition_tokens), ws_ptr,
                                    ws_bytes, _stream_handle(stream))
    _check(st, "decode_step_prologue")


def decode_step_prologue_fp8(k, v, k_cache, v_cache, slot_mapping, block_pairs, context_lens, num_heads: int,
                             max_blocks_per_seq: int, workspace, k_scale, v_scale, *, partition_tokens: int = 0,
                             stream=None):
    """decode_step_prologue for an fp8 cache: copy_blocks, reshape_and_cache_fp8
    with the scales (a float, or a GPU float32 tensor [num_kv_heads], each) and
    the plan, in one launch; bit-identical to the three calls."""
    torch = _torch()
    desc, n, npairs, S, ws_ptr, ws_bytes = _prologue_args(k, v, k_cache, slot_mapping, block_pairs, context_lens,
                                                          max_blocks_per_seq, workspace)
    sc = fp8_scales(k.dtype, k_scale, v_scale, desc.num_kv_heads)
    st = lib().decode_step_prologue_fp8(_gpu(k, "k"), _gpu(v, "v", k.dtype), _gpu(k_cache, "k_cache", torch.uint8),
                                        _gpu(v_cache, "v_cache", torch.uint8),
                                        _gpu(slot_mapping, "slot_mapping", torch.int32, 1), n,
                                        _gpu(block_pairs, "block_pairs", torch.int32, 2) if npairs else None, npairs,
                                        _gpu(context_lens, "context_lens", torch.int32, 1), S, int(num_heads),
                                        int(max_blocks_per_seq), ctypes.byref(desc), ctypes.byref(sc),
                                        int(partition_tokens), ws_ptr, ws_bytes, _stream_handle(stream))
    _check(st, "decode_step_prologue_fp8")


def swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs, *, stream=None):
    """Copy block src of (src_k, src_v) to block dst of (dst_k, dst_v) for every
    (src, dst) row of block_pairs; either side may be a pinned host tensor
    (torch pin_memory), which the GPU reaches through its device mapping."""
    torch = _torch()
    dd, sd = _desc_of(dst_k), _desc_of(src_k)
    for t, name, dt in ((dst_k, "dst_k", None), (dst_v, "dst_v", dst_k.dtype), (src_k, "src_k", dst_k.dtype),
                        (src_v, "src_v", dst_k.dtype)):
        if not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a GPU tensor or pinned host memory")
        if not t.is_contiguous() or (dt is not None and t.dtype != dt):
            raise ValueError(f"{name} must be contiguous and of one dtype with dst_k")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2 or block_pairs.dtype != torch.int32:
        raise ValueError("block_pairs must be int32 [num_pairs, 2]")
    if not (block_pairs.is_cuda or block_pairs.is_pinned()) or not block_pairs.is_contiguous():
        raise ValueError("block_pairs must be contiguous, on the GPU or pinned")
    n = int(block_pairs.shape[0])
    if n == 0:
        return
    if _validate.enabled():
        _validate.check_swap_pairs(block_pairs, sd.num_blocks, dd.num_blocks)
    st = lib().swap_blocks(dst_k.data_ptr(), dst_v.data_ptr(), ctypes.byref(dd), src_k.data_ptr(), src_v.data_ptr(),
                           ctypes.byref(sd), block_pairs.data_ptr(), n, _stream_handle(stream))
    _check(st, "swap_blocks")


def gather_cache(k_out, v_out, k_cache, v_cache, block_tables, context_lens, out_offsets, *, stream=None):
    """Paged K/V of every sequence into contiguous [tokens, num_kv_heads, 128]."""
    torch = _torch()
    desc = _desc_of(k_cache)
    num_seqs, mbps = block_tables.shape
    if _validate.enabled():
        _validate.check_tables(block_tables, context_lens, desc.num_blocks)
    st = lib().gather_cache(_gpu(k_out, "k_out", k_cache.dtype), _gpu(v_out, "v_out", k_cache.dtype),
                            _gpu(k_cache, "k_cache"), _gpu(v_cache, "v_cache", k_cache.dtype),
                            _gpu(block_tables, "block_tables", torch.int32, 2),
                            _gpu(context_lens, "context_lens", torch.int32, 1), int(num_seqs), int(mbps),
                            _gpu(out_offsets, "out_offsets", torch.int32, 1), ctypes.byref(desc),
                            _stream_handle(stream))
    _check(st, "gather_cache")


# ---------------------------------------------------------------------------
# host block manager (C++)
# ---------------------------------------------------------------------------

def _i32_array(values) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(values, dtype=np.int32))


def _p(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


class BlockManager:
    """The library's host block manager (pkv_bm_*): free list, refcounts,
    per-sequence block tables, copy-on-write on append."""

    def __init__(self, num_blocks: int, block_size: int = BLOCK_SIZE, free_order=None):
        order = None if free_order is None else _i32_array(free_order)
        if order is not None and order.shape[0] != num_blocks:
            raise ValueError("free_order must have num_blocks entries")
        self._order = order
        h = lib().pkv_bm_create(int(num_blocks), int(block_size), None if order is None else _p(order))
        if not h:
            raise ValueError("pkv_bm_create rejected its arguments")
        self._h = ctypes.c_void_p(h)
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _LIB is not None:
            _LIB.pkv_bm_destroy(h)
            self._h = None

    def add(self, seq: int, num_tokens: int) -> np.ndarray:
        slots = np.empty(max(int(num_tokens), 1), dtype=np.int32)
        _check(lib().pkv_bm_add(self._h, int(seq), int(num_tokens), _p(slots)), "pkv_bm_add")
        return slots[: int(num_tokens)]

    def fork(self, parent: int, child: int) -> None:
        _check(lib().pkv_bm_fork(self._h, int(parent), int(child)), "pkv_bm_fork")

    def append_slot(self, seq: int):
        slot = np.zeros(1, dtype=np.int32)
        pair = np.zeros(2, dtype=np.int32)
        _check(lib().pkv_bm_append_slot(self._h, int(seq), _p(slot), _p(pair)), "pkv_bm_append_slot")
        return int(slot[0]), (None if pair[0] < 0 else (int(pair[0]), int(pair[1])))

    def step(self, seqs: Sequence[int]):
        seqs_a = _i32_array(list(seqs))
        n = int(seqs_a.shape[0])
        slots = np.empty(max(n, 1), dtype=np.int32)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        npairs = np.zeros(1, dtype=np.int32)
        _check(lib().pkv_bm_step(self._h, _p(seqs_a), n, _p(slots), _p(pairs), _p(npairs)), "pkv_bm_step")
        return slots[:n].copy(), pairs[: int(npairs[0])].copy()

    def free_seq(self, seq: int) -> None:
        _check(lib().pkv_bm_free(self._h, int(seq)), "pkv_bm_free")

    def block_table(self, seqs: Sequence[int], max_blocks: int) -> np.ndarray:
        seqs_a = _i32_array(list(seqs))
        n = int(seqs_a.shape[0])
        table = np.empty((max(n, 1), max(int(max_blocks), 1)), dtype=np.int32)
        _check(lib().pkv_bm_block_table(self._h, _p(seqs_a), n, int(max_blocks), _p(table), None),
               "pkv_bm_block_table")
        return table[:n, : int(max_blocks)].copy()

    def context_lens(self, seqs: Sequence[int]) -> np.ndarray:
        return np.asarray([self.length(s) for s in seqs], dtype=np.int32)

    def num_free(self) -> int:
        return int(lib().pkv_bm_num_free(self._h))

    def num_used(self) -> int:
        return self.num_blocks - self.num_free()

    def refcount(self, block: int) -> int:
        return int(lib().pkv_bm_refcount(self._h, int(block)))

    def length(self, seq: int) -> int:
        return int(lib().pkv_bm_length(self._h, int(seq)))

    def num_seq_blocks(self, seq: int) -> int:
        return int(lib().pkv_bm_num_seq_blocks(self._h, int(seq)))

    def waste(self, seq: int) -> int:
        return int(lib().pkv_bm_waste(self._h, int(seq)))

    def free_list(self) -> np.ndarray:
        """The free list, front to back (evictable prefix-cache blocks not included)."""
        n = self.num_free()
        out = np.empty(max(n, 1), dtype=np.int32)
        m = lib().pkv_bm_free_list(self._h, _p(out), n)
        return out[:m].copy()

    # prefix caching
    def add_cached(self, seq: int, token_ids) -> Tuple[np.ndarray, int]:
        """New sequence with these token ids, reusing registered full blocks of
        its prefix: (slots, number of tokens already cached)."""
        ids = _i32_array(token_ids)
        n = int(ids.shape[0])
        slots = np.empty(max(n, 1), dtype=np.int32)
        cached = np.zeros(1, dtype=np.int32)
        _check(lib().pkv_bm_add_cached(self._h, int(seq), n, _p(ids) if n else None, _p(slots), _p(cached)),
               "pkv_bm_add_cached")
        return slots[:n].copy(), int(cached[0])

    def append_token(self, seq: int, token_id: int):
        slot = np.zeros(1, dtype=np.int32)
        pair = np.zeros(2, dtype=np.int32)
        _check(lib().pkv_bm_append_token(self._h, int(seq), int(token_id), _p(slot), _p(pair)),
               "pkv_bm_append_token")
        return int(slot[0]), (None if pair[0] < 0 else (int(pair[0]), int(pair[1])))

    def num_evictable(self) -> int:
        return int(lib().pkv_bm_num_evictable(self._h))


__all__ = [
    "LIB_PATH", "BLOCK_SIZE", "HEAD_SIZE", "PAGE_ELEMS", "CacheDesc", "PagedKVError", "OutOfBlocks",
    "lib", "status_string", "version", "cache_desc", "allocate_cache", "k_index", "v_index",
    "workspace_size", "partition_tokens_for", "paged_attn_decode", "paged_attn_decode_plan",
    "paged_attn_decode_run", "reshape_and_cache", "copy_blocks", "PKV_FP8_E4M3", "Fp8Scales", "fp8_scales",
    "paged_attn_decode_fp8", "paged_attn_decode_run_fp8", "reshape_and_cache_fp8", "paged_attn_prefill",
    "prefill_workspace_size", "swap_blocks", "decode_step_prologue", "decode_step_prologue_fp8",
    "paged_attn_decode_noalloc", "paged_attn_decode_read_pages", "NOALLOC_SCRATCH_BYTES",
    "gather_cache", "BlockManager", "SIGNATURES",
]
