"""Helpers of the full-size parity tests (test code; not collected).

At the batches' real sizes the oracle is run on every (sequence, head) row, one
sequence per task on a host thread pool.  NumPy releases the interpreter lock
inside its array work; BLAS is held to one thread per task so the pool does not
oversubscribe the cores.
"""

from __future__ import annotations

import numpy as np

import oracle
import synth
from oracle import fp8 as ofp8


def host_map(fn, items):
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"):
        return synth.thread_map(fn, items)


def seq_rows_f64(wl, s):
    """The float64 K/V rows sequence s attends to, in logical order: the
    generator's contiguous 16-bit rows, or their dequantised E4M3 codes for an
    fp8 cache (the oracle's encoder and decoder)."""
    k, v = wl.seq_kv(s)
    if wl.kv_dtype == "fp8e4m3":
        kf = ofp8.dequantize_ref(ofp8.quantize_ref(k, wl.dtype, wl.k_scale), wl.k_scale)
        vf = ofp8.dequantize_ref(ofp8.quantize_ref(v, wl.dtype, wl.v_scale), wl.v_scale)
        return kf, vf
    return oracle.to_f64(k, wl.dtype), oracle.to_f64(v, wl.dtype)


def decode_errors(wl, got):
    """Max-abs error of every sequence's output rows [Hq, D] (float64 got
    [S, Hq, D]) against the oracle's decode attention."""
    def one(s):
        kf, vf = seq_rows_f64(wl, s)
        ref = oracle.attention_ref(oracle.to_f64(wl.q[s], wl.dtype), kf, vf, wl.scale)
        return float(np.abs(got[s] - ref).max())

    return np.array(host_map(one, range(wl.num_seqs)))


def prefill_errors(wl, got):
    """Max-abs error of every sequence's chunk rows against the oracle's
    causal chunk attention (float64 got [Tq, Hq, D])."""
    from oracle import prefill as opre

    qs = wl.query_start

    def one(s):
        L, C = int(wl.context_lens[s]), int(wl.chunk_lens[s])
        if C == 0:
            return 0.0
        kf, vf = seq_rows_f64(wl, s)
        q = oracle.to_f64(wl.q[qs[s]:qs[s] + C], wl.dtype)
        ref = opre.causal_chunk_ref(q, kf, vf, wl.scale, L - C)
        return float(np.abs(got[qs[s]:qs[s] + C] - ref).max())

    return np.array(host_map(one, range(wl.num_seqs)))


def report(name, errs, tol, what):
    worst = float(errs.max())
    print(f"\n[parity] {name}: {what}: max-abs {worst:.3e} (sequence {int(errs.argmax())}), "
          f"tolerance {tol:g}", flush=True)
    return worst
