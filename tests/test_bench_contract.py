"""bench.py's contract, on the CPU: the algorithmic byte and flop counts its
figures divide by, the refusal of more than one GPU, and the rule that a
committed HBM-traffic summary is used only while the kernel sources it was
taken on are unchanged."""

import os
import subprocess
import sys
import types

import numpy as np
import pytest

import bench
import synth
from oracle.block_manager import BlockManager

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _host_step(wl):
    """The block tables, copy pairs and slots of the workload's decode step,
    from the oracle's block manager (no cache contents)."""
    bm = BlockManager(wl.pool_blocks, 16, wl.free_order)
    slots = pairs = None
    for op in wl.ops:
        if op[0] == "add":
            bm.add(op[1], op[2])
        elif op[0] == "fork":
            bm.fork(op[1], op[2])
        elif op[0] == "step":
            slots, pairs = bm.step(op[1])
    S = wl.num_seqs
    maxb = max(len(bm.blocks[s]) for s in range(S))
    return types.SimpleNamespace(block_tables_host=np.asarray(bm.block_table(range(S), maxb)),
                                 block_pairs_host=np.asarray(pairs, dtype=np.int64).reshape(-1, 2),
                                 slot_mapping_host=np.asarray(slots))


def _unique_live_slots(wl, step):
    """Live (block, slot) pairs counted per physical block: a sequence uses a
    prefix of each of its blocks, so a block shared by several sequences
    holds max over them of their prefix lengths live slots."""
    live = {}
    for s in range(wl.num_seqs):
        L = int(wl.context_lens[s])
        for j in range(-(-L // 16)):
            b = int(step.block_tables_host[s, j])
            live[b] = max(live.get(b, 0), min(16, L - 16 * j))
    return sum(live.values())


@pytest.mark.parametrize("name", ["tiny", "llama13b"])
def test_decode_bytes(name):
    wl = synth.make_workload(name)
    step = _host_step(wl)
    nb = bench.step_bytes(wl, step)
    per_slot = 2 * wl.num_kv_heads * 128 * 2
    assert nb["kv_unique"] == _unique_live_slots(wl, step) * per_slot
    assert nb["kv_per_sequence"] == int(wl.context_lens.sum()) * per_slot
    nblk = sum(-(-int(L) // 16) for L in wl.context_lens)
    assert nb["decode"] == nb["kv_unique"] + 2 * wl.num_seqs * wl.num_heads * 128 * 2 + 4 * nblk + 4 * wl.num_seqs
    if name == "tiny":  # no parallel samples: every slot is one sequence's own
        assert nb["kv_unique"] == nb["kv_per_sequence"] and nb["copy"] == 0
    else:  # the LLaMA-13B-shaped batch: 13 groups of 3 samples, 22 copy-on-write pairs
        assert step.block_pairs_host.shape == (22, 2)
        assert nb["kv_unique"] < nb["kv_per_sequence"]
        assert nb["decode"] == 1_636_970_892


def test_prefill_flops_by_brute_force():
    rng = np.random.default_rng(5)
    L = rng.integers(1, 300, 9)
    C = np.minimum(rng.integers(0, 80, 9), L)
    brute = sum(L[s] - C[s] + j + 1 for s in range(9) for j in range(C[s]))  # keys seen by each chunk query
    assert bench.prefill_flops(L, C, 3) == int(brute) * 4 * 128 * 3
    assert bench.prefill_flops([5], [0], 8) == 0
    assert bench.prefill_flops([1], [1], 1) == 4 * 128  # position 0 sees itself


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_summaries_follow_their_sources(tmp_path):
    stems = [f[:-len("_hbm_traffic.md")] for f in os.listdir(os.path.join(ROOT, "profiles"))
             if f.endswith("_hbm_traffic.md")]
    assert stems
    for stem in stems:
        sources = bench.PREFILL_SOURCES if stem.startswith("prefill_") else bench.DECODE_SOURCES
        got = bench.measured_traffic(stem, sources)
        assert got is None or got > 0
        # taken on other sources: never used
        assert bench.measured_traffic(stem, ("bench.py",)) is None
    assert bench.measured_traffic("no_such_workload") is None
