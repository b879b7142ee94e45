"""The decode step and chunked prefill replayed from a captured HIP graph.
Marked gpu.

Every call of the library is asynchronous on the caller's stream, allocates
nothing and never synchronises, so a serving loop can capture a whole step
(copy_blocks, reshape_and_cache, paged_attn_decode_plan, paged_attn_decode_run)
once and replay it without host launch work (the step's copy, write and plan
also as one decode_step_prologue[_fp8] launch).  Each replay must give the bits
of the eager step: the graph is replayed several times, with eager work of the
program and synchronisations between replays, and every replay's output is
compared with the eager result after the output buffer was overwritten.
"""

import numpy as np
import pytest

import harness
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import paged_kv_cache_345_amd as pkv  # noqa: E402

REPLAYS = 4


def _bits(t):
    return t.view(torch.int16).clone()


def _decode_cases():
    return {
        "tiny": (lambda: synth.make_workload("tiny"), None),
        "gqa-split-groups": (lambda: synth.make_random_workload(71, num_seqs=9, num_heads=16, num_kv_heads=2,
                                                                 dtype="bf16", max_len=700, groups=2), 128),
        "mha-fp8-groups": (lambda: synth.make_random_workload(72, num_seqs=7, num_heads=4, num_kv_heads=4,
                                                               dtype="fp16", max_len=300, groups=1,
                                                               kv_dtype="fp8e4m3", k_scale=0.0125,
                                                               v_scale=0.0125), None),
    }


def _prologue(step, fused):
    if fused:  # copy, write and plan in one launch
        step.prologue()
    else:
        step.copy()
        step.write()
        step.plan()


@pytest.mark.parametrize("fused", [False, True], ids=["three-calls", "fused-prologue"])
@pytest.mark.parametrize("name", sorted(_decode_cases()))
def test_decode_step_graph_replays_match_eager(name, fused, monkeypatch):
    monkeypatch.delenv("PKV_VALIDATE", raising=False)  # host checks copy to the host: not capturable
    make, pt = _decode_cases()[name]
    wl = make()
    step = harness.build_step(wl, partition_tokens=pt, run=False)
    # eager step
    _prologue(step, fused)
    eager = _bits(step.run())
    torch.cuda.synchronize()

    out_g = torch.empty_like(step.out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _prologue(step, fused)
        step.run(out=out_g)
    torch.cuda.synchronize()

    scratch = torch.empty_like(step.out)
    for r in range(REPLAYS):
        out_g.view(torch.int16).fill_(-1 - r)  # NaN bits: a replay that skipped the write would show
        torch.cuda.synchronize()
        graph.replay()
        step.run(out=scratch)  # eager work of the program between replays
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), eager), f"replay {r}"
        assert torch.equal(scratch.view(torch.int16), eager), f"eager run after replay {r}"


def test_prefill_graph_replays_match_eager(monkeypatch):
    monkeypatch.delenv("PKV_VALIDATE", raising=False)
    wl = synth.make_prefill_workload(8700, num_seqs=5, num_heads=8, num_kv_heads=2, dtype="bf16",
                                     context=(20, 400), chunk=(1, 120))
    pre = harness.build_prefill(wl, partition_tokens=64)  # several segments: the merge kernel runs too
    torch.cuda.synchronize()
    eager = _bits(pre.out)

    out_g = torch.empty_like(pre.out)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        pre.run(out=out_g)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        out_g.view(torch.int16).fill_(-1 - r)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), eager), f"replay {r}"
    assert np.isfinite(out_g.float().cpu().numpy()).all()
