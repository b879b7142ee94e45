"""The library's host block manager (csrc/block_manager.cpp) built on its own
with the address and undefined-behaviour sanitizers, driven through the C ABI
by a command-line driver (tests/bm_driver.cpp), against the oracle's block
manager (host only; no GPU).

The mechanism is that of page "vLLM 部署与 PagedAttention 原理 · 检索整理", item 2
(blocks taken on demand, per-sequence block tables, reference counts and
copy-on-write for parallel samples) and, for prefix caching, page "vLLM 深度
解析：以 PagedAttention 与内核生态构建高吞吐 LLM 推理引擎", §2.2.  The transcript of
every call (slots, copy pairs, cached counts, errors) and a state dump after
every call (free list, evictable count, every refcount, every live sequence's
length, waste and block table) must be identical, and the sanitized build must
report no error and no leak.
"""

import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BS = 16
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path_factory.mktemp("bm_san") / "bm_driver")
    cmd = [gxx, "-std=c++20", "-O1", "-g", *SAN, f"-I{ROOT}/include",
           os.path.join(ROOT, "tests", "bm_driver.cpp"),
           os.path.join(ROOT, "paged_kv_cache_345_amd", "csrc", "block_manager.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return exe


def _run(exe, lines):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, env=env,
                       timeout=600)
    assert r.returncode == 0 and "runtime error" not in r.stderr and "ERROR" not in r.stderr, r.stderr[-4000:]
    return r.stdout.splitlines()


class Transcript:
    """Feeds calls to the oracle's manager and records the commands for the
    driver next to the answers the oracle gives."""

    def __init__(self, nb, order):
        self.ref = oracle.BlockManager(nb, BS, order)
        self.cmds = [f"create {nb} {BS} " + " ".join(str(int(b)) for b in order)]
        self.want = ["ok"]

    def _call(self, cmd, fn, fmt):
        self.cmds.append(cmd)
        try:
            r = fn()
        except oracle.OutOfBlocks:
            self.want.append("err 4")
            return None
        except (ValueError, KeyError):
            self.want.append("err 1")
            return None
        self.want.append(fmt(r))
        return r

    def add(self, seq, n):
        return self._call(f"add {seq} {n}", lambda: self.ref.add(seq, n),
                          lambda r: " ".join(["ok"] + [str(s) for s in r]))

    def add_cached(self, seq, ids):
        return self._call(f"addc {seq} {len(ids)} " + " ".join(map(str, ids)),
                          lambda: self.ref.add_cached(seq, ids),
                          lambda r: " ".join(["ok", str(r[1])] + [str(s) for s in r[0]]))

    def fork(self, p, c):
        return self._call(f"fork {p} {c}", lambda: self.ref.fork(p, c) or True, lambda r: "ok")

    @staticmethod
    def _slot_pair(r):
        slot, pair = r
        a, b = pair if pair is not None else (-1, -1)
        return f"ok {slot} {a} {b}"

    def append(self, seq):
        return self._call(f"app {seq}", lambda: self.ref.append_slot(seq), self._slot_pair)

    def token(self, seq, tid):
        return self._call(f"tok {seq} {tid}", lambda: self.ref.append_token(seq, tid), self._slot_pair)

    def step(self, seqs):
        def fmt(r):
            slots, pairs = r
            return " ".join(["ok"] + [str(int(s)) for s in slots] + [";"] + [str(int(x)) for x in pairs.ravel()])
        return self._call(f"step {len(seqs)} " + " ".join(map(str, seqs)), lambda: self.ref.step(seqs), fmt)

    def free(self, seq):
        return self._call(f"free {seq}", lambda: self.ref.free_seq(seq) or True, lambda r: "ok")

    def state(self, seqs):
        ref = self.ref
        parts = [f"free {ref.num_free()} evict {ref.num_evictable()} list"] + [str(b) for b in ref.free]
        parts += [";", "ref"] + [str(r) for r in ref.ref]
        for s in seqs:
            blk = ref.blocks[s]
            parts += [";", str(ref.length[s]), str(ref.waste(s)), str(len(blk))] + [str(b) for b in blk]
        self.cmds.append(f"state {len(seqs)} " + " ".join(map(str, seqs)))
        self.want.append(" ".join(parts))


def _check(driver, tr):
    got = _run(driver, tr.cmds)
    assert len(got) == len(tr.want)
    for i, (g, w) in enumerate(zip(got, tr.want)):
        assert g == w, (i, tr.cmds[i][:200], g[:300], w[:300])


@pytest.mark.parametrize("seed", range(6))
def test_random_streams_with_prefix_cache(driver, seed):
    """Random streams of plain and cached prompts, forks, frees, steps, tokens
    with and without ids, plus calls the manager must refuse (duplicate and
    unknown ids), with a state dump after every call."""
    rng = np.random.default_rng(900 + seed)
    nb = int(rng.integers(6, 60))
    tr = Transcript(nb, rng.permutation(nb))
    bases = [rng.integers(0, 3, 90).tolist() for _ in range(3)]
    live, nxt = [], 0
    for _ in range(400):
        op = int(rng.integers(0, 12))
        if op <= 1 or not live:
            n = int(rng.integers(0, 70))
            base = bases[int(rng.integers(0, 3))]
            k = int(rng.integers(0, min(n, len(base)) + 1))
            ids = base[:k] + rng.integers(0, 4, n - k).tolist()
            ok = tr.add(nxt, n) if op == 1 and rng.random() < 0.3 else tr.add_cached(nxt, ids)
            if ok is not None:
                live.append(nxt)
                nxt += 1
        elif op == 2:
            tr.fork(int(rng.choice(live)), nxt)
            live.append(nxt)
            nxt += 1
        elif op == 3 and len(live) > 1:
            s = int(rng.choice(live))
            tr.free(s)
            live.remove(s)
        elif op == 9:
            tr.step([int(x) for x in rng.choice(live, size=min(len(live), 3), replace=False)])
        elif op == 10:  # refused calls: an existing id, an unknown sequence
            tr.add(int(rng.choice(live)), 3)
            tr.free(nxt + 1000)
            tr.fork(nxt + 1000, nxt + 1001)
        elif op == 8:
            tr.append(int(rng.choice(live)))
        else:
            tr.token(int(rng.choice(live)), int(rng.integers(0, 3)))
        tr.state(live)
    _check(driver, tr)


@pytest.mark.parametrize("name", ["tiny", "llama7b", "llama13b"])
def test_batch_op_streams(driver, name):
    """The block-manager calls that build each decode batch (prompts, parallel
    samples forked from their group's prompt, the decode step with its
    copy-on-write pairs), then every sequence freed."""
    wl = synth.make_workload(name, with_q=False)
    tr = Transcript(wl.pool_blocks, wl.free_order)
    for op in wl.ops:
        if op[0] == "add":
            tr.add(op[1], op[2])
        elif op[0] == "fork":
            tr.fork(op[1], op[2])
        else:
            tr.step(list(op[1]))
    S = wl.num_seqs
    tr.state(list(range(S)))
    for s in range(S):
        tr.free(s)
    tr.state([])
    _check(driver, tr)
