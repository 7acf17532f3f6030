"""HIP-graph capture of the library's calls.

The entry points enqueue kernels only (no allocation, no synchronisation, no
memset), so a sequence of them can be captured once and replayed.  Checked on
the GPU through the C ABI: a captured sequence (a fused fold-and-step, a plain
monolith step, a plain split step with its workspace, a flush) is replayed
three times on one copy of a cache, with the same calls run eagerly on a
second copy between the replays; outputs, caches and status words must match
bit for bit after every replay.  The same holds in a fresh process whose very
first library calls are the ones being captured (the library's per-device
occupancy lookup then runs inside the capture).
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import synth
from synth import device as sd

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_harness as gh
    import speculative_replay_state_amd as ssu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


# (state dtype, num_slots, nheads, ngroups, batch), by the kernel the plain
# monolith step runs in: fp8 persistent (12 x 32 pairs) and one head per wave
# (256 x 128); fp16 two heads per wave (256 x 128); bf16 head rows in 4 parts
# (9 x 16)
SHAPES = {"small": ("fp8", 40, 32, 4, 12), "per_head": ("fp8", 300, 128, 8, 256),
          "f16_pair": ("f16", 300, 128, 8, 256), "bf16_parts": ("bf16", 24, 16, 2, 9)}


@pytest.mark.parametrize("shape", list(SHAPES))
def test_graph_replays_match_eager(shape):
    state_dtype, num_slots, H, G, batch = SHAPES[shape]
    spec = synth.CacheSpec(num_slots=num_slots, nheads=H, ngroups=G, state_dtype=state_dtype)
    cache = synth.make_cache(spec, 7100 + H)
    step = synth.make_step(spec, batch, 4, 7101 + H, 8, n_padding=2)
    rng = np.random.default_rng(7102)
    k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
    k2 = np.minimum(step.pnat, 2).astype(np.int32)
    st = sd.upload_step(step, gh.DEV)
    kt = torch.from_numpy(k).to(gh.DEV)
    k2t = torch.from_numpy(k2).to(gh.DEV)
    print("case graph", shape, "batch", batch, "H", H, flush=True)

    def make(t):
        dc = gh.device_cache(spec, t)
        outs = [gh.out_tensor(step, spec, "bf16") for _ in range(3)]
        ws = torch.empty(max(ssu.workspace_size(dc, step.batch, step.T) // 4, 1), dtype=torch.float32,
                         device=gh.DEV)
        descs = [ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                                    st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16",
                                    w, algo, num_fold=f)
                 for out, w, algo, f in ((outs[0], None, "auto", kt), (outs[1], None, "monolith", None),
                                         (outs[2], ws, "split", None))]
        return dc, outs, descs

    def calls(dc, descs):
        for d in descs:
            ssu.replay_step(dc, d)
        ssu.flush(dc, st["slot_idx"], k2t, st["A"])

    # every path once, eagerly, on a scratch copy (the library caches an
    # occupancy query per kernel on first use)
    dcw, _, descw = make(sd.upload_cache(cache, gh.DEV))
    calls(dcw, descw)
    torch.cuda.synchronize()
    assert int(dcw.status.item()) == 0

    ta, tb = sd.upload_cache(cache, gh.DEV), sd.upload_cache(cache, gh.DEV)
    dca, outa, desca = make(ta)
    dcb, outb, descb = make(tb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(dca, desca)
    for rep in range(3):
        graph.replay()
        calls(dcb, descb)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outa, outb)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "replay %d, output %d" % (rep, i)
        ga, gb = sd.download_cache(spec, ta), sd.download_cache(spec, tb)
        for f in sd.CACHE_FIELDS + ("ring_start",):
            assert np.array_equal(getattr(ga, f), getattr(gb, f)), "replay %d, %s" % (rep, f)
        assert int(dca.status.item()) == 0 and int(dcb.status.item()) == 0


ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def first_calls_in_capture():
    """Run in a fresh process: capture the library's first calls (a plain
    monolith step on the persistent kernel (20 x 32 = 640 pairs), a split
    step, a flush), replay the graph three times and compare with the same
    calls run eagerly on a copy."""
    spec = synth.CacheSpec(num_slots=40, nheads=32, ngroups=4, state_dtype="f16")
    cache = synth.make_cache(spec, 7300)
    step = synth.make_step(spec, 20, 4, 7301, 8, n_padding=2)
    k2 = np.minimum(step.pnat, 2).astype(np.int32)
    st = sd.upload_step(step, gh.DEV)
    k2t = torch.from_numpy(k2).to(gh.DEV)

    def make(t):
        dc = gh.device_cache(spec, t)
        outs = [gh.out_tensor(step, spec, "bf16") for _ in range(2)]
        ws = torch.empty(max(ssu.workspace_size(dc, step.batch, step.T) // 4, 1), dtype=torch.float32,
                         device=gh.DEV)
        descs = [ssu.make_step_desc(step.batch, step.T, st["slot_idx"], st["pnat"], st["cu_seqlens"], st["x"],
                                    st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16",
                                    w, algo)
                 for out, w, algo in ((outs[0], None, "monolith"), (outs[1], ws, "split"))]
        return dc, outs, descs

    def calls(dc, descs):
        for d in descs:
            ssu.replay_step(dc, d)
        ssu.flush(dc, st["slot_idx"], k2t, st["A"])

    ta, tb = sd.upload_cache(cache, gh.DEV), sd.upload_cache(cache, gh.DEV)
    dca, outa, desca = make(ta)
    dcb, outb, descb = make(tb)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls(dca, desca)  # the process's first library calls
    for rep in range(3):
        graph.replay()
        calls(dcb, descb)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outa, outb)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "replay %d, output %d" % (rep, i)
        ga, gb = sd.download_cache(spec, ta), sd.download_cache(spec, tb)
        for f in sd.CACHE_FIELDS + ("ring_start",):
            assert np.array_equal(getattr(ga, f), getattr(gb, f)), "replay %d, %s" % (rep, f)
        assert int(dca.status.item()) == 0 and int(dcb.status.item()) == 0
    print("FIRST_CALLS_IN_CAPTURE_OK", flush=True)


def test_first_library_calls_inside_capture():
    print("case graph: first calls inside capture (fresh process)", flush=True)
    p = subprocess.run([sys.executable, "-c", "import tests.test_gpu_graph as t; t.first_calls_in_capture()"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert p.returncode == 0 and "FIRST_CALLS_IN_CAPTURE_OK" in p.stdout, (p.returncode, p.stdout[-2000:],
                                                                          p.stderr[-2000:])
