"""Calls on several streams at once.

The entry points keep no state between calls beyond a per-device occupancy
lookup, and every launch goes on the stream it is given, so calls on two
streams that touch different caches may run concurrently.  Checked on the GPU
through the C ABI: three caches of different shapes and state types, whose
plain steps take three kernels (fp16, 256 x 128 pairs: two heads per wave;
bf16, 30 x 32: the persistent kernel; fp8, 12 x 32: one head per wave), each
driven on a stream of its own by the same sequence (a fused fold-and-step, a
plain monolith step, a split step with its workspace, a flush), the sequences
issued interleaved, three rounds.  The same sequences run one after the other
on the current stream give the reference: outputs, caches and status words
must match bit for bit.  Another run puts every sequence on one side stream,
in issue order.
"""
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


# (state dtype, num_slots, nheads, ngroups, batch)
CACHES = (("f16", 300, 128, 8, 256), ("bf16", 64, 32, 4, 30), ("fp8", 40, 32, 4, 12))
ROUNDS = 3


class Driver:
    """One cache (on the device) and its per-round calls."""

    def __init__(self, cfg, seed):
        state_dtype, num_slots, H, G, batch = cfg
        self.spec = spec = synth.CacheSpec(num_slots=num_slots, nheads=H, ngroups=G, state_dtype=state_dtype)
        self.cache = synth.make_cache(spec, seed)
        self.steps = []
        rng = np.random.default_rng(seed + 1)
        for r in range(ROUNDS):
            # pnat <= 4 leaves room for the three steps' appends before the flush
            step = synth.make_step(spec, batch, 4, seed + 10 + r, 4, n_padding=2)
            k = np.array([rng.integers(0, int(p) + 1) for p in step.pnat], np.int32)
            self.steps.append((step, k))

    def upload(self):
        t = sd.upload_cache(self.cache, gh.DEV)
        dc = gh.device_cache(self.spec, t)
        rounds = []
        for step, k in self.steps:
            st = sd.upload_step(step, gh.DEV)
            kt = torch.from_numpy(k).to(gh.DEV)
            # every step accepts all its tokens: the fused step leaves
            # pnat - k + T live ring tokens, each plain step adds T, and the
            # flush then folds 2 of them
            p1 = torch.from_numpy((step.pnat - k + step.T).astype(np.int32)).to(gh.DEV)
            p2 = p1 + step.T
            fk = torch.full((step.batch,), 2, dtype=torch.int32, device=gh.DEV)
            outs = [gh.out_tensor(step, self.spec, "bf16") for _ in range(3)]
            ws = torch.empty(max(ssu.workspace_size(dc, step.batch, step.T) // 4, 1), dtype=torch.float32,
                             device=gh.DEV)
            descs = [ssu.make_step_desc(step.batch, step.T, st["slot_idx"], pnat, st["cu_seqlens"], st["x"],
                                        st["B"], st["C"], st["dt"], st["A"], st["D"], st["dt_bias"], out, "bf16",
                                        w, algo, num_fold=f)
                     for out, pnat, w, algo, f in ((outs[0], st["pnat"], None, "auto", kt),
                                                   (outs[1], p1, None, "monolith", None),
                                                   (outs[2], p2, ws, "split", None))]
            rounds.append((st, descs, fk, outs, (p1, p2)))
        return t, dc, rounds

    def issue(self, dc, rnd, stream):
        st, descs, fk, _, _ = rnd
        for d in descs:
            ssu.replay_step(dc, d, stream=stream)
        ssu.flush(dc, st["slot_idx"], fk, st["A"], stream=stream)


def test_streams_match_one_stream():
    drivers = [Driver(cfg, 7400 + 100 * i) for i, cfg in enumerate(CACHES)]
    for d in drivers:
        assert all(int(s.pnat.max()) + 3 * s.T <= d.spec.ring_len for s, _ in d.steps)  # no BAD_PNAT
    print("case streams: caches", [c[:2] for c in CACHES], flush=True)

    # reference: every call on the current stream, one cache after the other
    ref = [d.upload() for d in drivers]
    cur = torch.cuda.current_stream()
    for d, (t, dc, rounds) in zip(drivers, ref):
        for rnd in rounds:
            d.issue(dc, rnd, cur)
    torch.cuda.synchronize()

    def check(runs, what):
        for d, (ta, dca, ra), (tb, dcb, rb) in zip(drivers, ref, runs):
            assert int(dca.status.item()) == 0 and int(dcb.status.item()) == 0, what
            for r, (x, y) in enumerate(zip(ra, rb)):
                for i, (a, b) in enumerate(zip(x[3], y[3])):
                    assert torch.equal(a.view(torch.int16), b.view(torch.int16)), \
                        "%s: %s round %d output %d" % (what, d.spec.state_dtype, r, i)
            ga, gb = sd.download_cache(d.spec, ta), sd.download_cache(d.spec, tb)
            for f in sd.CACHE_FIELDS + ("ring_start",):
                assert np.array_equal(getattr(ga, f), getattr(gb, f)), "%s: %s %s" % (what, d.spec.state_dtype, f)

    # a side stream per cache (default priority), issued interleaved
    runs = [d.upload() for d in drivers]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in drivers]
    for r in range(ROUNDS):
        for d, (t, dc, rounds), s in zip(drivers, runs, streams):
            d.issue(dc, rounds[r], s)
    for s in streams:
        cur.wait_stream(s)
    torch.cuda.synchronize()
    check(runs, "a stream per cache")

    # one side stream, both caches in issue order
    runs = [d.upload() for d in drivers]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for r in range(ROUNDS):
        for d, (t, dc, rounds) in zip(drivers, runs):
            d.issue(dc, rounds[r], side)
    cur.wait_stream(side)
    torch.cuda.synchronize()
    check(runs, "one side stream")
