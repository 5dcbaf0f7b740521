"""The BF16 kernel's dynamic tile schedule: a container with more than three
steps of tiles is decoded with tiles handed out by device counters.  Each
dispatch claims a counter slot on the device (keyed by its own dispatch
packet), starting at a slot the host hints, and frees it clean when its last
grab is served.  These tests decode such containers bit-exactly past a full
cycle of hints, on two streams at once, from a replayed HIP graph, and from
several instances of one captured graph (one frozen hint) launched on
several streams at once.  Every call goes through the C ABI."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import synth

pytestmark = pytest.mark.gpu

# counter slots; launches take them as hints in turn
SLOTS = 4096


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


@pytest.fixture(scope="module")
def block(torch_dev):
    """64M BF16 weights (about 10,400 tiles, more than three steps of the
    2,048 tile groups of a full grid) on the device, with the reference."""
    torch, dev = torch_dev
    src = synth.bf16_rne(np.random.default_rng(77).normal(0, 0.02, 64 << 20).astype(np.float32))
    c = dfh.compress(dfh.KIND_BF16, src)
    assert c.info()["n_tiles"] > 3 * 2048
    dc = dfh.to_device(c, dev)
    ref = torch.from_numpy(src.view(np.int16)).to(dev)
    return dc, ref


def test_decodes_past_a_cycle_of_counter_slots(torch_dev, block):
    # every launch is hinted the next slot; past SLOTS launches the hints
    # come round again, so each slot must have been freed clean
    torch, dev = torch_dev
    dc, ref = block
    outs = [dc.empty_output() for _ in range(2)]
    bad = torch.zeros(1, dtype=torch.int64, device=dev)
    n = SLOTS + 200
    say("dynamic schedule:", n, "launches")
    for k in range(n):
        o = outs[k % 2]
        o.view(torch.int16).fill_(0)
        dfh.df_decompress(dc, o)
        bad += (o.view(torch.int16) != ref).any().to(torch.int64)
        if k % 1000 == 999:
            say("  launches", k + 1)
    torch.cuda.synchronize()
    assert int(bad.item()) == 0


def test_two_streams_at_once(torch_dev, block):
    torch, dev = torch_dev
    dc, ref = block
    side = torch.cuda.Stream(device=dev)  # default priority
    main = torch.cuda.current_stream(dev)
    a, b = dc.empty_output(), dc.empty_output()
    for k in range(40):
        a.view(torch.int16).fill_(0)
        b.view(torch.int16).fill_(0)
        side.wait_stream(main)
        dfh.df_decompress(dc, a, main)
        dfh.df_decompress(dc, b, side)
        main.wait_stream(side)
        assert torch.equal(a.view(torch.int16), ref), k
        assert torch.equal(b.view(torch.int16), ref), k


def test_graph_replays(torch_dev, block):
    # a captured launch keeps its hint; every replay claims a slot and must
    # free it clean
    torch, dev = torch_dev
    dc, ref = block
    out = dc.empty_output()
    eager = dc.empty_output()
    dfh.df_decompress(dc, eager)
    torch.cuda.synchronize()
    assert torch.equal(eager.view(torch.int16), ref)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(s):
        dfh.df_decompress(dc, out, s)  # warm-up outside the capture
    torch.cuda.current_stream(dev).wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        dfh.df_decompress(dc, out)
    for r in range(6):
        out.view(torch.int16).fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), r
        dfh.df_decompress(dc, eager)  # eager work between replays
        torch.cuda.synchronize()


def test_batched_jobs_each_with_a_slot(torch_dev):
    # a batched launch splits the grid between its jobs; sixteen containers
    # of 2.9M-4.4M weights (about 450-700 tiles, each job some 32
    # workgroups) are each dealt by their own counters, four parts per job
    # and uneven workgroup counts per part
    torch, dev = torch_dev
    rng = np.random.default_rng(5)
    sizes = [2_900_000 + 100_003 * k for k in range(16)]
    srcs = [synth.bf16_rne(rng.normal(0, 0.02, n).astype(np.float32)) for n in sizes]
    cs = [dfh.compress(dfh.KIND_BF16, s) for s in srcs]
    assert min(c.info()["n_tiles"] for c in cs) > 3 * 32 * 4
    dcs = [dfh.to_device(c, dev) for c in cs]
    outs = [dc.empty_output() for dc in dcs]
    refs = [torch.from_numpy(s.view(np.int16)).to(dev) for s in srcs]
    for rep in range(3):
        for o in outs:
            o.view(torch.int16).fill_(0)
        dfh.df_decompress_batch(dcs, outs)
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs, refs)):
            assert torch.equal(o.view(torch.int16), r), (rep, k)


def test_batched_large_jobs(torch_dev, block):
    # three large jobs in one launch (about 170 workgroups each)
    torch, dev = torch_dev
    dc, ref = block
    outs = [dc.empty_output() for _ in range(3)]
    for rep in range(3):
        for o in outs:
            o.view(torch.int16).fill_(0)
        dfh.df_decompress_batch([dc, dc, dc], outs)
        torch.cuda.synchronize()
        for k, o in enumerate(outs):
            assert torch.equal(o.view(torch.int16), ref), (rep, k)


class _HipGraphs:
    """Stream capture and graph instances through the HIP runtime that torch
    has loaded (torch's CUDAGraph instantiates a capture only once)."""

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.L = ctypes.CDLL("libamdhip64.so")
        P = ctypes.c_void_p
        for name, args in (("hipStreamBeginCapture", [P, ctypes.c_int]),
                           ("hipStreamEndCapture", [P, ctypes.POINTER(P)]),
                           ("hipGraphInstantiate", [ctypes.POINTER(P), P, P, P, ctypes.c_size_t]),
                           ("hipGraphLaunch", [P, P]), ("hipGraphExecDestroy", [P]),
                           ("hipGraphDestroy", [P])):
            getattr(self.L, name).argtypes = args
            getattr(self.L, name).restype = ctypes.c_int

    def capture(self, stream, fn):
        ct = self.ct
        assert self.L.hipStreamBeginCapture(ct.c_void_p(stream.cuda_stream), 2) == 0   # relaxed mode
        fn()
        g = ct.c_void_p()
        assert self.L.hipStreamEndCapture(ct.c_void_p(stream.cuda_stream), ct.byref(g)) == 0
        return g

    def instantiate(self, g):
        e = self.ct.c_void_p()
        assert self.L.hipGraphInstantiate(self.ct.byref(e), g, None, None, 0) == 0
        return e

    def launch(self, e, stream):
        assert self.L.hipGraphLaunch(e, self.ct.c_void_p(stream.cuda_stream)) == 0


def test_instances_of_one_graph_on_several_streams(torch_dev, block):
    # one captured decode (one frozen hint, one destination) instantiated
    # three times, the instances launched on three streams at once: each
    # dispatch must claim its own slot (two find the hinted one taken) and
    # free it clean.  Afterwards each instance replayed alone into a cleared
    # destination, and eager decodes, must be exact: a slot left dirty would
    # make them skip tiles.
    torch, dev = torch_dev
    dc, ref = block
    hg = _HipGraphs()
    out = dc.empty_output()
    eager = dc.empty_output()
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    g = hg.capture(cap, lambda: dfh.df_decompress(dc, out, cap))
    execs = [hg.instantiate(g) for _ in range(3)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(3)]
    try:
        for rnd in range(8):
            out.view(torch.int16).fill_(0)
            torch.cuda.synchronize()
            for e, st in zip(execs, streams):
                hg.launch(e, st)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), ref), rnd
            for k, (e, st) in enumerate(zip(execs, streams)):
                out.view(torch.int16).fill_(0)
                torch.cuda.synchronize()
                hg.launch(e, st)
                torch.cuda.synchronize()
                assert torch.equal(out.view(torch.int16), ref), (rnd, k)
            eager.view(torch.int16).fill_(0)
            dfh.df_decompress(dc, eager)
            torch.cuda.synchronize()
            assert torch.equal(eager.view(torch.int16), ref), rnd
        say("graph instances: 8 rounds of 3 concurrent launches exact")
    finally:
        torch.cuda.synchronize()
        for e in execs:
            hg.L.hipGraphExecDestroy(e)
        hg.L.hipGraphDestroy(g)


def test_graph_instances_next_to_eager_launches(torch_dev, block):
    # two instances of one graph on two streams while eager decodes of the
    # same container run on a third, into separate buffers, several rounds
    torch, dev = torch_dev
    dc, ref = block
    hg = _HipGraphs()
    gout = dc.empty_output()
    eouts = [dc.empty_output() for _ in range(3)]
    cap = torch.cuda.Stream(device=dev)
    cap.wait_stream(torch.cuda.current_stream(dev))
    torch.cuda.synchronize()
    g = hg.capture(cap, lambda: dfh.df_decompress(dc, gout, cap))
    execs = [hg.instantiate(g) for _ in range(2)]
    streams = [torch.cuda.Stream(device=dev) for _ in range(3)]
    try:
        for rnd in range(6):
            gout.view(torch.int16).fill_(0)
            for o in eouts:
                o.view(torch.int16).fill_(0)
            torch.cuda.synchronize()
            hg.launch(execs[0], streams[0])
            for o in eouts:
                dfh.df_decompress(dc, o, streams[2])
            hg.launch(execs[1], streams[1])
            torch.cuda.synchronize()
            assert torch.equal(gout.view(torch.int16), ref), rnd
            for k, o in enumerate(eouts):
                assert torch.equal(o.view(torch.int16), ref), (rnd, k)
    finally:
        torch.cuda.synchronize()
        for e in execs:
            hg.L.hipGraphExecDestroy(e)
        hg.L.hipGraphDestroy(g)


@pytest.mark.parametrize("cap", [1, 2, 7, 8, 33, 64, 300])
def test_workgroup_cap(torch_dev, block, cap):
    # a capped launch: few workgroups walk many steps (dynamically dealt
    # units from step 3 on; one counter below eight workgroups)
    torch, dev = torch_dev
    dc, ref = block
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for checked in (False, True):
        out.view(torch.int16).fill_(0)
        if checked:
            dfh.df_decompress_checked(dc, out, err, max_workgroups=cap)
        else:
            dfh.df_decompress(dc, out, max_workgroups=cap)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert torch.equal(out.view(torch.int16), ref), (cap, checked)
