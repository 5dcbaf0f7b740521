"""The BF16 kernel's dynamic tile schedule: a container with more than three
steps of tiles is decoded with tiles handed out by device counters, which
each launch leaves at zero for the next launch that uses the same slot.
These tests decode such containers bit-exactly past a full cycle of counter
slots, on two streams at once, and from a replayed HIP graph.  Every call
goes through the C ABI."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import synth

pytestmark = pytest.mark.gpu

# slots launches cycle through outside stream capture (4096 - 512)
EAGER_SLOTS = 3584


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
    # every launch takes the next slot; past EAGER_SLOTS launches the slots
    # come round again, so each must have been left at zero
    torch, dev = torch_dev
    dc, ref = block
    outs = [dc.empty_output() for _ in range(2)]
    bad = torch.zeros(1, dtype=torch.int64, device=dev)
    n = EAGER_SLOTS + 200
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
    # a captured launch keeps its slot; every replay must leave it at zero
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
