"""Full-size GPU parity for the two largest workloads, in the launch
configuration the benchmark times: the whole 32-block Llama-3-8B-shaped
weight set (one container per block, decoded in sequence into one reused
scratch buffer) and one Llama-3.1-405B-shaped block with Student-t(3)
weights (3,187,671,040 weights, codes up to the 32-bit limit, 64-bit stream
offsets).  Every output is compared bit for bit with its input on the
device; sampled tile ranges are compared with the CPU oracle's own decode
of the same container."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def oracle_view(c):
    inf = c.info()
    d = {k: np.asarray(c.section(k)) for k in ("bitstream", "gaps", "tile_out", "sign_mantissa")}
    d.update(kind=inf["kind"], n=inf["n"], n_tiles=inf["n_tiles"], n_threads=inf["n_threads"],
             lengths=inf["lengths"])
    return d


def check_sampled_ranges(torch, orc, c, out, ranges):
    d = oracle_view(c)
    to = d["tile_out"]
    for b0, b1 in ranges:
        lo, hi = int(to[b0]), int(to[b1])
        ref = orc.decode_tile_range(d, b0, b1)
        got = out[lo:hi].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, ref), (b0, b1)


@pytest.mark.parametrize("seed", [0, 1])
def test_llama3_8b_32_blocks(torch_dev, orc, seed):
    torch, dev = torch_dev
    scratch = None
    for j in range(32):
        src, _ = synth.bf16_block(seed, config=synth.CONFIG_8B_FULL, block=j)
        c = dfh.compress(0, src)
        dc = dfh.to_device(c, dev)
        if scratch is None:
            scratch = dc.empty_output()
        dfh.df_decompress(dc, scratch)
        ref = torch.from_numpy(src.view(np.int16)).to(dev)
        assert torch.equal(scratch.view(torch.int16), ref), j
        if j in (0, 31):
            nt = int(c.info()["n_tiles"])
            check_sampled_ranges(torch, orc, c, scratch, [(0, 8), (nt // 2, nt // 2 + 8), (nt - 8, nt)])
        say("block", j, "seed", seed, "ok")
        del dc, ref


@pytest.mark.parametrize("seed", [0, 1])
def test_llama31_405b_block_t3(torch_dev, orc, seed):
    torch, dev = torch_dev
    say("405B block: generate, seed", seed)
    src, _ = synth.bf16_block(seed, config=synth.CONFIG_405B, shapes=synth.LLAMA31_405B_BLOCK, dist="t3")
    assert src.size == 3_187_671_040
    say("405B block: compress")
    c = dfh.compress(0, src)
    inf = c.info()
    say("405B block:", {k: inf[k] for k in ("total_bits", "n_tiles", "n_luts", "max_tile_elems")},
        "max code length", int(inf["lengths"].max()))
    assert inf["total_bits"] > 2 ** 32                  # 64-bit stream offsets
    assert inf["lengths"].max() > 24 and inf["n_luts"] >= 4
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dfh.df_decompress_checked(dc, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    say("405B block: compare")
    ok = True
    step = 1 << 28
    for lo in range(0, src.size, step):
        hi = min(src.size, lo + step)
        ref = torch.from_numpy(src[lo:hi].view(np.int16)).to(dev)
        ok = ok and bool(torch.equal(out[lo:hi].view(torch.int16), ref))
    assert ok
    nt = int(inf["n_tiles"])
    rng = np.random.default_rng(7 + seed)
    ranges = [(0, 4), (nt // 2, nt // 2 + 4), (nt - 4, nt)]
    ranges += [(int(b), int(b) + 2) for b in rng.integers(0, nt - 2, 5)]
    say("405B block: oracle ranges")
    check_sampled_ranges(torch, orc, c, out, ranges)


def test_llama3_8b_lm_head(torch_dev, orc):
    """One large matrix on its own (the Llama-3-8B LM head, 128256 x 4096 =
    525,336,576 BF16 weights), one codebook, one launch."""
    torch, dev = torch_dev
    src, _ = synth.bf16_block(0, config=synth.CONFIG_LM_HEAD, shapes=synth.LLAMA3_8B_LM_HEAD)
    assert src.size == 128256 * 4096
    c = dfh.compress(0, src)
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dfh.df_decompress_checked(dc, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ok = True
    step = 1 << 27
    for lo in range(0, src.size, step):
        hi = min(src.size, lo + step)
        ref = torch.from_numpy(src[lo:hi].view(np.int16)).to(dev)
        ok = ok and bool(torch.equal(out[lo:hi].view(torch.int16), ref))
    assert ok
    nt = int(c.info()["n_tiles"])
    check_sampled_ranges(torch, orc, c, out, [(0, 8), (nt // 2, nt // 2 + 8), (nt - 8, nt)])
    say("lm head ok", nt, "tiles")
