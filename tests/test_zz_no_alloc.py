"""df_encode_device_noalloc (workspace in the library's code object, no
allocation) against df_encode_device (the caller's workspace): the same
sections and largest tile size, on two calls in a row, the second with a
smaller input, so the second runs over the first one's workspace contents.
Also the size limit.  Every call goes through the C ABI."""
import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def device_input(torch, dev, kind, a):
    if kind == dfh.KIND_BF16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def check_same(torch, dev, kind, a, n):
    """Encode with df_encode_device (via compress_device), then again with
    df_encode_device_noalloc into sections filled with a byte pattern."""
    t = device_input(torch, dev, kind, a)
    dc = dfh.compress_device(kind, t, n=n if kind == dfh.KIND_U4 else None)
    torch.cuda.synchronize()
    sec = {name: torch.full_like(dc.sections[name], 0xA5) for name in ("bitstream", "gaps", "tile_out", "sign_mantissa")}
    mt = torch.full((1,), -1, dtype=torch.int32, device=dev)
    dfh.df_encode_device_noalloc(kind, t, dc.n, dc.lengths, dc.layout, sec, mt)
    torch.cuda.synchronize()
    for name in sec:
        size = dc.info["section_bytes"][name]
        assert torch.equal(sec[name][:size], dc.sections[name][:size]), name
    assert int(mt.item()) == dc.info["max_tile_elems"]
    return dc


def test_noalloc_matches_workspace_encoder_twice(torch_dev):
    torch, dev = torch_dev
    src, _ = synth.bf16_block(0, shapes=synth.scaled_shapes(synth.LLAMA3_8B_BLOCK, 2))   # 54.5M weights
    print("no-alloc encode: BF16", src.size, flush=True)
    check_same(torch, dev, dfh.KIND_BF16, src, src.size)
    q = synth.quantize_u8(np.random.default_rng(3).normal(0, 0.02, 1_000_003).astype(np.float32), True)
    print("no-alloc encode: uint8", q.size, flush=True)
    check_same(torch, dev, dfh.KIND_U8, q, q.size)


def test_noalloc_small_and_empty(torch_dev):
    torch, dev = torch_dev
    q = np.clip(np.rint(np.random.default_rng(4).normal(7.5, 2.2, 70_001)), 0, 15).astype(np.uint8)
    check_same(torch, dev, dfh.KIND_U4, synth.pack_u4(q), q.size)
    check_same(torch, dev, dfh.KIND_BF16, np.zeros(0, np.uint16), 0)


def test_noalloc_rejects_inputs_beyond_its_workspace(torch_dev):
    torch, dev = torch_dev
    n = 5_000_000_000
    assert dfh.df_encode_workspace_bytes(n) > dfh.ENCODE_SCRATCH_BYTES
    hist = np.zeros(256, np.uint64)
    hist[7] = n
    lengths = np.zeros(256, np.uint8)
    lengths[7] = 1
    lay = dfh.df_encode_layout(dfh.KIND_U8, n, hist, 7, lengths)
    t = torch.zeros(64, dtype=torch.uint8, device=dev)
    sec = {name: torch.zeros(64, dtype=torch.uint8, device=dev) for name in ("bitstream", "gaps", "tile_out",
                                                                             "sign_mantissa")}
    mt = torch.zeros(1, dtype=torch.int32, device=dev)
    with pytest.raises(dfh.DFError) as e:
        dfh.df_encode_device_noalloc(dfh.KIND_U8, t, n, lengths, lay, sec, mt)
    assert e.value.status == -1
    # the largest n the workspace takes is accepted by the size check
    assert dfh.df_encode_workspace_bytes(4_000_000_000) <= dfh.ENCODE_SCRATCH_BYTES
