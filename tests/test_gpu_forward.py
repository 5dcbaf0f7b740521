"""Block decompression overlapped with a Llama-shaped forward pass: the
output must be bit-identical to the same forward pass with every weight
resident (the DF11 digest's claim that the compressed model computes exactly
what the BF16 model computes)."""
import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import forward as fw

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def run(torch, dev, shape, n_blocks, tokens, seed, cap=0):
    host = fw.random_blocks(n_blocks, shape, seed)
    model = fw.CompressedBlocks([dfh.compress(0, h) for h in host], shape, dev, decode_workgroups=cap)
    g = torch.Generator(device="cpu").manual_seed(seed)
    x = (torch.randn(tokens, shape.hidden, generator=g) * 0.5).to(torch.bfloat16).to(dev)
    ref = fw.resident_forward(x, [fw.to_torch(h, dev) for h in host], shape)
    over = model.forward(x, overlap=True)
    serial = model.forward(x, overlap=False)
    again = model.forward(x, overlap=True)
    torch.cuda.synchronize()
    assert torch.isfinite(ref.float()).all()
    for y in (over, serial, again):
        assert torch.equal(y.view(torch.int16), ref.view(torch.int16))


def test_small_blocks_bit_identical(torch_dev):
    torch, dev = torch_dev
    shape = fw.BlockShape(hidden=512, heads=8, kv_heads=2, ffn=1536)
    run(torch, dev, shape, n_blocks=5, tokens=64, seed=3)


def test_llama3_8b_blocks_bit_identical(torch_dev):
    torch, dev = torch_dev
    run(torch, dev, fw.LLAMA3_8B, n_blocks=3, tokens=128, seed=0)


def test_llama3_8b_blocks_capped_side_decode(torch_dev):
    # the side-stream decode limited to 32 workgroups runs beside the blocks
    torch, dev = torch_dev
    run(torch, dev, fw.LLAMA3_8B, n_blocks=3, tokens=256, seed=1, cap=32)
