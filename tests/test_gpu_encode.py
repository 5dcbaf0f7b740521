"""Device-side encoding: the sections the GPU encoder writes must be
byte-identical to the CPU oracle's encoding of the same input (histogram,
code lengths, stream, gaps, tile offsets, sign|mantissa plane, hierarchical
tables) and to the host encoder's, and decode back to the input on the GPU."""
import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from decoder_tables import dtab_of
from lossless_entropy_coded_huffman_amd import synth

pytestmark = pytest.mark.gpu

SIZES = [0, 1, 2, 63, 64, 65, 4095, 4096, 4097, 16384, 16385, 100_003, 1_000_001]


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def host_input(kind, n, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 0.02, n).astype(np.float32)
    if kind == dfh.KIND_BF16:
        return synth.bf16_rne(x)
    if kind == dfh.KIND_U8:
        return synth.quantize_u8(x, bool(seed & 1))
    return synth.pack_u4(synth.quantize_u4(x, bool(seed & 1)))


def device_tensor(torch, dev, kind, a):
    if kind == dfh.KIND_BF16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def check_against_oracle(orc, dc, kind, a, nn):
    """The device container against the oracle's own encoding of the same
    input: histogram -> code lengths -> bit-serial encode -> hierarchical
    tables, and the decoder-side table from its test-side definition."""
    o = orc.compress(kind, a, n=nn)
    assert np.array_equal(dc.info["lengths"], o["lengths"])
    for k in ("n", "total_bits", "n_threads", "n_tiles", "max_tile_elems", "n_luts"):
        assert dc.info[k] == o[k], k
    for name in ("bitstream", "gaps", "tile_out", "sign_mantissa", "lut"):
        want = o[name]
        if want is None:   # no sign|mantissa plane for uint8 and uint4
            assert dc.info["section_bytes"][name] == 0
            continue
        want = np.ascontiguousarray(want).view(np.uint8)
        assert dc.info["section_bytes"][name] == want.size, name
        assert np.array_equal(dc.sections[name][: want.size].cpu().numpy(), want), name
    want = dtab_of(kind, o["lengths"], orc.canonical_codes(o["lengths"]))
    assert np.array_equal(dc.sections["dtab"][: want.size].cpu().numpy(), want)


def check(torch, dev, kind, a, n, orc=None):
    nn = n if kind == dfh.KIND_U4 else None
    host = dfh.compress(kind, a, n=nn)
    t = device_tensor(torch, dev, kind, a)
    h_dev = dfh.df_histogram_device(kind, t, nn).cpu().numpy().view(np.uint64)
    assert np.array_equal(h_dev, dfh.df_histogram(kind, a, nn))
    if orc is not None:
        assert np.array_equal(h_dev, orc.histogram(kind, a, nn))
    dc = dfh.compress_device(kind, t, n=nn)
    torch.cuda.synchronize()
    if orc is not None:
        check_against_oracle(orc, dc, kind, a, nn)
    hi = host.info()
    for k in ("n", "total_bits", "n_threads", "n_tiles", "n_luts", "max_tile_elems"):
        assert dc.info[k] == hi[k], k
    for name in dfh.SECTION_NAMES:
        size = hi["section_bytes"][name]
        got = dc.sections[name][:size].cpu().numpy()
        assert np.array_equal(got, np.asarray(host.section(name)).view(np.uint8)), name
    if n:
        out = dc.empty_output()
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        dfh.df_decompress_checked(dc, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        want = a.view(np.int16) if kind == dfh.KIND_BF16 else a
        got = out.view(torch.int16) if kind == dfh.KIND_BF16 else out
        assert torch.equal(got, torch.from_numpy(want).to(dev))


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("n", SIZES)
def test_device_encoder_matches_oracle_and_host(torch_dev, orc, kind, n):
    torch, dev = torch_dev
    print("encode", kind, n, flush=True)
    check(torch, dev, kind, host_input(kind, n, n + 11 * kind), n, orc)


def test_device_encoder_long_codes_and_one_symbol(torch_dev, orc):
    torch, dev = torch_dev
    rng = np.random.default_rng(4)
    t3 = synth.bf16_rne((rng.standard_t(3, 2_000_000) * 0.02 / np.sqrt(3)).astype(np.float32))
    check(torch, dev, 0, t3, t3.size, orc)
    # geometric counts: uint8 and uint4 codes past the decoder tables' index width
    g = np.minimum(rng.geometric(0.45, 1_000_001) - 1, 255).astype(np.uint8)
    check(torch, dev, 1, g, g.size, orc)
    q = np.minimum(rng.geometric(0.55, 1_000_001) - 1, 15).astype(np.uint8)
    check(torch, dev, 2, synth.pack_u4(q), q.size, orc)
    check(torch, dev, 1, np.full(70_001, 9, np.uint8), 70_001, orc)
    check(torch, dev, 2, synth.pack_u4(np.full(70_001, 3, np.uint8)), 70_001, orc)


def test_device_encoder_8b_block(torch_dev, orc):
    torch, dev = torch_dev
    src, _ = synth.bf16_block(0)
    check(torch, dev, 0, src, src.size, orc)
    layers = synth.u4_block(0)
    _, p, n, _ = layers[4]
    check(torch, dev, 2, p, n, orc)
    _, q, _ = synth.u8_block(1)[0]
    check(torch, dev, 1, q, q.size, orc)


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_symbol_device(torch_dev, orc, kind):
    # the coded symbol of single elements, against the oracle's field split
    # (BF16 exponent), the byte itself (uint8) and the nibble (uint4)
    torch, dev = torch_dev
    n = 100_001
    a = host_input(kind, n, 31 + kind)
    if kind == dfh.KIND_BF16:
        a = np.random.default_rng(5).integers(0, 65536, n).astype(np.uint16)   # every exponent
    t = device_tensor(torch, dev, kind, a)
    for i in (0, 1, 2, 77, n // 2, n - 2, n - 1):
        got = int(dfh.df_symbol_device(kind, t, i).item())
        if kind == dfh.KIND_BF16:
            want = int(orc.split_bf16(a[i:i + 1])[0][0])
        elif kind == dfh.KIND_U8:
            want = int(a[i])
        else:
            want = int(a[i // 2] >> (4 * (i % 2))) & 15
        assert got == want, (kind, i)


def test_device_encoder_rejects_misaligned_source(torch_dev):
    # the encoder kernels read 16-byte vectors: a source that does not start
    # on a 16-byte boundary is refused before any launch
    torch, dev = torch_dev
    src = torch.zeros(1000, dtype=torch.int16, device=dev)[1:]
    with pytest.raises(dfh.DFError) as e:
        dfh.df_histogram_device(dfh.KIND_BF16, src)
    assert e.value.status == -1


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_device_encoder_batch_on_a_side_stream(torch_dev, kind):
    # compress_device_batch: one histogram read-back and one tile-size
    # read-back for all containers, tables through one pinned copy; run on a
    # stream other than the current one, with an empty container among them
    torch, dev = torch_dev
    sizes = [70_001, 0, 1, 16_385, 1_000_001, 4096]
    hosts = [host_input(kind, n, 500 + i) for i, n in enumerate(sizes)]
    ts = [device_tensor(torch, dev, kind, a) for a in hosts]
    nn = sizes if kind == dfh.KIND_U4 else None
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    dcs = dfh.compress_device_batch(kind, ts, ns=nn, stream=side)
    torch.cuda.current_stream(dev).wait_stream(side)
    for a, n, dc in zip(hosts, sizes, dcs):
        host = dfh.compress(kind, a, n=n if kind == dfh.KIND_U4 else None)
        hi = host.info()
        for k in ("n", "total_bits", "n_threads", "n_tiles", "n_luts", "max_tile_elems"):
            assert dc.info[k] == hi[k], k
        for name in dfh.SECTION_NAMES:
            size = hi["section_bytes"][name]
            got = dc.sections[name][:size].cpu().numpy()
            assert np.array_equal(got, np.asarray(host.section(name)).view(np.uint8)), name
        if n:
            out = dc.empty_output()
            dfh.df_decompress(dc, out)
            want = a.view(np.int16) if kind == dfh.KIND_BF16 else a
            got = out.view(torch.int16) if kind == dfh.KIND_BF16 else out
            assert torch.equal(got, torch.from_numpy(want).to(dev))


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("n", [0, 1, 65, 4097])
def test_device_encoder_writes_every_section_byte(torch_dev, orc, kind, n):
    # sections handed in full of a byte pattern come out equal to the
    # oracle's, padding included (an empty input's stream and gap sections
    # are all padding)
    torch, dev = torch_dev
    a = host_input(kind, n, 900 + n)
    t = device_tensor(torch, dev, kind, a)
    nn = n if kind == dfh.KIND_U4 else None
    dc = dfh.compress_device(kind, t, n=nn)
    sec = {name: torch.full_like(dc.sections[name], 0xA5) for name in ("bitstream", "gaps", "tile_out", "sign_mantissa")}
    ws = torch.empty(max(dfh.df_encode_workspace_bytes(n), 16), dtype=torch.uint8, device=dev)
    mt = torch.full((1,), -1, dtype=torch.int32, device=dev)
    dfh.df_encode_device(kind, t, n, dc.lengths, dc.layout, sec, ws, mt)
    torch.cuda.synchronize()
    o = orc.compress(kind, a, n=nn)
    for name in sec:
        if o[name] is None:
            continue
        want = np.ascontiguousarray(o[name]).view(np.uint8)
        assert np.array_equal(sec[name][: want.size].cpu().numpy(), want), name
    assert int(mt.item()) == o["max_tile_elems"]
