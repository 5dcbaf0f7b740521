"""GPU parity: the HIP decoder against the definition of the result
(decode(encode(x)) == x, bit for bit) and against the CPU oracle's own
decode of the same container.  Bit-exact (0 ULP) everywhere: this is
integer work.  Every call goes through the C ABI."""
import sys

import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from lossless_entropy_coded_huffman_amd import synth

pytestmark = pytest.mark.gpu

EDGE_SIZES = [1, 2, 63, 64, 65, 255, 256, 257, 6143, 16384, 16385, 100_003, 1_000_001]


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def host_of(t, kind):
    import torch
    a = t.view(torch.int16) if kind == 0 else t
    a = a.cpu().numpy()
    return a.view(np.uint16) if kind == 0 else a


def gpu_decode(torch_dev, c, checked=True):
    torch, dev = torch_dev
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    if checked:
        dfh.df_decompress_checked(dc, out, err)
    else:
        dfh.df_decompress(dc, out)
    torch.cuda.synchronize()
    return host_of(out, dc.kind), int(err.item())


def oracle_container(c):
    inf = c.info()
    d = {k: np.asarray(c.section(k)) for k in dfh.SECTION_NAMES}
    d.update(kind=inf["kind"], n=inf["n"], n_tiles=inf["n_tiles"], n_threads=inf["n_threads"],
             lengths=inf["lengths"])
    return d


def check(torch_dev, orc, kind, src, checked=True, oracle_threads=8):
    c = dfh.compress(kind, src)
    got, err = gpu_decode(torch_dev, c, checked)
    assert err == 0
    assert np.array_equal(got, src)
    ref = orc.decode_tiles(oracle_container(c), oracle_threads)
    assert np.array_equal(got, ref)
    return c


def bf16_normal(n, seed, std=0.02):
    return synth.bf16_rne(np.random.default_rng(seed).normal(0, std, n).astype(np.float32))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_c1_tensor(torch_dev, orc, seed):
    say("c1 seed", seed)
    check(torch_dev, orc, 0, synth.c1_tensor(seed))


@pytest.mark.parametrize("n", EDGE_SIZES)
@pytest.mark.parametrize("kind", [0, 1])
def test_edge_sizes(torch_dev, orc, kind, n):
    say("edge", kind, n)
    if kind == 0:
        src = bf16_normal(n, n)
    else:
        src = synth.quantize_u8(np.random.default_rng(n).normal(0, 1, n).astype(np.float32), n % 2 == 1)
    check(torch_dev, orc, kind, src)


def test_unchecked_equals_checked(torch_dev, orc):
    src = bf16_normal(3_000_000, 7)
    c = dfh.compress(0, src)
    a, _ = gpu_decode(torch_dev, c, checked=False)
    b, err = gpu_decode(torch_dev, c, checked=True)
    assert err == 0 and np.array_equal(a, src) and np.array_equal(b, src)


def test_empty(torch_dev):
    torch, dev = torch_dev
    for kind in (0, 1):
        c = dfh.compress(kind, np.zeros(0, np.uint16 if kind == 0 else np.uint8))
        dc = dfh.to_device(c, dev)
        out = torch.empty(16, dtype=torch.uint8, device=dev)
        dfh.df_decompress(dc, out)
        torch.cuda.synchronize()


@pytest.mark.parametrize("n", [1, 64, 65, 16384, 16385, 40000])
def test_single_symbol(torch_dev, orc, n):
    say("single symbol", n)
    check(torch_dev, orc, 0, np.full(n, 0xBC00, np.uint16))
    check(torch_dev, orc, 1, np.full(n, 77, np.uint8))


def test_all_bf16_patterns(torch_dev, orc):
    u = np.random.default_rng(11).permutation(65536).astype(np.uint16)
    check(torch_dev, orc, 0, np.concatenate([u, u[::-1], u]))


def test_stream_ends_on_chunk_and_tile_boundaries(torch_dev, orc):
    # 256 equal counts give 8-bit codes: total bits = 8 n
    for n in (8, 2048, 4096, 2048 * 7):
        src = np.tile(np.arange(256, dtype=np.uint8), n // 256 + 1)[:n]
        if n < 256:
            continue
        c = check(torch_dev, orc, 1, src)
        assert c.info()["total_bits"] % 64 == 0


def test_codes_of_every_length_up_to_32(torch_dev, orc):
    # lengths 1, 2, ..., 32, 32 (Kraft sum exactly 1): symbols drawn uniformly,
    # so codes of 25-32 bits (four table levels) are frequent and straddle
    # chunk and tile ends
    ln = np.zeros(256, np.uint8)
    syms = np.arange(40, 73)
    ln[syms] = list(range(1, 33)) + [32]
    rng = np.random.default_rng(5)
    for kind in (0, 1):
        s = rng.choice(syms, 300_000).astype(np.uint8)
        if kind == 0:
            src = (s.astype(np.uint16) << 7) | rng.integers(0, 2, s.size).astype(np.uint16) << 15 \
                | rng.integers(0, 128, s.size).astype(np.uint16)
        else:
            src = s
        c = dfh.df_encode(kind, src, ln)
        assert c.info()["n_luts"] >= 4
        got, err = gpu_decode(torch_dev, c)
        assert err == 0 and np.array_equal(got, src)
        assert np.array_equal(got, orc.decode_tiles(oracle_container(c), 8))


def test_heavy_tail_t3(torch_dev, orc):
    src = synth.bf16_rne((np.random.default_rng(3).standard_t(3, 4_000_000) * 0.02 / np.sqrt(3))
                         .astype(np.float32))
    c = check(torch_dev, orc, 0, src)
    assert c.info()["lengths"].max() > 12


def test_u8_entrollm_layers(torch_dev, orc):
    layers = synth.u8_block(0, shapes=synth.scaled_shapes(synth.LLAMA3_8B_BLOCK, 8))
    for name, q, asym in layers:
        say("u8 layer", name, q.size, asym)
        check(torch_dev, orc, 1, q)


def test_batch_matches_single(torch_dev, orc):
    torch, dev = torch_dev
    for kind in (0, 1):
        srcs = []
        for i, n in enumerate([1, 5000, 700_001, 65, 3_000_000]):
            if kind == 0:
                srcs.append(bf16_normal(n, 40 + i, 0.01 * (i + 1)))
            else:
                srcs.append(synth.quantize_u8(np.random.default_rng(i).normal(0, 1, n).astype(np.float32), i % 2 == 0))
        cs = [dfh.compress(kind, s) for s in srcs]
        dcs = [dfh.to_device(c, dev) for c in cs]
        outs = [dc.empty_output() for dc in dcs]
        dfh.df_decompress_batch(dcs, outs)
        torch.cuda.synchronize()
        for s, o in zip(srcs, outs):
            assert np.array_equal(host_of(o, kind), s)


def test_batch_more_than_16(torch_dev):
    torch, dev = torch_dev
    srcs = [bf16_normal(10_000 + 977 * i, 90 + i) for i in range(21)]
    dcs = [dfh.to_device(dfh.compress(0, s), dev) for s in srcs]
    outs = [dc.empty_output() for dc in dcs]
    dfh.df_decompress_batch(dcs, outs)
    torch.cuda.synchronize()
    for s, o in zip(srcs, outs):
        assert np.array_equal(host_of(o, 0), s)


def test_no_writes_outside_dst(torch_dev):
    torch, dev = torch_dev
    for kind, n in ((0, 100_003), (1, 100_003), (0, 17), (1, 33)):
        src = bf16_normal(n, 1) if kind == 0 else np.random.default_rng(2).integers(0, 40, n).astype(np.uint8)
        dc = dfh.to_device(dfh.compress(kind, src), dev)
        esz = 2 if kind == 0 else 1
        guard = 4096
        buf = torch.full((guard * 2 + n * esz + 16,), 0xA5, dtype=torch.uint8, device=dev)
        dst = buf[guard: guard + n * esz]
        dfh.df_decompress(dc, dst)
        torch.cuda.synchronize()
        b = buf.cpu().numpy()
        assert (b[:guard] == 0xA5).all() and (b[guard + n * esz:] == 0xA5).all()
        got = b[guard: guard + n * esz].view(np.uint16 if kind == 0 else np.uint8)
        assert np.array_equal(got, src)


def test_checked_reports_bad_tile_offsets(torch_dev):
    # error path forced from the host: a tile offset edited on the device;
    # the kernel clamps every access and exits normally, reporting the count
    # mismatch
    torch, dev = torch_dev
    src = bf16_normal(500_000, 4)
    dc = dfh.to_device(dfh.compress(0, src), dev)
    to = dc.sections["tile_out"].view(torch.int64)
    to[1] += 1
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dfh.df_decompress_checked(dc, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) & dfh.DEVERR_COUNT


@pytest.mark.parametrize("checked", [True, False])
def test_corrupt_tile_is_contained(torch_dev, checked):
    # error path forced from the host: one lane's 64 stream bits in one tile
    # are zeroed on the device (all-zero bits decode as the first, shortest
    # canonical code over and over, so the tile's code count no longer
    # matches its offsets).  Tiles share a tile group's staging buffer in
    # turn (each group decodes several tiles here: more tiles than the GPU
    # has group slots), so this checks that a corrupt tile leaves no bytes
    # behind for the next one: every element outside the corrupt tile and
    # the tile before it (whose last lane reads ahead into it) is exact.
    torch, dev = torch_dev
    src = bf16_normal(30_000_000, 12)
    c = dfh.compress(0, src)
    nt = int(c.info()["n_tiles"])
    assert nt > 4096
    to = np.asarray(c.section("tile_out")).astype(np.int64)
    dc = dfh.to_device(c, dev)
    t = nt // 3
    bits = dc.sections["bitstream"].view(torch.int32)
    bits[t * 512 + 200: t * 512 + 202] = 0
    out = dc.empty_output()
    if checked:
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        dfh.df_decompress_checked(dc, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) != 0
    else:
        dfh.df_decompress(dc, out)
    got = host_of(out, 0)
    lo, hi = int(to[t - 1]), int(to[t + 1])
    assert np.array_equal(got[:lo], src[:lo])
    assert np.array_equal(got[hi:], src[hi:])


def u8_normal(n, seed, asym=False):
    return synth.quantize_u8(np.random.default_rng(seed).normal(0, 1, n).astype(np.float32), asym)


def test_u8_tile_pairs_odd_and_even_tile_counts(torch_dev, orc):
    # a uint8 lane group decodes two tiles per step, each lane two
    # neighbouring chunks: containers of 1..9 tiles (a last pair of one tile
    # when the count is odd), streams ending inside a lane's first and
    # second chunk, checked and unchecked
    counts = set()
    for i, n in enumerate([2000, 2600, 5100, 7700, 9900, 12_600, 17_700, 19_999, 22_222]):
        src = u8_normal(n, 300 + i, i % 2 == 1)
        c = check(torch_dev, orc, 1, src, checked=i % 2 == 0)
        counts.add(int(c.info()["n_tiles"]) % 2)
    assert counts == {0, 1}


def test_u8_chunk_pairs_split_by_stream_end(torch_dev, orc):
    # 8-bit codes: the stream ends exactly at a chunk end, so the last lane
    # has its first chunk only (n_threads odd) or both (n_threads even)
    for n in (8 * 129, 8 * 130, 2048 + 8, 2048 * 3 - 8, 2048 * 3 + 8):
        src = np.tile(np.arange(256, dtype=np.uint8), n // 256 + 1)[:n]
        c = check(torch_dev, orc, 1, src)
        assert c.info()["total_bits"] == 8 * n


def test_u8_checked_reports_bad_tile_offsets(torch_dev):
    # error path forced from the host, as for BF16: the offset where a tile
    # pair starts edited on the device (a uint8 launch reads the offsets of
    # pair starts only, tile_out[2p])
    torch, dev = torch_dev
    dc = dfh.to_device(dfh.compress(1, u8_normal(200_000, 6)), dev)
    to = dc.sections["tile_out"].view(torch.int64)
    to[2] += 1
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dfh.df_decompress_checked(dc, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) & dfh.DEVERR_COUNT


@pytest.mark.parametrize("checked", [True, False])
def test_u8_corrupt_tile_is_contained(torch_dev, checked):
    # as for BF16, with uint8 tile pairs: every element outside the corrupt
    # tile's pair and the pair before it is exact.  The lane's bits are set
    # to ones, which decode as the longest code (24 bits here), so its code
    # count drops to three; zero bits would decode as the shortest code,
    # 6 bits, about as many codes as the real stream holds
    torch, dev = torch_dev
    src = u8_normal(12_000_000, 13)
    c = dfh.compress(1, src)
    nt = int(c.info()["n_tiles"])
    assert nt > 4096
    to = np.asarray(c.section("tile_out")).astype(np.int64)
    dc = dfh.to_device(c, dev)
    t = nt // 3
    bits = dc.sections["bitstream"].view(torch.int32)
    bits[t * 512 + 300: t * 512 + 302] = -1
    out = dc.empty_output()
    if checked:
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        dfh.df_decompress_checked(dc, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) != 0
    else:
        dfh.df_decompress(dc, out)
    got = host_of(out, 1)
    p = t // 2 * 2
    lo, hi = int(to[max(p - 2, 0)]), int(to[min(p + 2, nt)])
    assert np.array_equal(got[:lo], src[:lo])
    assert np.array_equal(got[hi:], src[hi:])


def test_rejects_bad_arguments(torch_dev):
    torch, dev = torch_dev
    dc = dfh.to_device(dfh.compress(0, bf16_normal(1000, 1)), dev)
    out = torch.empty(1000 * 2 + 16, dtype=torch.uint8, device=dev)
    with pytest.raises(dfh.DFError):
        dfh.df_decompress(dc, out[1:1 + 2000])      # misaligned destination
    dc.view.n_luts = 0
    with pytest.raises(dfh.DFError):
        dfh.df_decompress(dc, out)


# ------------------------------------------------------------ full-size cases
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_llama3_8b_block_bf16(torch_dev, orc, seed):
    """One Llama-3-8B-shaped block (218,103,808 BF16 weights), one codebook,
    one launch -- the benchmark's workload and launch."""
    torch, dev = torch_dev
    say("8B block: generate, seed", seed)
    src, _ = synth.bf16_block(seed)
    say("8B block: compress")
    c = dfh.compress(0, src)
    inf = c.info()
    say("8B block:", {k: inf[k] for k in ("n", "total_bits", "n_tiles", "n_luts", "max_tile_elems")})
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dfh.df_decompress_checked(dc, out, err)
    dfh.df_decompress(dc, out)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    ref = torch.from_numpy(src.view(np.int16)).to(dev)
    assert torch.equal(out.view(torch.int16), ref)
    say("8B block: oracle decode")
    got = host_of(out, 0)
    assert np.array_equal(got, orc.decode_tiles(oracle_container(c), 16))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_llama3_8b_block_u8(torch_dev, orc, seed):
    """The EntroLLM-style block: seven per-layer uint8 containers, one batched
    launch; every layer against its input and the oracle's decode."""
    torch, dev = torch_dev
    layers = synth.u8_block(seed)
    cs = [dfh.compress(1, q) for _, q, _ in layers]
    dcs = [dfh.to_device(c, dev) for c in cs]
    outs = [dc.empty_output() for dc in dcs]
    dfh.df_decompress_batch(dcs, outs)
    torch.cuda.synchronize()
    for (name, q, _), c, o in zip(layers, cs, outs):
        say("u8 layer", name, "seed", seed)
        assert torch.equal(o, torch.from_numpy(q).to(dev))
        assert np.array_equal(host_of(o, 1), orc.decode_tiles(oracle_container(c), 16))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_llama3_8b_block_u4(torch_dev, orc, seed):
    """The 4-bit EntroLLM-style block: seven per-layer uint4 containers, one
    batched launch, packed outputs; every layer against its input and the
    oracle's packed decode."""
    torch, dev = torch_dev
    layers = synth.u4_block(seed)
    cs = [dfh.compress(dfh.KIND_U4, p, n=n) for _, p, n, _ in layers]
    dcs = [dfh.to_device(c, dev) for c in cs]
    outs = [dc.empty_output() for dc in dcs]
    dfh.df_decompress_batch(dcs, outs)
    torch.cuda.synchronize()
    for (name, p, n, _), c, o in zip(layers, cs, outs):
        say("u4 layer", name, "seed", seed)
        assert torch.equal(o, torch.from_numpy(p).to(dev))
        assert np.array_equal(host_of(o, 2), orc.pack_u4(orc.decode_tiles(oracle_container(c), 16)))


def test_offsets_beyond_2_pow_31(torch_dev):
    """Element indices and tile offsets at and above 2^31 (uint8, two symbols,
    one-bit codes: 2^31 + 2^20 + 37 weights, 2.2 GB)."""
    torch, dev = torch_dev
    n = (1 << 31) + (1 << 20) + 37
    src = np.zeros(n, np.uint8)
    src[1::3] = 200
    src[n - 5:] = 200
    c = dfh.compress(1, src)
    assert int(np.asarray(c.section("tile_out"))[-2]) > (1 << 31)
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    dfh.df_decompress_checked(dc, out, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out, torch.from_numpy(src).to(dev))


# ------------------------------------------------------------------- uint4
def u4_symbols(n, seed, std=2.2):
    return np.clip(np.rint(np.random.default_rng(seed).normal(7.5, std, n)), 0, 15).astype(np.uint8)


def check_u4(torch_dev, orc, q, checked=True):
    """q: one symbol 0..15 per element.  The decoder's packed output must equal
    the packed input and the oracle's packed decode of the same container."""
    n = q.size
    packed = synth.pack_u4(q)
    c = dfh.compress(dfh.KIND_U4, packed, n=n)
    got, err = gpu_decode(torch_dev, c, checked)
    assert err == 0
    assert got.size == (n + 1) // 2
    assert np.array_equal(got, packed)
    assert np.array_equal(got, orc.pack_u4(orc.decode_tiles(oracle_container(c), 8)))
    return c


@pytest.mark.parametrize("n", EDGE_SIZES)
def test_u4_edge_sizes(torch_dev, orc, n):
    say("u4 edge", n)
    check_u4(torch_dev, orc, u4_symbols(n, n))


def test_u4_odd_tile_boundaries(torch_dev, orc):
    # many tiles: about half end on an odd element, sharing an output byte
    # with the next tile, and of those some take the next symbol from the
    # last lookup's lookahead and some decode it separately
    for seed, std in ((1, 2.2), (2, 0.9), (3, 4.0)):
        q = u4_symbols(3_000_001, seed, std)
        c = check_u4(torch_dev, orc, q)
        to = np.asarray(c.section("tile_out")).astype(np.int64)
        assert (to[1:-1] % 2 == 1).sum() > 50


def test_u4_long_codes_and_single_symbol(torch_dev, orc):
    # geometric-like counts give codes up to 15 bits (past the 12-bit table)
    rng = np.random.default_rng(9)
    q = np.minimum(rng.geometric(0.55, 2_000_000) - 1, 15).astype(np.uint8)
    c = check_u4(torch_dev, orc, q)
    assert c.info()["lengths"].max() > 12
    for n in (1, 2, 3, 16385, 40001):
        check_u4(torch_dev, orc, np.full(n, 5, np.uint8))


def test_u4_batch_and_checked(torch_dev, orc):
    torch, dev = torch_dev
    layers = synth.u4_block(0, shapes=synth.scaled_shapes(synth.LLAMA3_8B_BLOCK, 8))
    cs = [dfh.compress(dfh.KIND_U4, p, n=n) for _, p, n, _ in layers]
    dcs = [dfh.to_device(c, dev) for c in cs]
    outs = [dc.empty_output() for dc in dcs]
    dfh.df_decompress_batch(dcs, outs)
    torch.cuda.synchronize()
    for (_, p, n, _), o in zip(layers, outs):
        assert np.array_equal(host_of(o, 2), p)


def test_u4_codes_up_to_32_bits(torch_dev, orc):
    # an incomplete uint4 code: lengths 1..15 and one 32-bit code (Kraft sum
    # below 1), symbols drawn uniformly, so codes past the 12-bit table (up
    # to four table levels) are frequent and straddle chunk and tile ends,
    # and tiles end on odd elements with long codes next
    ln = np.zeros(256, np.uint8)
    ln[:16] = list(range(1, 16)) + [32]
    q = np.random.default_rng(11).integers(0, 16, 300_001).astype(np.uint8)
    packed = synth.pack_u4(q)
    c = dfh.df_encode(dfh.KIND_U4, packed, ln, n=q.size)
    assert c.info()["n_luts"] >= 4
    for checked in (True, False):
        got, err = gpu_decode(torch_dev, c, checked)
        assert err == 0 and np.array_equal(got, packed)
    assert np.array_equal(got, orc.pack_u4(orc.decode_tiles(oracle_container(c), 8)))


@pytest.mark.parametrize("cap", [1, 7, 33])
@pytest.mark.parametrize("kind", [1, 2])
def test_u8_u4_capped_launch(torch_dev, orc, kind, cap):
    # a launch capped to a few workgroups runs its waves at the base priority
    # and walks many steps per workgroup (the uint8 waves' own stores, the
    # uint4 nibble staging)
    torch, dev = torch_dev
    if kind == 1:
        want = u8_normal(2_000_003, 5)
        c = dfh.compress(1, want)
    else:
        q = u4_symbols(2_000_003, 6)
        want = synth.pack_u4(q)
        c = dfh.compress(2, want, n=q.size)
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for checked in (False, True):
        out.zero_()
        if checked:
            dfh.df_decompress_checked(dc, out, err, max_workgroups=cap)
        else:
            dfh.df_decompress(dc, out, max_workgroups=cap)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert np.array_equal(host_of(out, kind), want), (kind, cap, checked)


@pytest.mark.parametrize("cap", [0, 1, 5])
def test_u4_large_tiles_many_steps(torch_dev, orc, cap):
    # one symbol in 99.5% of the elements: 1-bit codes, tiles of close to
    # 16384 elements, so each group's two staging buffers are near their
    # largest (the launch then fits fewer groups or workgroups per CU), and
    # capped launches walk many steps per group, the buffers alternating
    torch, dev = torch_dev
    rng = np.random.default_rng(70 + cap)
    q = np.full(3_000_001, 5, np.uint8)
    pick = rng.random(q.size) < 0.005
    q[pick] = rng.integers(0, 16, int(pick.sum()))
    want = synth.pack_u4(q)
    c = dfh.compress(2, want, n=q.size)
    assert int(c.info()["max_tile_elems"]) > 14000
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for checked in (False, True):
        out.zero_()
        if checked:
            dfh.df_decompress_checked(dc, out, err, max_workgroups=cap)
        else:
            dfh.df_decompress(dc, out, max_workgroups=cap)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        got = host_of(out, 2)
        assert np.array_equal(got, want), (cap, checked)
    assert np.array_equal(got, orc.pack_u4(orc.decode_tiles(oracle_container(c), 8)))


def test_u4_batch_of_large_and_small_tiles(torch_dev, orc):
    # one launch over containers whose tiles differ four-fold in size: the
    # staging buffers (two per group) are sized by the largest, and each
    # container's tiles are checked against its own input and the oracle
    torch, dev = torch_dev
    rng = np.random.default_rng(81)
    qs = [np.full(1_000_003, 9, np.uint8), rng.integers(0, 16, 700_001).astype(np.uint8),
          np.clip(np.rint(rng.normal(7.5, 2.2, 900_002)), 0, 15).astype(np.uint8)]
    qs[0][rng.random(qs[0].size) < 0.004] = 3
    cs = [dfh.compress(dfh.KIND_U4, synth.pack_u4(q), n=q.size) for q in qs]
    sizes = [int(c.info()["max_tile_elems"]) for c in cs]
    assert max(sizes) > 3 * min(sizes)
    dcs = [dfh.to_device(c, dev) for c in cs]
    outs = [dc.empty_output() for dc in dcs]
    dfh.df_decompress_batch(dcs, outs)
    torch.cuda.synchronize()
    for q, c, o in zip(qs, cs, outs):
        got = host_of(o, 2)
        assert np.array_equal(got, synth.pack_u4(q))
        assert np.array_equal(got, orc.pack_u4(orc.decode_tiles(oracle_container(c), 8)))


@pytest.mark.parametrize("cap", [0, 1, 5])
def test_u8_large_tiles_many_steps(torch_dev, orc, cap):
    # one byte value in 99.5% of the elements: 1-bit codes, tile pairs of
    # close to 32768 elements, so a group's staging is near its largest and
    # the launch fits fewer groups per CU; capped launches walk many steps
    # per wave (each wave's own store of its range)
    torch, dev = torch_dev
    rng = np.random.default_rng(90 + cap)
    want = np.full(3_000_001, 131, np.uint8)
    pick = rng.random(want.size) < 0.005
    want[pick] = rng.integers(120, 128, int(pick.sum()))  # (255 rare values would need over 64 table levels)
    c = dfh.compress(1, want)
    assert int(c.info()["max_tile_elems"]) > 14000
    dc = dfh.to_device(c, dev)
    out = dc.empty_output()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    for checked in (False, True):
        out.zero_()
        if checked:
            dfh.df_decompress_checked(dc, out, err, max_workgroups=cap)
        else:
            dfh.df_decompress(dc, out, max_workgroups=cap)
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        got = host_of(out, 1)
        assert np.array_equal(got, want), (cap, checked)
    assert np.array_equal(got, orc.decode_tiles(oracle_container(c), 8))


def test_u8_random_sizes_and_distributions(torch_dev, orc):
    # seeded sweep over container sizes (1 element to 40 tiles) and symbol
    # distributions: quantised normals, uniform bytes, geometric skews whose
    # rare symbols take long codes (up to 19 bits here; 32-bit codes are
    # test_codes_of_every_length_up_to_32's), three symbols; every case
    # bit-exact against the input and the oracle's decode
    rng = np.random.default_rng(2024)
    lengths_seen = set()
    for case in range(36):
        n = int(rng.integers(1, 120_000)) if case % 3 else int(rng.integers(1, 3000))
        d = case % 4
        if d == 0:
            src = u8_normal(n, 700 + case, case % 8 == 0)
        elif d == 1:
            src = rng.integers(0, 256, n).astype(np.uint8)
        elif d == 2:
            src = np.minimum(rng.geometric(0.35 + 0.1 * rng.random(), n) - 1, 255).astype(np.uint8)
        else:
            src = rng.choice(rng.choice(256, 3, replace=False), n).astype(np.uint8)
        say("u8 random case", case, n, d)
        c = check(torch_dev, orc, 1, src, checked=bool(case & 1))
        lengths_seen.add(int(c.info()["lengths"].max()))
    assert max(lengths_seen) >= 16 and min(lengths_seen) <= 2


@pytest.mark.parametrize("checked", [True, False])
def test_u4_corrupt_tile_is_contained(torch_dev, checked):
    # as for BF16 and uint8, with uint4's two staging buffers per group: one
    # lane's 64 stream bits in one tile set to ones (the longest code over
    # and over), so the tile's code count no longer matches its offsets.
    # Every output byte outside the corrupt tile and the tile before it
    # (whose last lane reads ahead into it, and which may share its last byte
    # with it) is exact: the corrupt tile leaves nothing behind in either
    # buffer for the tiles after it
    torch, dev = torch_dev
    q = u4_symbols(30_000_001, 14)
    want = synth.pack_u4(q)
    c = dfh.compress(2, want, n=q.size)
    nt = int(c.info()["n_tiles"])
    assert nt > 4096
    to = np.asarray(c.section("tile_out")).astype(np.int64)
    dc = dfh.to_device(c, dev)
    t = nt // 3
    bits = dc.sections["bitstream"].view(torch.int32)
    bits[t * 512 + 300: t * 512 + 302] = -1
    out = dc.empty_output()
    if checked:
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        dfh.df_decompress_checked(dc, out, err)
        torch.cuda.synchronize()
        assert int(err.item()) != 0
    else:
        dfh.df_decompress(dc, out)
    got = host_of(out, 2)
    lo, hi = int(to[t - 1]) // 2, (int(to[t + 1]) + 1) // 2
    assert np.array_equal(got[:lo], want[:lo])
    assert np.array_equal(got[hi:], want[hi:])


def test_u4_random_sizes_and_distributions(torch_dev, orc):
    # seeded sweep over uint4 container sizes (1 element to about 40 tiles,
    # odd and even counts) and nibble distributions: quantised normals of
    # several widths, uniform nibbles, geometric skews (codes up to 15
    # bits), two symbols; checked and unchecked, every case bit-exact
    # against the packed input and the oracle's packed decode
    rng = np.random.default_rng(4242)
    lengths_seen = set()
    for case in range(36):
        n = int(rng.integers(1, 250_000)) if case % 3 else int(rng.integers(1, 3000))
        d = case % 4
        if d == 0:
            q = u4_symbols(n, 900 + case, 0.5 + 3.5 * rng.random())
        elif d == 1:
            q = rng.integers(0, 16, n).astype(np.uint8)
        elif d == 2:
            q = np.minimum(rng.geometric(0.3 + 0.3 * rng.random(), n) - 1, 15).astype(np.uint8)
        else:
            q = rng.choice(rng.choice(16, 2, replace=False), n).astype(np.uint8)
        say("u4 random case", case, n, d)
        c = check_u4(torch_dev, orc, q, checked=bool(case & 1))
        lengths_seen.add(int(c.info()["lengths"].max()))
    assert max(lengths_seen) >= 10 and min(lengths_seen) <= 1


def test_bf16_random_sizes_and_distributions(torch_dev, orc):
    # seeded sweep: normals of random scale, Student-t(3) tails, uniformly
    # random 16-bit patterns (every exponent), near-constant values; small
    # containers (static tile order) and three of 40-70M weights, which take
    # the dynamic tile order; every case bit-exact against the input and,
    # below 8M weights, against the oracle's decode
    rng = np.random.default_rng(77)
    big = {5: 40_000_000, 11: 55_000_000, 17: 70_000_000}
    for case in range(20):
        n = big.get(case, int(rng.integers(1, 2_000_000)))
        d = case % 4
        if d == 0:
            src = bf16_normal(n, 900 + case, float(rng.uniform(0.002, 0.2)))
        elif d == 1:
            src = synth.bf16_rne((rng.standard_t(3, n) * 0.02).astype(np.float32))
        elif d == 2:
            src = rng.integers(0, 65536, n).astype(np.uint16)
        else:
            src = (0x3F80 + rng.integers(0, 3, n)).astype(np.uint16)
        say("bf16 random case", case, n, d)
        if n < 8_000_000:
            check(torch_dev, orc, 0, src, checked=bool(case & 1))
        else:
            got, err = gpu_decode(torch_dev, dfh.compress(0, src), checked=bool(case & 1))
            assert err == 0 and np.array_equal(got, src)


# ------------------------------------------- damaged decoder-side table
@pytest.mark.parametrize("kind", [0, 1, 2])
def test_table_entries_that_consume_no_bits(torch_dev, orc, kind):
    """Every entry of the decoder-side table replaced from the host by one that
    claims a code but consumes no bits (the kind of damage a caller-made view
    with a bad table could bring).  The kernel clears such entries while
    staging the table, so every code takes the hierarchical tables (intact
    here): the output is still the input, and a checked launch reports
    DF_DEVERR_CODE."""
    torch, dev = torch_dev
    n = 3_000_001
    if kind == 0:
        src = bf16_normal(n, 41)
        c = dfh.compress(0, src)
    elif kind == 1:
        src = u8_normal(n, 42, True)
        c = dfh.compress(1, src)
    else:
        q = u4_symbols(n, 43)
        src = synth.pack_u4(q)
        c = dfh.compress(2, src, n=n)
    dc = dfh.to_device(c, dev)
    tab = dc.sections["dtab"]
    if kind == 1:   # uint8: 8192 u32 pair entries (count 1, 0 bits), lengths left
        tab[: 4 * 8192].view(torch.int32).fill_(1 << 24)
    else:           # u64 entries: high word count 1, 0 bits; low word symbols
        tab[: 8 * 4096].view(torch.int32).view(-1, 2)[:, 1].fill_(1 << 24)
    for checked in (False, True):
        out = dc.empty_output()
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        if checked:
            dfh.df_decompress_checked(dc, out, err)
        else:
            dfh.df_decompress(dc, out)
        torch.cuda.synchronize()
        say("damaged table", kind, "checked", checked, "err", int(err.item()))
        assert np.array_equal(host_of(out, kind), src)
        assert int(err.item()) == (dfh.DEVERR_CODE if checked else 0)


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_table_entries_that_hold_no_codes(torch_dev, orc, kind):
    """Every entry of the decoder-side table replaced from the host by one
    that claims no codes but carries other bits (a consumed-bit field, symbol
    bytes, start flags).  The library's tables hold zero there; the kernel
    clears such entries whole while staging the table, and its kept runs take
    a cleared entry as one that moves nothing, so every code takes the
    hierarchical tables (intact here): the output is still the input, with no
    error reported."""
    torch, dev = torch_dev
    n = 2_000_003
    if kind == 0:
        src = bf16_normal(n, 44)
        c = dfh.compress(0, src)
    elif kind == 1:
        src = u8_normal(n, 45, False)
        c = dfh.compress(1, src)
    else:
        q = u4_symbols(n, 46)
        src = synth.pack_u4(q)
        c = dfh.compress(2, src, n=n)
    dc = dfh.to_device(c, dev)
    tab = dc.sections["dtab"]
    if kind == 1:   # uint8: 8192 u32 pair entries, count 0, every other bit set
        tab[: 4 * 8192].view(torch.int32).fill_(0x00FFFFFF)
    else:           # u64 entries: high word count 0, other bits set; low word set
        w = tab[: 8 * 4096].view(torch.int32).view(-1, 2)
        w[:, 0].fill_(-1)
        w[:, 1].fill_(0x00FFFFFF)
    for checked in (False, True):
        out = dc.empty_output()
        err = torch.zeros(1, dtype=torch.int32, device=dev)
        if checked:
            dfh.df_decompress_checked(dc, out, err)
        else:
            dfh.df_decompress(dc, out)
        torch.cuda.synchronize()
        say("no-code table entries", kind, "checked", checked, "err", int(err.item()))
        assert np.array_equal(host_of(out, kind), src)
        assert int(err.item()) == 0
