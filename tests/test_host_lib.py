"""Host half of the product library (C ABI through the ctypes binding) against
the CPU oracle: same histograms, same code lengths, byte-identical sections,
decoder-side tables equal to their test-side definition (decoder_tables.py),
cross-decoding, container files and validation.  No GPU needed."""
import os
import re

import numpy as np
import pytest

import lossless_entropy_coded_huffman_amd as dfh
from decoder_tables import dtab_of
from lossless_entropy_coded_huffman_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SECTIONS = ["bitstream", "gaps", "tile_out", "sign_mantissa", "lut"]
EDGE_SIZES = [0, 1, 2, 63, 64, 65, 255, 256, 257, 6143, 16384, 16385, 100_003]


def header_functions():
    text = open(os.path.join(ROOT, "include", "dfh.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(df_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert "df_decompress" in names and "df_encode" in names and len(names) >= 13
    L = dfh.lib()
    for name in names:
        assert hasattr(L, name), name


def inputs(kind, n, seed, dist="normal"):
    """Host input of n elements; for uint4 the packed bytes."""
    rng = np.random.default_rng(seed)
    if kind == dfh.KIND_BF16:
        x = rng.standard_t(3, n) * 0.02 if dist == "t3" else rng.normal(0, 0.02, n)
        return synth.bf16_rne(x.astype(np.float32))
    x = rng.normal(0, 0.02, n).astype(np.float32)
    if kind == dfh.KIND_U4:
        return synth.pack_u4(synth.quantize_u4(x, bool(seed & 1)))
    return synth.quantize_u8(x, bool(seed & 1))


def decoded_of(kind, src, n):
    """What the decoder must return for an input (oracle's view for uint4:
    one symbol byte per element)."""
    return synth.unpack_u4(src, n) if kind == dfh.KIND_U4 else src


def lib_sections(c):
    return {k: np.asarray(c.section(k)) for k in dfh.SECTION_NAMES}


def as_oracle_container(c):
    inf = c.info()
    d = lib_sections(c)
    d.update(kind=inf["kind"], n=inf["n"], n_tiles=inf["n_tiles"], n_threads=inf["n_threads"],
             lengths=inf["lengths"])
    return d


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("n", EDGE_SIZES)
def test_sections_identical_to_oracle(orc, kind, n):
    src = inputs(kind, n, n + kind)
    nn = n if kind == dfh.KIND_U4 else None
    h = dfh.df_histogram(kind, src, nn)
    assert np.array_equal(h, orc.histogram(kind, src, nn))
    ln = dfh.df_build_codebook(h)
    assert np.array_equal(ln, orc.code_lengths(h))
    c = dfh.df_encode(kind, src, ln, nn)
    o = orc.encode(kind, src, ln, nn)
    o["lut"], o["n_luts"] = orc.build_lut(ln)
    inf = c.info()
    for k in ("n", "total_bits", "n_threads", "n_tiles", "max_tile_elems", "n_luts"):
        assert inf[k] == o[k], k
    got = lib_sections(c)
    for k in SECTIONS:
        if k == "sign_mantissa" and kind != 0:
            assert got[k].size == 0
            continue
        assert np.array_equal(got[k], o[k]), k
    assert np.array_equal(got["dtab"].view(np.uint8), dtab_of(kind, ln, orc.canonical_codes(ln)))
    c.validate()
    assert np.array_equal(orc.decode_tiles(as_oracle_container(c), 4), decoded_of(kind, src, n))


@pytest.mark.parametrize("seed", range(8))
def test_codebook_matches_oracle_random(orc, seed):
    rng = np.random.default_rng(1000 + seed)
    h = np.zeros(256, np.uint64)
    m = int(rng.integers(1, 257))
    h[rng.choice(256, m, replace=False)] = (rng.pareto(0.7, m) * 10 + 1).astype(np.uint64)
    assert np.array_equal(dfh.df_build_codebook(h), orc.code_lengths(h))
    for L in (12, 16, 24):
        if m <= 2 ** L:
            assert np.array_equal(dfh.df_build_codebook(h, L), orc.code_lengths(h, L))


def test_codebook_length_limited_fibonacci(orc):
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    h = np.zeros(256, np.uint64)
    h[100:140] = fib
    ln = dfh.df_build_codebook(h)
    assert ln.max() == 32
    assert np.array_equal(ln, orc.code_lengths(h))


def test_codebook_errors():
    with pytest.raises(dfh.DFError) as e:
        dfh.df_build_codebook(np.ones(256, np.uint64), 7)
    assert e.value.status == -3
    with pytest.raises(dfh.DFError) as e:
        dfh.df_build_codebook(np.ones(256, np.uint64), 33)
    assert e.value.status == -1


def test_encode_rejects_symbol_without_code():
    src = np.array([1, 2, 3], np.uint8)
    ln = np.zeros(256, np.uint8)
    ln[1] = ln[2] = 1
    with pytest.raises(dfh.DFError) as e:
        dfh.df_encode(dfh.KIND_U8, src, ln)
    assert e.value.status == -3


def test_encode_rejects_kraft_violation():
    ln = np.zeros(256, np.uint8)
    ln[:3] = 1
    with pytest.raises(dfh.DFError):
        dfh.df_encode(dfh.KIND_U8, np.zeros(4, np.uint8), ln)


def test_all_bf16_patterns(orc):
    u = np.random.default_rng(3).permutation(65536).astype(np.uint16)
    c = dfh.compress(dfh.KIND_BF16, u)
    o = orc.compress(dfh.KIND_BF16, u)
    for k in SECTIONS:
        assert np.array_equal(np.asarray(c.section(k)), o[k]), k
    assert np.array_equal(orc.decode_tiles(as_oracle_container(c), 2), u)


def test_heavy_tail_reaches_long_codes(orc):
    src = inputs(0, 2_000_000, 5, "t3")
    c = dfh.compress(0, src)
    inf = c.info()
    assert inf["lengths"].max() > 12          # exercises the long-code path
    o = orc.compress(0, src)
    for k in SECTIONS:
        assert np.array_equal(np.asarray(c.section(k)), o[k]), k


@pytest.mark.parametrize("kind", [0, 1, 2])
def test_save_load_round_trip(tmp_path, kind):
    src = inputs(kind, 50_001, 9)
    c = dfh.compress(kind, src, n=50_001 if kind == dfh.KIND_U4 else None)
    p = str(tmp_path / "c.dfh")
    c.save(p)
    c2 = dfh.df_container_load(p)
    for k in dfh.SECTION_NAMES:
        assert np.array_equal(np.asarray(c.section(k)), np.asarray(c2.section(k))), k
    assert c.info()["total_bits"] == c2.info()["total_bits"]
    assert c2.info()["kind"] == kind and c2.info()["n"] == 50_001


def test_u4_element_count_checks():
    p = inputs(dfh.KIND_U4, 10, 1)
    assert p.size == 5
    with pytest.raises(ValueError):
        dfh.compress(dfh.KIND_U4, p, n=11)       # more elements than nibbles
    with pytest.raises(ValueError):
        dfh.compress(dfh.KIND_U8, p, n=6)        # uint8: n must be the array size
    assert dfh.compress(dfh.KIND_U4, p).info()["n"] == 10
    assert dfh.output_bytes(dfh.KIND_U4, 11) == 6


def test_load_rejects_corrupt_files(tmp_path):
    src = inputs(1, 40_000, 4)
    c = dfh.compress(1, src)
    p = str(tmp_path / "c.dfh")
    c.save(p)
    raw = bytearray(open(p, "rb").read())
    # bad magic
    bad = bytearray(raw)
    bad[0] ^= 0xFF
    open(p + ".1", "wb").write(bad)
    with pytest.raises(dfh.DFError) as e:
        dfh.df_container_load(p + ".1")
    assert e.value.status == -4
    # truncated
    open(p + ".2", "wb").write(raw[: len(raw) // 2])
    with pytest.raises(dfh.DFError):
        dfh.df_container_load(p + ".2")
    # tile_out edited: find the tile_out section (third stored section)
    inf = c.info()
    sb = inf["section_bytes"]
    off = 64 + 256
    for name in ("bitstream", "gaps"):
        off += 64 + (sb[name] + 63) // 64 * 64
    off += 64
    bad = bytearray(raw)
    bad[off + 8: off + 16] = (inf["n"] + 5).to_bytes(8, "little")   # tile_out[1] > n
    open(p + ".3", "wb").write(bad)
    with pytest.raises(dfh.DFError) as e:
        dfh.df_container_load(p + ".3")
    assert e.value.status == -6
    # a length byte changed: Kraft no longer holds
    bad = bytearray(raw)
    first_used = 64 + int(np.nonzero(inf["lengths"])[0][0])
    bad[first_used] += 1
    open(p + ".4", "wb").write(bad)
    with pytest.raises(dfh.DFError):
        dfh.df_container_load(p + ".4")


def test_one_symbol_and_empty(orc):
    src = np.full(70_000, 0x3F80, np.uint16)
    c = dfh.compress(0, src)
    assert c.info()["total_bits"] == 70_000
    assert np.array_equal(orc.decode_tiles(as_oracle_container(c), 3), src)
    ln = c.info()["lengths"]
    assert np.array_equal(np.asarray(c.section("dtab")).view(np.uint8), dtab_of(0, ln, orc.canonical_codes(ln)))
    e = dfh.compress(1, np.zeros(0, np.uint8))
    assert e.info()["n_tiles"] == 0 and list(np.asarray(e.section("tile_out"))) == [0]


def test_forward_block_shape_matches_benchmark_block():
    from lossless_entropy_coded_huffman_amd import forward as fw, synth
    assert fw.LLAMA3_8B.matrices() == synth.LLAMA3_8B_BLOCK
    assert fw.LLAMA3_8B.elements() == synth.block_elems(synth.LLAMA3_8B_BLOCK) == 218_103_808


def test_encode_rejects_more_tables_than_the_cap(orc):
    # 96 codes of 7 bits and 128 of 9 bits (Kraft sum exactly 1): the 9-bit
    # codes spread over 64 distinct 8-bit prefixes, each needing a second
    # level table, so the code needs 65 tables (cap 64)
    ln = np.zeros(256, np.uint8)
    ln[:96] = 7
    ln[96:224] = 9
    assert sum(2.0 ** -int(l) for l in ln if l) == 1.0
    with pytest.raises(ValueError):
        orc.build_lut(ln, cap=64)
    assert orc.build_lut(ln, cap=65)[1] == 65
    src = np.arange(224, dtype=np.uint8)
    with pytest.raises(dfh.DFError) as e:
        dfh.df_encode(dfh.KIND_U8, src, ln)
    assert e.value.status == -3


@pytest.mark.parametrize("kind", [0, 1, 2])
@pytest.mark.parametrize("n", [0, 1, 65, 16385, 100_003])
def test_encode_layout_and_tables_match_the_encoder(kind, n):
    # the host calls that size a device encoding: same header scalars and
    # section sizes as the encoder's container, same LUT and DTAB
    src = inputs(kind, n, 7 + n)
    nn = n if kind == dfh.KIND_U4 else None
    c = dfh.compress(kind, src, n=nn)
    inf = c.info()
    h = dfh.df_histogram(kind, src, nn)
    sym = decoded_of(kind, src, n) if kind != 0 else ((src.view(np.uint16) >> 7) & 0xFF)
    lay = dfh.df_encode_layout(kind, n, h, int(sym[-1]) if n else 0, inf["lengths"])
    for k in ("n", "total_bits", "n_threads", "n_tiles", "n_luts"):
        assert getattr(lay, k) == inf[k], k
    assert [int(x) for x in lay.section_bytes] == [inf["section_bytes"][k] for k in dfh.SECTION_NAMES]
    if n:
        lut, nl, dtab = dfh.df_build_tables(kind, inf["lengths"])
        assert nl == inf["n_luts"]
        assert np.array_equal(lut, np.asarray(c.section("lut")))
        assert np.array_equal(dtab, np.asarray(c.section("dtab")))


def test_decompress_argument_checks_run_before_any_device_call():
    # the view checks are host-side: a view of 2^31 tiles (the kernels index
    # tiles in 32 bits) and inconsistent header scalars are rejected with
    # DF_ERR_ARG before the device is touched; no GPU needed
    import ctypes
    L = dfh.lib()
    fake = 1 << 20   # aligned, never dereferenced by the checks
    v = dfh.dfh.df_device_view()
    v.kind = dfh.KIND_U8
    v.n_luts = 1
    v.max_tile_elems = 100
    for name in ("bitstream", "gaps", "tile_out", "lut", "dtab"):
        setattr(v, name, fake)

    def call(n_tiles, n_threads, total_bits):
        v.n, v.n_tiles, v.n_threads, v.total_bits = 1000, n_tiles, n_threads, total_bits
        return L.df_decompress(ctypes.byref(v), ctypes.c_void_p(fake), ctypes.c_void_p(0))

    t = 1 << 31
    assert call(t, (t - 1) * 256 + 1, ((t - 1) * 256 + 1) * 64 - 10) == -1
    t = 3
    assert call(t, 1, 64) == -1                       # n_threads below (n_tiles - 1) * 256
    assert call(t, 2 * 256 + 1, 40) == -1             # total_bits below the last thread's start


def test_codebook_beyond_the_table_cap_is_refused():
    # one dominant byte value and every other value rare: the rare values'
    # long codes spread over more 8-bit prefixes than DF_MAX_LUTS tables
    # hold, so the codebook is refused (DF_ERR_CODEBOOK) rather than built
    # into a container the decoder cannot stage; with eight rare values the
    # same skew needs one table
    rng = np.random.default_rng(12)
    x = np.full(3_000_001, 131, np.uint8)
    pick = rng.random(x.size) < 0.005
    x[pick] = rng.integers(0, 256, int(pick.sum()))
    h = dfh.df_histogram(dfh.KIND_U8, x)
    with pytest.raises(dfh.DFError) as e:
        dfh.df_build_codebook(h)
    assert e.value.status == -3
    x[pick] = rng.integers(120, 128, int(pick.sum()))
    c = dfh.compress(dfh.KIND_U8, x)
    assert c.info()["n_luts"] == 1
