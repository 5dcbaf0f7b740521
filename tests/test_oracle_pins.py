"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- brute force over tiny alphabets, closed forms, a worked example
printed in RFC 1951, hand-derived streams, library routines (numpy bincount,
math.frexp, heapq) and invariants the pages state (lossless round trip,
gaps in [0, 31], codes decoded per chunk are those that start in it).
"""
import heapq
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def kraft(lengths):
    return sum(Fraction(1, 2 ** int(l)) for l in lengths if l)


def cost(hist, lengths):
    return sum(int(h) * int(l) for h, l in zip(hist, lengths))


def textbook_huffman_cost(weights):
    """Cost of an optimal prefix code = sum of the weights of all merged
    (internal) nodes of Huffman's construction."""
    w = [int(x) for x in weights if x]
    if len(w) == 1:
        return w[0]
    heapq.heapify(w)
    total = 0
    while len(w) > 1:
        a = heapq.heappop(w)
        b = heapq.heappop(w)
        total += a + b
        heapq.heappush(w, a + b)
    return total


def brute_min_cost(weights, max_len):
    """Minimum of sum w*l over all integer length vectors in [1, max_len]^m
    with Kraft sum <= 1 (vectorised enumeration, m <= 7)."""
    w = np.array(weights, np.int64)
    m = len(w)
    grids = np.meshgrid(*[np.arange(1, max_len + 1)] * m, indexing="ij")
    L = np.stack([g.reshape(-1) for g in grids], 1)
    ok = (np.ldexp(1.0, max_len - L)).sum(1) <= 2.0 ** max_len
    return int((L[ok] * w).sum(1).min())


def bf16_from_f32(x):
    b = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def code_strings(lengths, codes):
    return {s: format(int(codes[s]), "0%db" % int(lengths[s])) for s in range(256) if lengths[s]}


# ---------------------------------------------------------------- field split
def test_split_merge_all_bf16_patterns(orc):
    u = np.arange(65536, dtype=np.uint16)
    e, sm = orc.split_bf16(u)
    assert np.array_equal(orc.merge_bf16(e, sm), u)
    # independent reading of the fields: sign from the value's sign bit, the
    # exponent of normal numbers from math.frexp, the mantissa from the scaled
    # significand
    f32 = (u.astype(np.uint32) << 16).view(np.float32)
    for i in range(0, 65536, 97):
        v = float(f32[i])
        if not math.isfinite(v) or v == 0.0 or e[i] == 0:
            continue
        mant, ex = math.frexp(abs(v))          # |v| = mant * 2^ex, mant in [0.5, 1)
        assert e[i] == ex - 1 + 127
        assert (sm[i] >> 7) == (1 if math.copysign(1.0, v) < 0 else 0)
        assert (sm[i] & 0x7F) == round((mant * 2 - 1) * 128)


def test_histogram_matches_bincount(orc):
    rng = np.random.default_rng(1)
    u = bf16_from_f32(rng.normal(0, 0.02, 50_000))
    h = orc.histogram(orc.KIND_BF16, u)
    assert np.array_equal(h, np.bincount((u >> 7) & 0xFF, minlength=256).astype(np.uint64))
    b = rng.integers(0, 256, 30_000).astype(np.uint8)
    assert np.array_equal(orc.histogram(orc.KIND_U8, b), np.bincount(b, minlength=256))


# ----------------------------------------------------------- Huffman lengths
def test_closed_forms(orc):
    # 256 equal counts: every length is 8
    assert (orc.huffman_lengths(np.full(256, 7, np.uint64)) == 8).all()
    # dyadic counts: l = -log2 p exactly, mean length = entropy
    h = np.zeros(256, np.uint64)
    h[:5] = [8, 4, 2, 1, 1]
    assert list(orc.huffman_lengths(h)[:5]) == [1, 2, 3, 4, 4]
    # one used symbol: a one-bit code
    h = np.zeros(256, np.uint64)
    h[77] = 1000
    ln = orc.code_lengths(h)
    assert ln[77] == 1 and ln.sum() == 1
    # empty histogram: no codes
    assert orc.code_lengths(np.zeros(256, np.uint64)).sum() == 0


def test_tie_rule_leaves_first(orc):
    # counts a=1, b=1, c=2, d=2.  Merging the two smallest (weight, key) with
    # leaves keyed by symbol and internal nodes by 256 + creation index:
    # (a,b) -> N0 (2); then c (2, key 2) and d (2, key 3) beat N0 (2, key 256)
    # -> N1 (4); then N0 + N1.  All four lengths are 2.  Preferring internal
    # nodes on ties would give (3, 3, 2, 1) at the same cost.
    h = np.zeros(256, np.uint64)
    h[:4] = [1, 1, 2, 2]
    assert list(orc.huffman_lengths(h)[:4]) == [2, 2, 2, 2]


@pytest.mark.parametrize("seed", range(6))
def test_huffman_random_histograms(orc, seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(2, 256))
    h = np.zeros(256, np.uint64)
    syms = rng.choice(256, m, replace=False)
    h[syms] = rng.integers(1, 10_000, m) ** rng.integers(1, 3)
    ln = orc.huffman_lengths(h)
    assert kraft(ln) == 1
    assert cost(h, ln) == textbook_huffman_cost(h)
    p = h[h > 0].astype(np.float64) / h.sum()
    H = -(p * np.log2(p)).sum()
    Lbar = cost(h, ln) / int(h.sum())
    assert H - 1e-9 <= Lbar < H + 1


@pytest.mark.parametrize("seed", range(10))
def test_huffman_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(100 + seed)
    m = int(rng.integers(2, 8))
    w = rng.integers(1, 50, m)
    h = np.zeros(256, np.uint64)
    syms = np.sort(rng.choice(256, m, replace=False))
    h[syms] = w
    ln = orc.huffman_lengths(h)
    assert cost(h, ln) == brute_min_cost(w, m - 1)


@pytest.mark.parametrize("seed", range(10))
def test_limited_brute_force_tiny(orc, seed):
    rng = np.random.default_rng(200 + seed)
    m = int(rng.integers(3, 8))
    w = (rng.integers(1, 6, m) ** rng.integers(1, 5, m)).astype(np.int64)
    L = int(rng.integers(math.ceil(math.log2(m)), 7))
    h = np.zeros(256, np.uint64)
    syms = np.sort(rng.choice(256, m, replace=False))
    h[syms] = w
    ln = orc.limited_lengths(h, L)
    assert ln.max() <= L
    assert kraft(ln) == 1
    assert cost(h, ln) == brute_min_cost(w, L)


def test_fibonacci_forces_limit(orc):
    fib = [1, 1]
    while len(fib) < 40:
        fib.append(fib[-1] + fib[-2])
    h = np.zeros(256, np.uint64)
    h[:40] = fib
    plain = orc.huffman_lengths(h)
    assert plain.max() == 39                      # a chain: depth m - 1
    ln = orc.code_lengths(h, 32)
    assert ln.max() == 32
    assert kraft(ln) == 1
    assert cost(h, ln) >= cost(h, plain)
    # package-merge with a limit the plain code already meets changes nothing
    assert cost(h, orc.limited_lengths(h, 39)) == cost(h, plain)


def test_limit_too_small(orc):
    h = np.ones(256, np.uint64)
    with pytest.raises(ValueError):
        orc.code_lengths(h, 7)


# ------------------------------------------------------------ canonical codes
def test_rfc1951_worked_example(orc):
    rows = [ln.split() for ln in open(os.path.join(GOLDEN, "rfc1951_canonical_example.txt"))
            if ln.strip() and not ln.startswith("#")]
    lengths = np.zeros(256, np.uint8)
    for i, (_, l, _) in enumerate(rows):
        lengths[i] = int(l)
    codes = orc.canonical_codes(lengths)
    for i, (_, l, c) in enumerate(rows):
        assert format(int(codes[i]), "0%db" % int(l)) == c


def test_uniform_code_is_identity(orc):
    codes = orc.canonical_codes(np.full(256, 8, np.uint8))
    assert np.array_equal(codes, np.arange(256))


@pytest.mark.parametrize("seed", range(4))
def test_canonical_prefix_free_and_complete(orc, seed):
    rng = np.random.default_rng(300 + seed)
    h = np.zeros(256, np.uint64)
    m = int(rng.integers(2, 40))
    h[rng.choice(256, m, replace=False)] = rng.integers(1, 5000, m)
    ln = orc.code_lengths(h)
    strs = code_strings(ln, orc.canonical_codes(ln))
    vals = sorted(strs.values())
    for a, b in zip(vals, vals[1:]):
        assert not b.startswith(a)
    # completeness: every bit string of the longest length has exactly one
    # code as a prefix (checked by counting covered leaves)
    Lm = max(len(v) for v in vals)
    covered = sum(2 ** (Lm - len(v)) for v in vals)
    assert covered == 2 ** Lm


# ----------------------------------------------------------------- encoding
def test_dyadic_stream_golden(orc):
    fields = {}
    for ln in open(os.path.join(GOLDEN, "dyadic_stream.txt")):
        if ln.strip() and not ln.startswith("#"):
            k, *v = ln.split()
            fields[k] = v
    lengths = np.zeros(256, np.uint8)
    lengths[:5] = [int(x) for x in fields["lengths"]]
    seq = np.array([int(x) for x in fields["sequence"]], np.uint8)
    c = orc.encode(orc.KIND_U8, seq, lengths)
    expect = bytes(int(x, 16) for x in fields["stream_hex"])
    assert bytes(c["bitstream"][: len(expect)]) == expect
    assert not c["bitstream"][len(expect):].any()
    assert c["total_bits"] == int(fields["total_bits"][0])
    assert c["n_threads"] == 1 and c["n_tiles"] == 1
    assert list(c["tile_out"]) == [0, 5]
    assert c["gaps"][0] & 31 == 0


def test_uniform_stream_is_bit_reversed_bytes(orc):
    # 256 equal lengths of 8: code(s) = s, emitted most significant bit first
    # into a least-significant-bit-first stream, so each stream byte is s with
    # its bits reversed.
    rng = np.random.default_rng(5)
    seq = rng.integers(0, 256, 5000).astype(np.uint8)
    c = orc.encode(orc.KIND_U8, seq, np.full(256, 8, np.uint8))
    rev = np.array([int(format(s, "08b")[::-1], 2) for s in range(256)], np.uint8)
    assert np.array_equal(c["bitstream"][:5000], rev[seq])


def numpy_metadata(seq_lengths, n_tiles):
    """Gaps and tile_out from their definitions, vectorised."""
    starts = np.concatenate([[0], np.cumsum(seq_lengths)[:-1]]).astype(np.int64)
    n_threads = int(starts[-1] // 64 + 1)
    t = np.arange(n_threads, dtype=np.int64)
    first = starts[np.searchsorted(starts, 64 * t, side="left")]
    gaps = first - 64 * t
    tile_out = np.searchsorted(starts, 16384 * np.arange(n_tiles + 1), side="left")
    tile_out[-1] = len(starts)
    return n_threads, gaps, tile_out


def unpack_gaps(packed, count):
    bits = np.unpackbits(packed, bitorder="little")
    idx = 5 * np.arange(count)[:, None] + np.arange(5)[None, :]
    return (bits[idx] << np.arange(5)).sum(1)


@pytest.mark.parametrize("kind,n", [(0, 100_000), (1, 70_000), (0, 16385), (1, 1)])
def test_metadata_matches_definition(orc, kind, n):
    rng = np.random.default_rng(n)
    if kind == 0:
        src = bf16_from_f32(rng.standard_t(3, n) * 0.02)
        sym = (src >> 7) & 0xFF
    else:
        src = np.clip(np.rint(rng.normal(128, 12, n)), 0, 255).astype(np.uint8)
        sym = src
    c = orc.compress(kind, src)
    L = c["lengths"][sym].astype(np.int64)
    assert c["total_bits"] == L.sum()
    n_threads, gaps, tile_out = numpy_metadata(L, int(c["n_tiles"]))
    assert c["n_threads"] == n_threads
    assert c["n_tiles"] == -(-n_threads // 256)
    g = unpack_gaps(c["gaps"], int(c["n_tiles"]) * 256)
    assert np.array_equal(g[:n_threads], gaps)
    assert not g[n_threads:].any()
    assert g.max() <= 31
    assert np.array_equal(c["tile_out"].astype(np.int64), tile_out)
    assert c["max_tile_elems"] == np.diff(tile_out).max()
    if kind == 0:
        _, sm = orc.split_bf16(src)
        assert np.array_equal(c["sign_mantissa"][:n], sm)
        assert not c["sign_mantissa"][n:].any()


def test_empty_input(orc):
    for kind in (0, 1):
        src = np.zeros(0, np.uint16 if kind == 0 else np.uint8)
        c = orc.compress(kind, src)
        assert c["n"] == 0 and c["total_bits"] == 0 and c["n_threads"] == 0 and c["n_tiles"] == 0
        assert list(c["tile_out"]) == [0]
        assert orc.decode_serial(kind, c["lengths"], c["bitstream"], 0, c["sign_mantissa"]).size == 0
        assert orc.decode_tiles(c, 3).size == 0


# ------------------------------------------------------------ lookup tables
def walk(lut, stream_bits):
    """Walk the hierarchical tables over a bit sequence (first bit first)."""
    t, d = 0, 0
    while True:
        idx = sum(int(b) << k for k, b in enumerate(stream_bits[8 * d: 8 * d + 8]))
        e = int(lut[t * 256 + idx])
        if e == 0xFFFF:
            return None
        if e & 0x8000:
            t, d = e & 0x7FFF, d + 1
            continue
        return e & 0xFF, e >> 8


@pytest.mark.parametrize("kind,seed", [(0, 0), (0, 1), (1, 2), (1, 3)])
def test_lut_walk(orc, kind, seed):
    rng = np.random.default_rng(400 + seed)
    if kind == 0:
        src = bf16_from_f32(rng.standard_t(3, 400_000) * 0.02)
    else:
        src = np.clip(np.rint(rng.normal(128, 20, 200_000)), 0, 255).astype(np.uint8)
    c = orc.compress(kind, src)
    ln, lut, nl = c["lengths"], c["lut"], c["n_luts"]
    strs = code_strings(ln, orc.canonical_codes(ln))
    assert 1 <= nl <= 64
    for s, code in strs.items():
        for _ in range(8):
            suffix = "".join(rng.choice(["0", "1"], 32))
            assert walk(lut, [int(b) for b in code + suffix]) == (s, len(code))
    # every entry is a leaf, a pointer to a later table, or (never, for a
    # complete code) the "no code" marker
    e = lut.astype(np.int64)
    assert not (e == 0xFFFF).any()
    ptr = e[(e & 0x8000) != 0] & 0x7FFF
    assert ptr.min(initial=nl) >= 1 and ptr.max(initial=0) < nl
    # breadth-first numbering: pointers met in table order number 1, 2, ...
    assert list(ptr) == list(range(1, nl))


def test_lut_one_symbol(orc):
    h = np.zeros(256, np.uint64)
    h[9] = 5
    lut, nl = orc.build_lut(orc.code_lengths(h))
    assert nl == 1
    even = lut[0::2]
    assert (even == (1 << 8 | 9)).all() and (lut[1::2] == 0xFFFF).all()


# ------------------------------------------------------------------ decoding
def python_decode(strs, bits, n):
    inv = {v: k for k, v in strs.items()}
    out, cur = [], ""
    for b in bits:
        cur += b
        if cur in inv:
            out.append(inv[cur])
            cur = ""
            if len(out) == n:
                break
    return out


@pytest.mark.parametrize("kind,n,seed", [(0, 3000, 0), (1, 2500, 1), (0, 1, 2), (1, 17, 3)])
def test_decode_against_python_prefix_matcher(orc, kind, n, seed):
    rng = np.random.default_rng(500 + seed)
    if kind == 0:
        src = bf16_from_f32(rng.normal(0, 0.03, n))
        sym = (src >> 7) & 0xFF
    else:
        src = rng.integers(100, 160, n).astype(np.uint8)
        sym = src
    c = orc.compress(kind, src)
    strs = code_strings(c["lengths"], orc.canonical_codes(c["lengths"]))
    bits = "".join(str(b) for b in np.unpackbits(c["bitstream"], bitorder="little"))
    assert python_decode(strs, bits, n) == list(sym)
    out = orc.decode_serial(kind, c["lengths"], c["bitstream"], n, c["sign_mantissa"])
    assert np.array_equal(out, src)


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("threads", [1, 3, 8])
def test_decode_tiles_round_trip(orc, kind, threads):
    rng = np.random.default_rng(7 + kind)
    n = 300_001
    if kind == 0:
        src = bf16_from_f32(rng.normal(0, 0.02, n))
    else:
        src = np.clip(np.rint(rng.normal(128, 9, n)), 0, 255).astype(np.uint8)
    c = orc.compress(kind, src)
    assert c["n_tiles"] > 8
    assert np.array_equal(orc.decode_tiles(c, threads), src)


def test_all_bf16_patterns_round_trip(orc):
    u = np.random.default_rng(11).permutation(np.arange(65536, dtype=np.uint32)).astype(np.uint16)
    c = orc.compress(orc.KIND_BF16, u)
    assert np.array_equal(orc.decode_tiles(c, 4), u)
    assert np.array_equal(orc.decode_serial(0, c["lengths"], c["bitstream"], u.size,
                                            c["sign_mantissa"]), u)


def test_single_symbol_round_trip(orc):
    for n in (1, 64, 65, 16384, 16385, 40000):
        src = np.full(n, 0x3C80, np.uint16)       # one exponent value
        c = orc.compress(0, src)
        assert c["total_bits"] == n
        assert np.array_equal(orc.decode_tiles(c, 2), src)


def test_corruption_changes_output(orc):
    # a complete prefix code decodes any bit string, so a flipped stream bit
    # shows up as different output (or an undecodable tail), never silently
    rng = np.random.default_rng(12)
    src = bf16_from_f32(rng.normal(0, 0.02, 20000))
    c = orc.compress(0, src)
    c["bitstream"][100] ^= 0x10
    try:
        out = orc.decode_serial(0, c["lengths"], c["bitstream"], src.size, c["sign_mantissa"])
        assert not np.array_equal(out, src)
    except ValueError:
        pass


def test_tile_range_decode_matches_whole(orc):
    rng = np.random.default_rng(21)
    src = bf16_from_f32(rng.normal(0, 0.02, 200_000))
    c = orc.compress(0, src)
    nt = int(c["n_tiles"])
    for b0, b1 in ((0, 1), (3, 7), (nt - 2, nt), (0, nt)):
        part = orc.decode_tile_range(c, b0, b1)
        lo, hi = int(c["tile_out"][b0]), int(c["tile_out"][b1])
        assert np.array_equal(part, src[lo:hi])


# ------------------------------------------------------------- uint4 (EntroLLM)
def np_pack_u4(s):
    """Independent packing: element 2j in the low nibble of byte j."""
    s = np.asarray(s, np.uint8)
    if s.size % 2:
        s = np.concatenate([s, np.zeros(1, np.uint8)])
    return (s[0::2] | (s[1::2] << 4)).astype(np.uint8)


@pytest.mark.parametrize("n", [1, 2, 3, 16, 17, 1000, 1001])
def test_u4_pack_and_histogram(orc, n):
    rng = np.random.default_rng(n)
    s = rng.integers(0, 16, n).astype(np.uint8)
    packed = orc.pack_u4(s)
    assert np.array_equal(packed, np_pack_u4(s))
    h = orc.histogram(orc.KIND_U4, packed, n)
    assert np.array_equal(h[:16], np.bincount(s, minlength=16)) and h[16:].sum() == 0
    with pytest.raises(ValueError):
        orc.pack_u4(np.array([16], np.uint8))


@pytest.mark.parametrize("n", [1, 2, 5, 255, 16383, 16384, 16385, 60001, 150_000])
def test_u4_sections_equal_u8_of_the_same_symbols(orc, n):
    # the uint4 kind differs from uint8 only in where a symbol is read from, so
    # with the same lengths every section must be the same as for the unpacked
    # symbols coded as uint8
    rng = np.random.default_rng(100 + n)
    q = np.clip(np.rint(rng.normal(7.5, 2.2, n)), 0, 15).astype(np.uint8)
    packed = np_pack_u4(q)
    if n % 2:
        packed[-1] |= 0xA0          # the unused high nibble must be ignored
    c4 = orc.compress(orc.KIND_U4, packed, n=n)
    c8 = orc.encode(orc.KIND_U8, q, c4["lengths"])
    for k in ("bitstream", "gaps", "tile_out"):
        assert np.array_equal(c4[k], c8[k]), k
    assert (c4["n"], c4["total_bits"], c4["n_tiles"]) == (c8["n"], c8["total_bits"], c8["n_tiles"])
    assert max(c4["lengths"]) <= 15          # 16 symbols: depth at most 15
    d = orc.decode_tiles(c4, 4)
    assert np.array_equal(d, q)
    assert np.array_equal(orc.decode_serial(orc.KIND_U4, c4["lengths"], c4["bitstream"], n), q)
    assert np.array_equal(orc.pack_u4(d), np_pack_u4(q))
