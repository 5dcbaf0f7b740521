"""CPU oracle -- TEST INFRASTRUCTURE ONLY.

Plain, slow, scalar C implementation (``oracle.c``) of lossless Huffman coding
of LLM weights, wrapped with ctypes.  Only the test suite,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  It shares no code with the product library
(``lossless_entropy_coded_huffman_amd``), and the product never imports it.

What it computes (sources by page title and section heading):

* DFloat11 (the pt.news.hada.io digest "DFloat11: compressao sem perda para
  inferencia em GPU..." and the abstract page "70% Size, 100% Accuracy..."):
  the BF16 exponent byte is Huffman coded ("O formato DFloat11"), sign and
  mantissa stay raw; per-thread gaps and per-block output positions
  ("Kernel de GPU em 2 etapas e metadados auxiliares"); hierarchical 256-entry
  tables ("Decodificacao com LUT hierarquica").
* EntroLLM ("EntroLLM: Entropy Encoded Weight Compression...", section
  "Metodologia"): Huffman coding of whole uint8 codes, and of uint4 codes as a
  16-symbol alphabet (packed two per byte, element 2j in the low nibble of
  byte j), decoded in parallel on CPU threads.  For uint4 the decoders return
  one symbol byte per element; ``pack_u4`` packs them.

Every function here has pins in ``tests/test_oracle_*.py`` that do not rely on
the oracle itself (brute force, closed forms, invariants, round trips).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

KIND_BF16 = 0
KIND_U8 = 1
KIND_U4 = 2
MAX_LEN = 32

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB = os.path.join(_BUILD, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/_build/liboracle.so."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-shared", "-fPIC",
                               "-pthread", _SRC, "-o", tmp])
        os.replace(tmp, _LIB)
    return _LIB


class _Layout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_uint64) for name in (
        "n", "total_bits", "n_threads", "n_tiles", "bitstream_bytes", "gaps_bytes",
        "tile_out_entries", "sm_bytes", "max_tile_elems")]


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        U64 = ctypes.c_uint64
        I = ctypes.c_int
        sig = {
            "oracle_split_bf16": (I, [P, U64, P, P]),
            "oracle_merge_bf16": (I, [P, P, U64, P]),
            "oracle_histogram": (I, [I, P, U64, P]),
            "oracle_huffman_lengths": (I, [P, P]),
            "oracle_limited_lengths": (I, [P, I, P]),
            "oracle_code_lengths": (I, [P, I, P]),
            "oracle_canonical_codes": (I, [P, P]),
            "oracle_layout": (I, [I, P, U64, P, ctypes.POINTER(_Layout)]),
            "oracle_encode": (I, [I, P, U64, P, ctypes.POINTER(_Layout), P, P, P, P]),
            "oracle_build_lut": (I, [P, P, I, ctypes.POINTER(I)]),
            "oracle_decode_serial": (I, [I, P, P, U64, U64, P, P]),
            "oracle_decode_tiles": (I, [I, P, P, U64, P, P, U64, U64, P, P, I]),
            "oracle_decode_tile_range": (I, [I, P, P, U64, P, P, U64, U64, U64, P, P]),
            "oracle_pack_u4": (I, [P, U64, P]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _src(kind: int, src) -> np.ndarray:
    dt = np.uint16 if kind == KIND_BF16 else np.uint8
    a = np.ascontiguousarray(src)
    if a.dtype != dt:
        a = a.view(dt) if a.dtype.itemsize == np.dtype(dt).itemsize else a.astype(dt)
    return a.reshape(-1)


def split_bf16(w) -> tuple[np.ndarray, np.ndarray]:
    """BF16 bit patterns (uint16) -> (exponent bytes, sign|mantissa bytes)."""
    w = _src(KIND_BF16, w)
    e = np.empty(w.size, np.uint8)
    sm = np.empty(w.size, np.uint8)
    _load().oracle_split_bf16(_ptr(w), w.size, _ptr(e), _ptr(sm))
    return e, sm


def merge_bf16(e, sm) -> np.ndarray:
    e = np.ascontiguousarray(e, np.uint8)
    sm = np.ascontiguousarray(sm, np.uint8)
    out = np.empty(e.size, np.uint16)
    _load().oracle_merge_bf16(_ptr(e), _ptr(sm), e.size, _ptr(out))
    return out


def _count(kind: int, a: np.ndarray, n: int | None) -> int:
    """Elements in src: its size, or for uint4 (packed bytes) n, default 2 per byte."""
    if kind != KIND_U4:
        return a.size
    n = 2 * a.size if n is None else int(n)
    if (n + 1) // 2 > a.size:
        raise ValueError("uint4 input shorter than n elements")
    return n


def pack_u4(syms) -> np.ndarray:
    """Symbols 0..15, one per byte -> packed bytes (element 2j in the low nibble)."""
    a = np.ascontiguousarray(syms, np.uint8).reshape(-1)
    out = np.zeros((a.size + 1) // 2, np.uint8)
    if _load().oracle_pack_u4(_ptr(a), a.size, _ptr(out)) != 0:
        raise ValueError("symbol above 15")
    return out


def histogram(kind: int, src, n: int | None = None) -> np.ndarray:
    a = _src(kind, src)
    h = np.zeros(256, np.uint64)
    if _load().oracle_histogram(kind, _ptr(a), _count(kind, a, n), _ptr(h)) != 0:
        raise ValueError("bad kind")
    return h


def huffman_lengths(hist) -> np.ndarray:
    """Unlimited Huffman code lengths (int32, may exceed 32)."""
    h = np.ascontiguousarray(hist, np.uint64)
    out = np.zeros(256, np.int32)
    _load().oracle_huffman_lengths(_ptr(h), _ptr(out))
    return out


def limited_lengths(hist, max_len: int) -> np.ndarray:
    """Optimal max_len-limited lengths by package-merge (int32)."""
    h = np.ascontiguousarray(hist, np.uint64)
    out = np.zeros(256, np.int32)
    if _load().oracle_limited_lengths(_ptr(h), int(max_len), _ptr(out)) < 0:
        raise ValueError("max_len too small for the alphabet")
    return out


def code_lengths(hist, max_len: int = MAX_LEN) -> np.ndarray:
    """Codebook policy: plain Huffman if it fits max_len, else package-merge."""
    h = np.ascontiguousarray(hist, np.uint64)
    out = np.zeros(256, np.uint8)
    if _load().oracle_code_lengths(_ptr(h), int(max_len), _ptr(out)) < 0:
        raise ValueError("max_len too small for the alphabet")
    return out


def canonical_codes(lengths) -> np.ndarray:
    ln = np.ascontiguousarray(lengths, np.uint8)
    out = np.zeros(256, np.uint32)
    if _load().oracle_canonical_codes(_ptr(ln), _ptr(out)) != 0:
        raise ValueError("length above 32")
    return out


def encode(kind: int, src, lengths, n: int | None = None) -> dict:
    """Encode with the given lengths.  Returns a dict with the scalars
    n, total_bits, n_threads, n_tiles, max_tile_elems and the sections
    bitstream, gaps, tile_out, sign_mantissa (None unless BF16)."""
    lib = _load()
    a = _src(kind, src)
    n = _count(kind, a, n)
    ln = np.ascontiguousarray(lengths, np.uint8)
    lay = _Layout()
    if lib.oracle_layout(kind, _ptr(a), n, _ptr(ln), ctypes.byref(lay)) != 0:
        raise ValueError("a symbol of the input has no code")
    bs = np.zeros(lay.bitstream_bytes, np.uint8)
    gaps = np.zeros(lay.gaps_bytes, np.uint8)
    tile_out = np.zeros(lay.tile_out_entries, np.uint64)
    sm = np.zeros(lay.sm_bytes, np.uint8) if kind == KIND_BF16 else None
    rc = lib.oracle_encode(kind, _ptr(a), n, _ptr(ln), ctypes.byref(lay), _ptr(bs),
                           _ptr(gaps), _ptr(tile_out), _ptr(sm))
    if rc != 0:
        raise RuntimeError("oracle_encode failed: %d" % rc)
    return dict(kind=kind, n=lay.n, total_bits=lay.total_bits, n_threads=lay.n_threads,
                n_tiles=lay.n_tiles, max_tile_elems=lay.max_tile_elems, lengths=ln.copy(),
                bitstream=bs, gaps=gaps, tile_out=tile_out, sign_mantissa=sm)


def build_lut(lengths, cap: int = 64) -> tuple[np.ndarray, int]:
    ln = np.ascontiguousarray(lengths, np.uint8)
    lut = np.zeros(cap * 256, np.uint16)
    n = ctypes.c_int(0)
    if _load().oracle_build_lut(_ptr(ln), _ptr(lut), int(cap), ctypes.byref(n)) != 0:
        raise ValueError("more than %d tables" % cap)
    return lut[: n.value * 256].copy(), n.value


def compress(kind: int, src, max_len: int = MAX_LEN, n: int | None = None) -> dict:
    """histogram -> lengths -> encode -> hierarchical tables, all by the oracle."""
    h = histogram(kind, src, n)
    ln = code_lengths(h, max_len)
    c = encode(kind, src, ln, n)
    c["lut"], c["n_luts"] = build_lut(ln)
    c["hist"] = h
    return c


def decode_serial(kind: int, lengths, bitstream, n: int, sign_mantissa=None) -> np.ndarray:
    """Bit-serial canonical decode of n codes from the start of the stream."""
    ln = np.ascontiguousarray(lengths, np.uint8)
    bs = np.ascontiguousarray(bitstream, np.uint8)
    out = np.empty(n, np.uint16 if kind == KIND_BF16 else np.uint8)
    sm = None if kind != KIND_BF16 else np.ascontiguousarray(sign_mantissa, np.uint8)
    if kind == KIND_BF16 and (sm is None or sm.size < n):
        raise ValueError("sign_mantissa too short")
    if _load().oracle_decode_serial(kind, _ptr(ln), _ptr(bs), bs.size, n, _ptr(sm), _ptr(out)) != 0:
        raise ValueError("undecodable stream")
    return out


def decode_tiles(c: dict, cpu_threads: int = 1, out: np.ndarray | None = None) -> np.ndarray:
    """Decode a container over tile ranges on cpu_threads CPU threads, using its
    gaps and tile_out to find each range's start."""
    kind = int(c["kind"])
    n = int(c["n"])
    if out is None:
        out = np.empty(n, np.uint16 if kind == KIND_BF16 else np.uint8)
    ln = np.ascontiguousarray(c["lengths"], np.uint8)
    bs = np.ascontiguousarray(c["bitstream"], np.uint8)
    gaps = np.ascontiguousarray(c["gaps"], np.uint8)
    to = np.ascontiguousarray(c["tile_out"], np.uint64)
    sm = None if kind != KIND_BF16 else np.ascontiguousarray(c["sign_mantissa"], np.uint8)
    rc = _load().oracle_decode_tiles(kind, _ptr(ln), _ptr(bs), bs.size, _ptr(gaps), _ptr(to),
                                     int(c["n_tiles"]), int(c["n_threads"]), _ptr(sm), _ptr(out),
                                     int(cpu_threads))
    if rc != 0:
        raise ValueError("undecodable stream")
    return out


def decode_tile_range(c: dict, b0: int, b1: int) -> np.ndarray:
    """Decode tiles [b0, b1) of a container (one CPU thread); returns the
    elements tile_out[b0] .. tile_out[b1] - 1.  For sampled checks of
    containers too large to decode whole."""
    kind = int(c["kind"])
    to = np.ascontiguousarray(c["tile_out"], np.uint64)
    lo, hi = int(to[b0]), int(to[b1])
    out = np.empty(hi - lo, np.uint16 if kind == KIND_BF16 else np.uint8)
    ln = np.ascontiguousarray(c["lengths"], np.uint8)
    bs = np.ascontiguousarray(c["bitstream"], np.uint8)
    gaps = np.ascontiguousarray(c["gaps"], np.uint8)
    sm = None if kind != KIND_BF16 else np.ascontiguousarray(c["sign_mantissa"], np.uint8)
    # dst points lo elements before the buffer so that element i lands at i - lo;
    # the worker writes only indices in [lo, hi)
    esz = out.itemsize
    base = out.ctypes.data - lo * esz
    rc = _load().oracle_decode_tile_range(kind, _ptr(ln), _ptr(bs), bs.size, _ptr(gaps), _ptr(to),
                                          int(b0), int(b1), int(c["n_threads"]), _ptr(sm),
                                          ctypes.c_void_p(base))
    if rc != 0:
        raise ValueError("undecodable stream")
    return out
