"""ctypes binding of libdfh (include/dfh.h), with the same names.

Argument marshalling only: every step of encoding runs in the C++ host
library and every step of decompression in the HIP kernels.  PyTorch
provides device memory and streams.  The library is loaded after torch so
that it binds to the HIP runtime torch has loaded (same soname), and the
binding refuses to run without the built library: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np
import torch  # noqa: F401  (loads the HIP runtime libdfh binds to)

KIND_BF16 = 0
KIND_U8 = 1
KIND_U4 = 2   # two elements per byte, element 2j in the low nibble of byte j
SEC_BITSTREAM, SEC_GAPS, SEC_TILE_OUT, SEC_SIGN_MANTISSA, SEC_LUT, SEC_DTAB = range(6)
SECTION_NAMES = ("bitstream", "gaps", "tile_out", "sign_mantissa", "lut", "dtab")
MAX_LEN = 32
DEVERR_COUNT = 1
DEVERR_CODE = 2

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "_build", "libdfh.so")


class DFError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__("%s: %s (%d)" % (what or "dfh", df_status_string(status), status))


class df_info(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("max_len", ctypes.c_uint32),
                ("n", ctypes.c_uint64), ("total_bits", ctypes.c_uint64),
                ("n_threads", ctypes.c_uint64), ("n_tiles", ctypes.c_uint64),
                ("n_luts", ctypes.c_uint32), ("max_tile_elems", ctypes.c_uint32),
                ("bytes_per_thread", ctypes.c_uint32), ("threads_per_tile", ctypes.c_uint32),
                ("section_bytes", ctypes.c_uint64 * 6), ("lengths", ctypes.c_uint8 * 256)]


class df_device_view(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int), ("n_luts", ctypes.c_uint32),
                ("max_tile_elems", ctypes.c_uint32), ("max_workgroups", ctypes.c_uint32),
                ("n", ctypes.c_uint64), ("total_bits", ctypes.c_uint64),
                ("n_threads", ctypes.c_uint64), ("n_tiles", ctypes.c_uint64),
                ("bitstream", ctypes.c_void_p), ("gaps", ctypes.c_void_p),
                ("tile_out", ctypes.c_void_p), ("sign_mantissa", ctypes.c_void_p),
                ("lut", ctypes.c_void_p), ("dtab", ctypes.c_void_p)]


_lib = None
_lock = threading.Lock()

# name -> (restype, argtypes); the exported C ABI
_SIGNATURES = {
    "df_histogram_device": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                           ctypes.c_void_p]),
    "df_symbol_device": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p]),
    "df_encode_layout": (ctypes.c_int, [ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint8,
                                        ctypes.c_void_p, ctypes.c_void_p]),
    "df_build_tables": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint32,
                                       ctypes.POINTER(ctypes.c_uint32), ctypes.c_void_p]),
    "df_encode_workspace_bytes": (ctypes.c_uint64, [ctypes.c_uint64]),
    "df_encode_device": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "df_encode_device_noalloc": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "df_histogram": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
    "df_build_codebook": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_void_p]),
    "df_encode": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                 ctypes.POINTER(ctypes.c_void_p)]),
    "df_container_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(df_info)]),
    "df_container_section": (ctypes.c_void_p, [ctypes.c_void_p, ctypes.c_int,
                                               ctypes.POINTER(ctypes.c_uint64)]),
    "df_container_save": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_char_p]),
    "df_container_load": (ctypes.c_int, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p)]),
    "df_container_validate": (ctypes.c_int, [ctypes.c_void_p]),
    "df_container_free": (None, [ctypes.c_void_p]),
    "df_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "df_decompress": (ctypes.c_int, [ctypes.POINTER(df_device_view), ctypes.c_void_p, ctypes.c_void_p]),
    "df_decompress_checked": (ctypes.c_int, [ctypes.POINTER(df_device_view), ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p]),
    "df_decompress_batch": (ctypes.c_int, [ctypes.POINTER(df_device_view),
                                           ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint32,
                                           ctypes.c_void_p]),
}


def lib():
    """The loaded libdfh.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError("libdfh.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
            L = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(L, name)
                fn.restype = res
                fn.argtypes = args
            _lib = L
        return _lib


def df_status_string(status: int) -> str:
    return lib().df_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise DFError(status, what)


def _host_array(kind: int, src) -> np.ndarray:
    if isinstance(src, torch.Tensor):
        src = src.detach().cpu()
        src = src.view(torch.int16).numpy() if src.dtype == torch.bfloat16 else src.numpy()
    a = np.ascontiguousarray(src).reshape(-1)
    want = np.uint16 if kind == KIND_BF16 else np.uint8
    if a.dtype != want:
        if a.dtype.itemsize != np.dtype(want).itemsize:
            raise TypeError("kind %d needs %s elements, got %s" % (kind, np.dtype(want), a.dtype))
        a = a.view(want)
    return a


def _elements(kind: int, a: np.ndarray, n) -> int:
    """Element count of a host array: its size, or for uint4 (packed bytes) n,
    by default two per byte."""
    if kind != KIND_U4:
        if n is not None and int(n) != a.size:
            raise ValueError("n is only given for uint4 input")
        return a.size
    n = 2 * a.size if n is None else int(n)
    if n < 0 or (n + 1) // 2 > a.size:
        raise ValueError("uint4 input holds fewer than n elements")
    return n


def output_bytes(kind: int, n: int) -> int:
    """Bytes of a decoded container of n elements."""
    return 2 * n if kind == KIND_BF16 else n if kind == KIND_U8 else (n + 1) // 2


# ------------------------------------------------------------------- host API
def df_histogram(kind: int, src, n=None) -> np.ndarray:
    a = _host_array(kind, src)
    h = np.zeros(256, np.uint64)
    _check(lib().df_histogram(kind, a.ctypes.data, _elements(kind, a, n), h.ctypes.data), "df_histogram")
    return h


def df_build_codebook(hist, max_len: int = MAX_LEN) -> np.ndarray:
    h = np.ascontiguousarray(hist, np.uint64)
    out = np.zeros(256, np.uint8)
    _check(lib().df_build_codebook(h.ctypes.data, int(max_len), out.ctypes.data), "df_build_codebook")
    return out


class Container:
    """A library-owned container (df_container*)."""

    def __init__(self, handle: int):
        self._h = ctypes.c_void_p(handle)

    @property
    def handle(self):
        if not self._h:
            raise ValueError("container was freed")
        return self._h

    def info(self) -> dict:
        return df_container_info(self)

    def section(self, sec) -> np.ndarray:
        return df_container_section(self, sec)

    def validate(self):
        df_container_validate(self)

    def save(self, path: str):
        df_container_save(self, path)

    def free(self):
        if self._h:
            lib().df_container_free(self._h)
            self._h = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.free()
        except Exception:
            pass


def df_encode(kind: int, src, lengths, n=None) -> Container:
    a = _host_array(kind, src)
    ln = np.ascontiguousarray(lengths, np.uint8)
    out = ctypes.c_void_p()
    _check(lib().df_encode(kind, a.ctypes.data if a.size else None, _elements(kind, a, n),
                           ln.ctypes.data, ctypes.byref(out)), "df_encode")
    return Container(out.value)


def df_container_info(c: Container) -> dict:
    inf = df_info()
    _check(lib().df_container_info(c.handle, ctypes.byref(inf)), "df_container_info")
    d = {k: getattr(inf, k) for k, _ in df_info._fields_ if k not in ("section_bytes", "lengths")}
    d["section_bytes"] = {SECTION_NAMES[i]: int(inf.section_bytes[i]) for i in range(6)}
    d["lengths"] = np.frombuffer(bytes(inf.lengths), np.uint8).copy()
    return d


_SEC_DTYPE = {SEC_TILE_OUT: np.uint64, SEC_LUT: np.uint16, SEC_DTAB: np.uint64}


def _section_bytes(c: Container, sec: int) -> np.ndarray:
    """uint8 view of a section's bytes in library memory (no copy)."""
    nbytes = ctypes.c_uint64(0)
    ptr = lib().df_container_section(c.handle, int(sec), ctypes.byref(nbytes))
    if ptr is None:
        raise DFError(-1, "df_container_section")
    raw = (ctypes.c_uint8 * max(int(nbytes.value), 1)).from_address(ptr)
    return np.frombuffer(raw, np.uint8, count=int(nbytes.value))


def df_container_section(c: Container, sec) -> np.ndarray:
    """Read-only numpy view of a section, valid while the container lives."""
    if isinstance(sec, str):
        sec = SECTION_NAMES.index(sec)
    arr = _section_bytes(c, int(sec)).view(_SEC_DTYPE.get(int(sec), np.uint8))
    arr.flags.writeable = False
    # keep the container alive as long as the view
    return _Owned(arr, c)


class _Owned(np.ndarray):
    def __new__(cls, arr, owner):
        obj = arr.view(cls)
        obj._owner = owner
        return obj

    def __array_finalize__(self, obj):
        self._owner = getattr(obj, "_owner", None)


def df_container_save(c: Container, path: str):
    _check(lib().df_container_save(c.handle, os.fsencode(path)), "df_container_save")


def df_container_load(path: str) -> Container:
    out = ctypes.c_void_p()
    _check(lib().df_container_load(os.fsencode(path), ctypes.byref(out)), "df_container_load")
    return Container(out.value)


def df_container_validate(c: Container):
    _check(lib().df_container_validate(c.handle), "df_container_validate")


def df_container_free(c: Container):
    c.free()


def compress(kind: int, src, max_len: int = MAX_LEN, n=None) -> Container:
    """df_histogram -> df_build_codebook -> df_encode.  For uint4, src is the
    packed bytes and n the element count (default: two per byte)."""
    a = _host_array(kind, src)
    return df_encode(kind, a, df_build_codebook(df_histogram(kind, a, n), max_len), n)


# ----------------------------------------------------------------- device API
class DeviceContainer:
    """A container's sections copied to device memory (torch uint8 tensors)
    and the df_device_view that borrows them."""

    def __init__(self, c: Container | None, device="cuda", _info=None, _sections=None):
        if c is None:   # sections already on the device (compress_device)
            inf, self.sections = _info, _sections
            self.device = torch.device(device)
        else:
            inf = c.info()
            self.device = torch.device(device)
            self.sections = {}
            for i, name in enumerate(SECTION_NAMES):
                host = _section_bytes(c, i)
                t = torch.empty(max(host.size, 16), dtype=torch.uint8, device=self.device)
                if host.size:
                    t[: host.size].copy_(torch.from_numpy(host), non_blocking=False)
                self.sections[name] = t
        self.kind = int(inf["kind"])
        self.n = int(inf["n"])
        self.info = inf
        v = df_device_view()
        v.kind = self.kind
        v.n_luts = inf["n_luts"]
        v.max_tile_elems = inf["max_tile_elems"]
        v.n = inf["n"]
        v.total_bits = inf["total_bits"]
        v.n_threads = inf["n_threads"]
        v.n_tiles = inf["n_tiles"]
        v.bitstream = self.sections["bitstream"].data_ptr()
        v.gaps = self.sections["gaps"].data_ptr()
        v.tile_out = self.sections["tile_out"].data_ptr()
        v.sign_mantissa = self.sections["sign_mantissa"].data_ptr() if self.kind == KIND_BF16 else None
        v.lut = self.sections["lut"].data_ptr()
        v.dtab = self.sections["dtab"].data_ptr()
        self.view = v

    def compressed_bytes(self) -> int:
        """Bytes of the stored sections (every section but the derived DTAB)."""
        return sum(v for k, v in self.info["section_bytes"].items() if k != "dtab")

    def empty_output(self) -> torch.Tensor:
        if self.kind == KIND_BF16:
            return torch.empty(self.n, dtype=torch.bfloat16, device=self.device)
        return torch.empty(output_bytes(self.kind, self.n), dtype=torch.uint8, device=self.device)


def to_device(c: Container, device="cuda") -> DeviceContainer:
    return DeviceContainer(c, device)


# ------------------------------------------------------- device encoding
def _info_dict(inf: df_info) -> dict:
    d = {k: getattr(inf, k) for k, _ in df_info._fields_ if k not in ("section_bytes", "lengths")}
    d["section_bytes"] = {name: int(inf.section_bytes[i]) for i, name in enumerate(SECTION_NAMES)}
    d["lengths"] = np.frombuffer(bytes(inf.lengths), np.uint8).copy()
    return d


def _device_elements(kind: int, t: torch.Tensor, n) -> int:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("src must be a contiguous device tensor")
    nbytes = t.numel() * t.element_size()
    if kind == KIND_BF16:
        if t.element_size() != 2:
            raise TypeError("BF16 input needs 2-byte elements")
        return t.numel()
    if t.element_size() != 1:
        raise TypeError("uint8 / uint4 input is a byte tensor")
    if kind == KIND_U8:
        return nbytes
    n = 2 * nbytes if n is None else int(n)
    if n < 0 or (n + 1) // 2 > nbytes:
        raise ValueError("uint4 input holds fewer than n elements")
    return n


def df_histogram_device(kind: int, src: torch.Tensor, n=None, stream=None) -> torch.Tensor:
    """256 counts (a device int64 tensor holding uint64 values)."""
    n = _device_elements(kind, src, n)
    h = torch.empty(256, dtype=torch.int64, device=src.device)
    _check(lib().df_histogram_device(kind, ctypes.c_void_p(src.data_ptr()), n, ctypes.c_void_p(h.data_ptr()),
                                     _stream_handle(stream, src.device)), "df_histogram_device")
    return h


def df_symbol_device(kind: int, src: torch.Tensor, i: int, stream=None) -> torch.Tensor:
    """The coded symbol of element i (a device int64 tensor of one element)."""
    _device_elements(kind, src, None if kind != KIND_U4 else i + 1)
    out = torch.zeros(1, dtype=torch.int64, device=src.device)
    _check(lib().df_symbol_device(kind, ctypes.c_void_p(src.data_ptr()), int(i), ctypes.c_void_p(out.data_ptr()),
                                  _stream_handle(stream, src.device)), "df_symbol_device")
    return out


def df_encode_layout(kind: int, n: int, hist, last_symbol: int, lengths) -> df_info:
    h = np.ascontiguousarray(hist, np.uint64)
    ln = np.ascontiguousarray(lengths, np.uint8)
    out = df_info()
    _check(lib().df_encode_layout(kind, int(n), h.ctypes.data, int(last_symbol), ln.ctypes.data,
                                  ctypes.byref(out)), "df_encode_layout")
    return out


DTAB_BYTES_U8 = 4 * 8192 + 256   # uint8: pair table, then the code lengths
DTAB_BYTES = 8 * 4096             # BF16 and uint4: multi-code table


def df_build_tables(kind: int, lengths, lut_cap: int = 64):
    """(lut uint16[n_luts * 256], n_luts, dtab as uint64 words: the DTAB
    section's bytes)."""
    ln = np.ascontiguousarray(lengths, np.uint8)
    lut = np.zeros(lut_cap * 256, np.uint16)
    dtab = np.zeros((DTAB_BYTES_U8 if kind == KIND_U8 else DTAB_BYTES) // 8, np.uint64)
    nl = ctypes.c_uint32(0)
    _check(lib().df_build_tables(kind, ln.ctypes.data, lut.ctypes.data, int(lut_cap), ctypes.byref(nl),
                                 dtab.ctypes.data), "df_build_tables")
    return lut[: nl.value * 256].copy(), nl.value, dtab


def df_encode_workspace_bytes(n: int) -> int:
    return int(lib().df_encode_workspace_bytes(int(n)))


def df_encode_device(kind: int, src: torch.Tensor, n: int, lengths, layout: df_info, sections: dict,
                     workspace: torch.Tensor, max_tile: torch.Tensor, stream=None):
    ln = np.ascontiguousarray(lengths, np.uint8)
    ptr = lambda name: ctypes.c_void_p(sections[name].data_ptr())  # noqa: E731
    sm = ptr("sign_mantissa") if kind == KIND_BF16 else None
    _check(lib().df_encode_device(kind, ctypes.c_void_p(src.data_ptr()), int(n), ln.ctypes.data,
                                  ctypes.byref(layout), ptr("bitstream"), ptr("gaps"), ptr("tile_out"), sm,
                                  ctypes.c_void_p(workspace.data_ptr()), ctypes.c_void_p(max_tile.data_ptr()),
                                  _stream_handle(stream, src.device)), "df_encode_device")


ENCODE_SCRATCH_BYTES = 16 << 20   # df_encode_device_noalloc's workspace (DF_ENCODE_SCRATCH_BYTES)


def df_encode_device_noalloc(kind: int, src: torch.Tensor, n: int, lengths, layout: df_info, sections: dict,
                             max_tile: torch.Tensor, stream=None):
    """df_encode_device with the library's static workspace (no allocation)."""
    ln = np.ascontiguousarray(lengths, np.uint8)
    ptr = lambda name: ctypes.c_void_p(sections[name].data_ptr())  # noqa: E731
    sm = ptr("sign_mantissa") if kind == KIND_BF16 else None
    _check(lib().df_encode_device_noalloc(kind, ctypes.c_void_p(src.data_ptr()), int(n), ln.ctypes.data,
                                          ctypes.byref(layout), ptr("bitstream"), ptr("gaps"), ptr("tile_out"), sm,
                                          ctypes.c_void_p(max_tile.data_ptr()), _stream_handle(stream, src.device)),
           "df_encode_device_noalloc")


def compress_device(kind: int, src: torch.Tensor, max_len: int = MAX_LEN, n=None, stream=None) -> DeviceContainer:
    """Encode device-resident elements on the GPU: device histogram, codebook
    and tables on the host, device encode.  The sections equal compress()'s.
    For uint4, src is the packed bytes and n the element count."""
    return compress_device_batch(kind, [src], max_len, None if n is None else [n], stream)[0]


def compress_device_batch(kind: int, srcs, max_len: int = MAX_LEN, ns=None, stream=None) -> list:
    """compress_device over several tensors of one kind (the layers of a
    block) with two reads back to the host in all: the histograms and last
    symbols in one copy after the histogram launches, the largest tile sizes
    in one copy after every encode launch.  Codebooks, layouts and tables
    are built on the host between them; the tables go to the device in one
    copy from pinned memory.  Every step runs on `stream` (default: the
    current stream)."""
    srcs = list(srcs)
    if not srcs:
        return []
    dev = srcs[0].device
    ns = [_device_elements(kind, t, k) for t, k in zip(srcs, ns if ns is not None else [None] * len(srcs))]
    ts = _torch_stream(stream, dev)
    k = len(srcs)
    with torch.cuda.stream(ts):
        hists = torch.empty((k, 256), dtype=torch.int64, device=dev)
        lasts = torch.zeros(k, dtype=torch.int64, device=dev)
        for i, (t, n) in enumerate(zip(srcs, ns)):
            _check(lib().df_histogram_device(kind, ctypes.c_void_p(t.data_ptr()), n,
                                             ctypes.c_void_p(hists[i].data_ptr()), ctypes.c_void_p(ts.cuda_stream)),
                   "df_histogram_device")
            if n:   # the symbol of the element that ends the stream
                _check(lib().df_symbol_device(kind, ctypes.c_void_p(t.data_ptr()), n - 1,
                                              ctypes.c_void_p(lasts[i].data_ptr()), ctypes.c_void_p(ts.cuda_stream)),
                       "df_symbol_device")
        back = torch.cat([hists.view(-1), lasts]).cpu().numpy()

        def host_part(i):   # codebook, layout and tables of container i
            n = ns[i]
            hist = back[256 * i: 256 * i + 256].view(np.uint64)
            lengths = df_build_codebook(hist, max_len)
            lay = df_encode_layout(kind, n, hist, int(back[256 * k + i]), lengths)
            lut, _, dtab = df_build_tables(kind, lengths)
            return lay, lengths, (lut.view(np.uint8), dtab.view(np.uint8))

        parts = [host_part(i) for i in range(k)]
        lays = [p[0] for p in parts]
        infos = [_info_dict(p[0]) for p in parts]
        lens = [p[1] for p in parts]
        tabs = [p[2] for p in parts]
        # every container's LUT and DTAB in one pinned buffer, one copy; each
        # section is a 256-byte aligned view of the device copy
        offs, tot = [], 0
        for lut, dtab in tabs:
            offs.append((tot, tot + _round256(max(lut.size, 16))))
            tot = offs[-1][1] + _round256(max(dtab.size, 16))
        pinned = torch.zeros(tot, dtype=torch.uint8, pin_memory=True)
        pv = pinned.numpy()
        for (lut, dtab), (a, b) in zip(tabs, offs):
            pv[a: a + lut.size] = lut
            pv[b: b + dtab.size] = dtab
        tables = pinned.to(dev, non_blocking=True)
        ws = torch.empty(max(max(df_encode_workspace_bytes(n) for n in ns), 16), dtype=torch.uint8, device=dev)
        max_tiles = torch.zeros(k, dtype=torch.int32, device=dev)
        secs = []
        for i, (t, n) in enumerate(zip(srcs, ns)):
            inf = infos[i]
            sec = {name: torch.empty(max(inf["section_bytes"][name], 16), dtype=torch.uint8, device=dev)
                   for name in SECTION_NAMES if name not in ("lut", "dtab")}
            (lut, dtab), (a, b) = tabs[i], offs[i]
            sec["lut"] = tables[a: a + max(lut.size, 16)]
            sec["dtab"] = tables[b: b + max(dtab.size, 16)]
            df_encode_device(kind, t, n, lens[i], lays[i], sec, ws, max_tiles[i: i + 1], ts)
            secs.append({name: sec[name] for name in SECTION_NAMES})
        mt = max_tiles.cpu().numpy()
    out = []
    for i in range(k):
        infos[i]["max_tile_elems"] = int(mt[i])
        dc = DeviceContainer(None, dev, _info=infos[i], _sections=secs[i])
        dc.layout = lays[i]   # df_encode_layout's result, for encoding again
        dc.lengths = lens[i]
        out.append(dc)
    return out


def _round256(x: int) -> int:
    return (x + 255) // 256 * 256


def _torch_stream(stream, device):
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


def _stream_handle(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check_dst(dc: DeviceContainer, dst: torch.Tensor):
    need = output_bytes(dc.kind, dc.n)
    if not dst.is_cuda or not dst.is_contiguous() or dst.numel() * dst.element_size() < need:
        raise ValueError("dst must be a contiguous device tensor of at least %d bytes" % need)


def _view(dc: DeviceContainer, max_workgroups) -> df_device_view:
    """The container's view, with a workgroup cap when one is given."""
    if not max_workgroups:
        return dc.view
    v = df_device_view.from_buffer_copy(dc.view)
    v.max_workgroups = int(max_workgroups)
    return v


def df_decompress(dc: DeviceContainer, dst: torch.Tensor, stream=None, max_workgroups=None):
    """max_workgroups: cap on the launch's workgroups (None or 0: no cap)."""
    _check_dst(dc, dst)
    _check(lib().df_decompress(ctypes.byref(_view(dc, max_workgroups)), ctypes.c_void_p(dst.data_ptr()),
                               _stream_handle(stream, dst.device)), "df_decompress")


def df_decompress_checked(dc: DeviceContainer, dst: torch.Tensor, err: torch.Tensor, stream=None,
                          max_workgroups=None):
    """err: a device int32/uint32 tensor of one element, zeroed by the caller."""
    _check_dst(dc, dst)
    if not err.is_cuda or err.element_size() != 4:
        raise ValueError("err must be a 4-byte device tensor")
    _check(lib().df_decompress_checked(ctypes.byref(_view(dc, max_workgroups)), ctypes.c_void_p(dst.data_ptr()),
                                       ctypes.c_void_p(err.data_ptr()),
                                       _stream_handle(stream, dst.device)), "df_decompress_checked")


def df_decompress_batch(dcs, dsts, stream=None, max_workgroups=None):
    if len(dcs) != len(dsts):
        raise ValueError("one destination per container")
    for dc, d in zip(dcs, dsts):
        _check_dst(dc, d)
    views = (df_device_view * max(len(dcs), 1))(*[_view(dc, max_workgroups) for dc in dcs])
    ptrs = (ctypes.c_void_p * max(len(dsts), 1))(*[d.data_ptr() for d in dsts])
    dev = dsts[0].device if dsts else None
    _check(lib().df_decompress_batch(views, ptrs, len(dcs), _stream_handle(stream, dev)),
           "df_decompress_batch")
