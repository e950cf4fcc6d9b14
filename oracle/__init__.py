"""ctypes wrapper around the plain serial C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY.  The oracle defines what a correct decode is; it is
used by the tests, by the smoke entry point and by the benchmark's CPU-baseline
leg, and by nothing in the product package.  It shares no code with the HIP
path and never imports it.

``build()`` compiles ``liboracle.so`` next to this file with gcc.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")

ERRORS = {
    0: "ok", -1: "bad argument", -2: "bad magic/version/fixed field", -3: "truncated or misplaced section",
    -4: "code length out of range", -5: "Kraft sum wrong", -6: "prefix conflict",
    -7: "stream does not decode to n symbols", -8: "non-zero padding", -9: "gap mismatch",
    -10: "group table mismatch", -11: "tensor table mismatch", -12: "size fields inconsistent",
    -13: "out of memory", -14: "output too small", -15: "element kind differs",
}


class OracleError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"oracle {what}: {ERRORS.get(code, 'unknown')} ({code})")
        self.code = code


class Report(ctypes.Structure):
    _fields_ = [
        ("n_elems", ctypes.c_uint64),
        ("stream_bits", ctypes.c_uint64),
        ("n_chunks", ctypes.c_uint64),
        ("n_groups", ctypes.c_uint64),
        ("n_tensors", ctypes.c_uint32),
        ("chunks_per_group", ctypes.c_uint32),
        ("max_code_len", ctypes.c_uint32),
        ("n_symbols", ctypes.c_uint32),
        ("longest_code", ctypes.c_uint32),
        ("group_align", ctypes.c_uint32),
        ("group_max_elems", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
        ("kraft_num", ctypes.c_uint64),
        ("entropy_bits", ctypes.c_double),
        ("mean_code_bits", ctypes.c_double),
        ("hist", ctypes.c_uint64 * 256),
        ("layout", ctypes.c_uint32),
        ("seg_max_bits", ctypes.c_uint32),
        ("elem_kind", ctypes.c_uint32),
        ("coder", ctypes.c_uint32),
        ("gap_bits", ctypes.c_uint32),
    ]

    def as_dict(self):
        d = {k: getattr(self, k) for k, _ in self._fields_ if k != "hist"}
        d["hist"] = np.array(self.hist[:], dtype=np.uint64)
        return d


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (plain -O2, no vectorisation tricks)."""
    if force or not os.path.exists(_SO):
        src = os.path.join(_HERE, "oracle.c")
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared",
                               src, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        u16p = ctypes.POINTER(ctypes.c_uint16)
        u32p = ctypes.POINTER(ctypes.c_uint32)
        u64p = ctypes.POINTER(ctypes.c_uint64)
        L.orc_split_planes.argtypes = [u16p, ctypes.c_uint64, u8p, u8p]
        L.orc_split_planes.restype = None
        L.orc_join_planes.argtypes = [u8p, u8p, ctypes.c_uint64, u16p]
        L.orc_join_planes.restype = None
        L.orc_heap_huffman.argtypes = [u64p, u8p]
        L.orc_package_merge.argtypes = [u64p, ctypes.c_uint32, u8p]
        L.orc_canonical_codes.argtypes = [u8p, u32p]
        L.orc_encode.argtypes = [u16p, ctypes.c_uint64, u64p, ctypes.c_uint32, ctypes.c_uint32,
                                 ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(u8p), u64p]
        L.orc_encode_gaps.argtypes = [u16p, ctypes.c_uint64, u64p, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32,
                                      ctypes.POINTER(u8p), u64p]
        L.orc_encode_lanes.argtypes = [u16p, ctypes.c_uint64, u64p, ctypes.c_uint32, ctypes.c_uint32,
                                       ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(u8p), u64p]
        L.orc_encode_lanes_u8.argtypes = [u8p, ctypes.c_uint64, u64p, ctypes.c_uint32, ctypes.c_uint32,
                                          ctypes.c_uint32, ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(u8p), u64p]
        L.orc_encode_lanes_rans.argtypes = [u16p, ctypes.c_uint64, u64p, ctypes.c_uint32, ctypes.c_uint32,
                                            ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(u8p), u64p]
        L.orc_encode_lanes_rans_u8.argtypes = [u8p, ctypes.c_uint64, u64p, ctypes.c_uint32, ctypes.c_uint32,
                                               ctypes.c_uint32, ctypes.c_uint32, ctypes.POINTER(u8p), u64p]
        L.orc_decode_u8.argtypes = [u8p, ctypes.c_uint64, u8p, ctypes.c_uint64, ctypes.POINTER(Report)]
        L.orc_decode.argtypes = [u8p, ctypes.c_uint64, u16p, ctypes.c_uint64, ctypes.POINTER(Report)]
        L.orc_header.argtypes = [u8p, ctypes.c_uint64, ctypes.POINTER(Report)]
        L.orc_gemv_bf16.argtypes = [u16p, ctypes.c_uint64, ctypes.c_uint64, u16p,
                                    ctypes.POINTER(ctypes.c_double)]
        L.orc_free.argtypes = [ctypes.c_void_p]
        L.orc_free.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray, ct):
    return a.ctypes.data_as(ctypes.POINTER(ct))


def split_planes(w: np.ndarray):
    w = np.ascontiguousarray(w, dtype=np.uint16)
    e = np.empty(w.size, np.uint8)
    sm = np.empty(w.size, np.uint8)
    lib().orc_split_planes(_p(w, ctypes.c_uint16), w.size, _p(e, ctypes.c_uint8), _p(sm, ctypes.c_uint8))
    return e, sm


def join_planes(e: np.ndarray, sm: np.ndarray):
    e = np.ascontiguousarray(e, dtype=np.uint8)
    sm = np.ascontiguousarray(sm, dtype=np.uint8)
    assert e.size == sm.size
    w = np.empty(e.size, np.uint16)
    lib().orc_join_planes(_p(e, ctypes.c_uint8), _p(sm, ctypes.c_uint8), e.size, _p(w, ctypes.c_uint16))
    return w


def _counts(counts) -> np.ndarray:
    c = np.zeros(256, np.uint64)
    src = np.asarray(counts, dtype=np.uint64)
    c[: src.size] = src
    return c


def heap_huffman_lengths(counts) -> np.ndarray:
    c = _counts(counts)
    lens = np.zeros(256, np.uint8)
    st = lib().orc_heap_huffman(_p(c, ctypes.c_uint64), _p(lens, ctypes.c_uint8))
    if st:
        raise OracleError(st, "heap_huffman")
    return lens


def package_merge_lengths(counts, max_len: int) -> np.ndarray:
    c = _counts(counts)
    lens = np.zeros(256, np.uint8)
    st = lib().orc_package_merge(_p(c, ctypes.c_uint64), int(max_len), _p(lens, ctypes.c_uint8))
    if st:
        raise OracleError(st, "package_merge")
    return lens


def canonical_codes(lens) -> np.ndarray:
    L = np.zeros(256, np.uint8)
    src = np.asarray(lens, dtype=np.uint8)
    L[: src.size] = src
    codes = np.zeros(256, np.uint32)
    st = lib().orc_canonical_codes(_p(L, ctypes.c_uint8), _p(codes, ctypes.c_uint32))
    if st:
        raise OracleError(st, "canonical_codes")
    return codes


def encode(w: np.ndarray, numels=None, max_code_len: int = 24, chunks_per_group: int = 128,
           group_align: int = 128, group_max_elems: int = 4096, gap_bits: int = 8) -> np.ndarray:
    """Oracle's own serial container writer.  Returns the container bytes.

    chunks_per_group (G), group_align (A) and group_max_elems (M) set the group
    table: groups are runs of whole A-element blocks whose codewords touch at
    most G chunks, of at most M elements.  gap_bits: 8 (one byte per chunk) or
    5 (packed)."""
    w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
    if numels is None:
        nump, nt = None, 1
    else:
        arr = np.ascontiguousarray(numels, dtype=np.uint64)
        nump, nt = _p(arr, ctypes.c_uint64), arr.size
    out = ctypes.POINTER(ctypes.c_uint8)()
    nbytes = ctypes.c_uint64(0)
    st = lib().orc_encode_gaps(_p(w, ctypes.c_uint16), w.size, nump, nt, int(max_code_len),
                               int(chunks_per_group), int(group_align), int(group_max_elems), int(gap_bits),
                               ctypes.byref(out), ctypes.byref(nbytes))
    if st:
        raise OracleError(st, "encode")
    try:
        blob = np.ctypeslib.as_array(out, shape=(nbytes.value,)).copy() if nbytes.value else np.zeros(0, np.uint8)
    finally:
        lib().orc_free(out)
    return blob


def encode_lanes(w: np.ndarray, numels=None, max_code_len: int = 24, group_align: int = 128,
                 group_max_elems: int = 4096, seg_max_bits: int = 15872) -> np.ndarray:
    """Oracle's own serial writer of the interleaved-lane layout (version 3).

    Segments are runs of whole group_align-element blocks of at most
    group_max_elems elements and seg_max_bits stream bits; inside a segment,
    lane j of 64 takes the 8-element lane blocks j, j + 64, ..., and each
    lane's codewords are stored together, lane after lane."""
    w = np.ascontiguousarray(w, dtype=np.uint16).reshape(-1)
    if numels is None:
        nump, nt = None, 1
    else:
        arr = np.ascontiguousarray(numels, dtype=np.uint64)
        nump, nt = _p(arr, ctypes.c_uint64), arr.size
    out = ctypes.POINTER(ctypes.c_uint8)()
    nbytes = ctypes.c_uint64(0)
    st = lib().orc_encode_lanes(_p(w, ctypes.c_uint16), w.size, nump, nt, int(max_code_len), int(group_align),
                                int(group_max_elems), int(seg_max_bits), ctypes.byref(out), ctypes.byref(nbytes))
    if st:
        raise OracleError(st, "encode_lanes")
    try:
        blob = np.ctypeslib.as_array(out, shape=(nbytes.value,)).copy() if nbytes.value else np.zeros(0, np.uint8)
    finally:
        lib().orc_free(out)
    return blob


def encode_lanes_u8(codes: np.ndarray, numels=None, max_code_len: int = 24, group_align: int = 128,
                    group_max_elems: int = 4096, seg_max_bits: int = 15872) -> np.ndarray:
    """Oracle's writer of a u8-kind interleaved-lane container: every byte of
    `codes` is one symbol of the canonical code; no raw plane."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1)
    if numels is None:
        nump, nt = None, 1
    else:
        arr = np.ascontiguousarray(numels, dtype=np.uint64)
        nump, nt = _p(arr, ctypes.c_uint64), arr.size
    out = ctypes.POINTER(ctypes.c_uint8)()
    nbytes = ctypes.c_uint64(0)
    st = lib().orc_encode_lanes_u8(_p(codes, ctypes.c_uint8), codes.size, nump, nt, int(max_code_len),
                                   int(group_align), int(group_max_elems), int(seg_max_bits), ctypes.byref(out),
                                   ctypes.byref(nbytes))
    if st:
        raise OracleError(st, "encode_lanes_u8")
    try:
        blob = np.ctypeslib.as_array(out, shape=(nbytes.value,)).copy() if nbytes.value else np.zeros(0, np.uint8)
    finally:
        lib().orc_free(out)
    return blob


def _encode_call(fn, data, ct, numels, *params):
    data = np.ascontiguousarray(data).reshape(-1)
    if numels is None:
        nump, nt = None, 1
    else:
        arr = np.ascontiguousarray(numels, dtype=np.uint64)
        nump, nt = _p(arr, ctypes.c_uint64), arr.size
    out = ctypes.POINTER(ctypes.c_uint8)()
    nbytes = ctypes.c_uint64(0)
    st = fn(_p(data, ct), data.size, nump, nt, *[int(v) for v in params], ctypes.byref(out), ctypes.byref(nbytes))
    if st:
        raise OracleError(st, fn.__name__)
    try:
        blob = np.ctypeslib.as_array(out, shape=(nbytes.value,)).copy() if nbytes.value else np.zeros(0, np.uint8)
    finally:
        lib().orc_free(out)
    return blob


def encode_lanes_rans(w: np.ndarray, numels=None, group_align: int = 128, group_max_elems: int = 4096,
                      seg_max_bits: int = 15872) -> np.ndarray:
    """Oracle's writer of an rANS lane container (coder 1) over bf16 words:
    12-bit frequencies, one rANS stream per lane."""
    return _encode_call(lib().orc_encode_lanes_rans, np.asarray(w, dtype=np.uint16), ctypes.c_uint16, numels,
                        group_align, group_max_elems, seg_max_bits)


def encode_lanes_rans_u8(codes: np.ndarray, numels=None, group_align: int = 128, group_max_elems: int = 4096,
                         seg_max_bits: int = 15872) -> np.ndarray:
    """The same over a plane of 8-bit codes (element kind u8)."""
    return _encode_call(lib().orc_encode_lanes_rans_u8, np.asarray(codes, dtype=np.uint8), ctypes.c_uint8, numels,
                        group_align, group_max_elems, seg_max_bits)


def decode_u8(blob: np.ndarray, with_report: bool = False):
    """Serial decode of a u8-kind container: returns the bytes (uint8)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    h = header(blob)
    n = int(h["n_elems"])
    out = np.empty(max(n, 1), np.uint8)
    rep = Report()
    st = lib().orc_decode_u8(_p(blob, ctypes.c_uint8), blob.size, _p(out, ctypes.c_uint8), n, ctypes.byref(rep))
    if st:
        raise OracleError(st, "decode_u8")
    out = out[:n]
    return (out, rep.as_dict()) if with_report else out


def gemv_bf16(W: np.ndarray, x: np.ndarray) -> np.ndarray:
    """y = W x in float64 for bf16 bit patterns W (rows x cols, uint16) and x (cols)."""
    W = np.ascontiguousarray(W, dtype=np.uint16)
    x = np.ascontiguousarray(x, dtype=np.uint16).reshape(-1)
    rows, cols = W.shape
    assert x.size == cols
    y = np.zeros(rows, np.float64)
    st = lib().orc_gemv_bf16(_p(W, ctypes.c_uint16), rows, cols, _p(x, ctypes.c_uint16),
                             _p(y, ctypes.c_double))
    if st:
        raise OracleError(st, "gemv_bf16")
    return y


def header(blob: np.ndarray) -> dict:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    rep = Report()
    st = lib().orc_header(_p(blob, ctypes.c_uint8), blob.size, ctypes.byref(rep))
    if st:
        raise OracleError(st, "header")
    return rep.as_dict()


def decode(blob: np.ndarray, with_report: bool = False):
    """Serial bit-by-bit decode with every container check.

    Returns the bf16 bit patterns (uint16), plus the report dict if asked."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    h = header(blob)
    n = int(h["n_elems"])
    out = np.empty(max(n, 1), np.uint16)
    rep = Report()
    st = lib().orc_decode(_p(blob, ctypes.c_uint8), blob.size, _p(out, ctypes.c_uint16), n, ctypes.byref(rep))
    if st:
        raise OracleError(st, "decode")
    out = out[:n]
    return (out, rep.as_dict()) if with_report else out


def decode_status(blob: np.ndarray) -> int:
    """Status code of a full decode (0 = valid container)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    rep = Report()
    st = lib().orc_header(_p(blob, ctypes.c_uint8), blob.size, ctypes.byref(rep))
    if st:
        return st
    n = int(rep.n_elems)
    out = np.empty(max(n, 1), np.uint16)
    return lib().orc_decode(_p(blob, ctypes.c_uint8), blob.size, _p(out, ctypes.c_uint16), n, None)
