"""Thin ctypes binding of libwc (include/wc.h).

Argument marshalling only: every step of encoding, planning and decoding runs
in the native library (host C++ and gfx950 HIP kernels).  Importing this
module loads ``libwc.so`` from this package directory and fails loudly if it
has not been built (``python -m lossless_entropy_coded_amd.build``); there is
no Python or CPU fallback for any entry point.

PyTorch is used only as the owner of device memory and streams: callers pass
tensors (or raw integer device pointers) and the binding forwards
``data_ptr()`` and ``torch.cuda.current_stream().cuda_stream``.

The C entry points receive bare pointers without sizes, so before forwarding
a tensor the binding checks what the kernels will touch: the tensor must be a
CUDA tensor on the plan's device, contiguous, and at least as large as the
bytes the call reads or writes.  A failed check raises ``WCError`` with
``WC_ERR_INVALID_ARG`` and nothing is launched.  Raw integer pointers are
forwarded unchecked (the C side checks their alignment only).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libwc.so is not built at {LIB_PATH}; run `python -m lossless_entropy_coded_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_u8p = ctypes.POINTER(ctypes.c_uint8)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_u64p = ctypes.POINTER(ctypes.c_uint64)
_u32p = ctypes.POINTER(ctypes.c_uint32)


class EncodeOpts(ctypes.Structure):
    _fields_ = [("max_code_len", ctypes.c_uint32), ("chunk_bytes", ctypes.c_uint32),
                ("chunks_per_group", ctypes.c_uint32), ("n_threads", ctypes.c_uint32),
                ("group_align", ctypes.c_uint32), ("group_max_elems", ctypes.c_uint32),
                ("layout", ctypes.c_uint32), ("seg_max_bits", ctypes.c_uint32), ("coder", ctypes.c_uint32),
                ("gap_bits", ctypes.c_uint32)]


_lib.wc_encode_host.argtypes = [ctypes.POINTER(_u16p), _u64p, ctypes.c_uint32, ctypes.POINTER(EncodeOpts),
                                ctypes.POINTER(_u8p), _u64p]
_lib.wc_encode_host.restype = ctypes.c_int
_lib.wc_encode_u8_host.argtypes = [ctypes.POINTER(_u8p), _u64p, ctypes.c_uint32, ctypes.POINTER(EncodeOpts),
                                   ctypes.POINTER(_u8p), _u64p]
_lib.wc_encode_u8_host.restype = ctypes.c_int
_lib.wc_free_host.argtypes = [_u8p]
_lib.wc_free_host.restype = None
_lib.wc_plan.argtypes = [_u8p, ctypes.c_uint64, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p)]
_lib.wc_plan.restype = ctypes.c_int
_lib.wc_plan_info.argtypes = [ctypes.c_void_p, _u64p, _u32p, _u64p, _u64p]
_lib.wc_plan_info.restype = ctypes.c_int
_lib.wc_plan_stats.argtypes = [ctypes.c_void_p, _u64p, _u64p, _u64p, _u32p, _u32p, _u32p, _u32p]
_lib.wc_plan_stats.restype = ctypes.c_int
_lib.wc_decode_async.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.wc_decode_async.restype = ctypes.c_int
_lib.wc_decode_u8_async.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.wc_decode_u8_async.restype = ctypes.c_int
_lib.wc_plan_format.argtypes = [ctypes.c_void_p, _u32p, _u32p, _u32p]
_lib.wc_plan_format.restype = ctypes.c_int
_lib.wc_plan_decode_shape.argtypes = [ctypes.c_void_p, _u32p, _u32p, _u32p]
_lib.wc_plan_decode_shape.restype = ctypes.c_int
_lib.wc_gemv_bf16_async.argtypes = [ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
_lib.wc_gemv_bf16_async.restype = ctypes.c_int


class GemvOperand(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_uint32), ("cols", ctypes.c_uint32), ("x", ctypes.c_void_p),
                ("y", ctypes.c_void_p)]


_lib.wc_decode_gemv_work_bytes.argtypes = [ctypes.c_void_p, ctypes.POINTER(GemvOperand), ctypes.c_uint32, _u64p]
_lib.wc_decode_gemv_work_bytes.restype = ctypes.c_int
_lib.wc_decode_gemv_async.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(GemvOperand),
                                      ctypes.c_uint32, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]
_lib.wc_decode_gemv_async.restype = ctypes.c_int
_lib.wc_decode_gemv_noalloc_async.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(GemvOperand),
                                              ctypes.c_uint32, ctypes.c_void_p]
_lib.wc_decode_gemv_noalloc_async.restype = ctypes.c_int
_lib.wc_stream_reference_async.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_uint64,
                                           ctypes.c_void_p]
_lib.wc_stream_reference_async.restype = ctypes.c_int
_lib.wc_plan_debug_status.argtypes = [ctypes.c_void_p, _u32p, ctypes.c_int]
_lib.wc_plan_debug_status.restype = ctypes.c_int
_lib.wc_plan_destroy.argtypes = [ctypes.c_void_p]
_lib.wc_plan_destroy.restype = None
_lib.wc_status_str.argtypes = [ctypes.c_int]
_lib.wc_status_str.restype = ctypes.c_char_p

# status codes (include/wc.h)
WC_OK = 0
WC_ERR_INVALID_ARG = -1
WC_ERR_NOMEM = -2
WC_ERR_HIP = -3
WC_ERR_UNSUPPORTED = -4
WC_ERR_SCRATCH = -5
# the no-allocation fused product's static work array (include/wc.h)
NOALLOC_SCRATCH_BYTES = 8 << 20
WC_ERR_BAD_MAGIC = -10
WC_ERR_TRUNCATED = -11
WC_ERR_SECTION_BOUNDS = -12
WC_ERR_CODE_LENGTHS = -13
WC_ERR_KRAFT = -14
WC_ERR_GAP = -15
WC_ERR_GROUP_START = -16
WC_ERR_STREAM_BITS = -17
WC_ERR_TENSOR_TABLE = -18
# bits of a debug plan's status word (plans made with WC_DEBUG=1)
WC_DEBUG_GROUP_COUNT = 1
WC_DEBUG_LANE_BITS = 2

# Group table defaults (wc_encode_opts): G = chunks per group, what one wave64
# decodes in one pass (two 64-bit chunks per lane; wider groups take several
# passes); A = elements per block, so that every group's output starts on a
# 256-byte boundary; M = elements per group at most (eight 8-element merge
# steps per lane).  The writer takes any G, A a positive multiple of 8 and
# M <= 4096, the range the GPU decoder takes.
GROUP_CHUNKS = 128
GROUP_ALIGN = 128
GROUP_MAX_ELEMS = 4096
# Interleaved-lane layout (container v3): stream bits per segment at most; the
# GPU decoder stages a segment's stream (at most 1984 bytes) in LDS.
SEG_MAX_BITS = 15872
LAYOUTS = {"lanes": 0, "chunks": 1}
# Entropy coders of the interleaved-lane layout: canonical Huffman, or rANS
# (12-bit frequencies, 32-bit state, 16-bit words; lanes layout only).
CODERS = {"huffman": 0, "rans": 1}

EXPORTED = ("wc_encode_host", "wc_encode_u8_host", "wc_free_host", "wc_plan", "wc_plan_info", "wc_plan_stats",
            "wc_plan_format", "wc_plan_decode_shape", "wc_decode_u8_async",
            "wc_decode_async", "wc_gemv_bf16_async", "wc_decode_gemv_work_bytes", "wc_decode_gemv_async",
            "wc_decode_gemv_noalloc_async", "wc_stream_reference_async", "wc_plan_debug_status",
            "wc_plan_destroy", "wc_status_str")


class WCError(RuntimeError):
    def __init__(self, status: int, call: str, detail: str = ""):
        self.status = status
        super().__init__(f"{call} failed: {status_str(status)} ({status})" + (f": {detail}" if detail else ""))


def status_str(status: int) -> str:
    return _lib.wc_status_str(int(status)).decode()


def _check(status: int, call: str):
    if status != WC_OK:
        raise WCError(status, call)


def _as_u16(t) -> np.ndarray:
    if hasattr(t, "numpy"):                    # torch CPU tensor (bf16/int16/uint16)
        import torch
        t = t.detach()
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        t = t.contiguous().numpy()
    a = np.ascontiguousarray(t).reshape(-1)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def encode_host(tensors, max_code_len: int = 24, chunks_per_group: int = GROUP_CHUNKS,
                n_threads: int = 0, group_align: int = GROUP_ALIGN,
                group_max_elems: int = GROUP_MAX_ELEMS, layout: str = "lanes",
                seg_max_bits: int = SEG_MAX_BITS, coder: str = "huffman", gap_bits: int = 8) -> np.ndarray:
    """wc_encode_host over a list of bf16 tensors (numpy uint16 or torch CPU).

    layout: "lanes" (the default: container v3, interleaved lanes;
    seg_max_bits caps a segment's stream bits) or "chunks" (container v2,
    per-chunk gaps; chunks_per_group applies).  coder: "huffman" or "rans"
    (lanes only; max_code_len is then ignored).  gap_bits: 8, or 5 for packed
    gaps (chunks only).
    Returns the container as a numpy uint8 array (a copy of the library buffer)."""
    arrs = [_as_u16(t) for t in tensors]
    nt = len(arrs)
    ptrs = (_u16p * max(nt, 1))(*[a.ctypes.data_as(_u16p) for a in arrs])
    numels = (ctypes.c_uint64 * max(nt, 1))(*[a.size for a in arrs])
    opts = EncodeOpts(max_code_len, 8, chunks_per_group, n_threads, group_align, group_max_elems,
                      LAYOUTS[layout], seg_max_bits, CODERS[coder], gap_bits)
    out = _u8p()
    nbytes = ctypes.c_uint64(0)
    _check(_lib.wc_encode_host(ptrs, numels, nt, ctypes.byref(opts), ctypes.byref(out), ctypes.byref(nbytes)),
           "wc_encode_host")
    try:
        blob = np.empty(nbytes.value, np.uint8)
        ctypes.memmove(blob.ctypes.data, out, nbytes.value)
    finally:
        _lib.wc_free_host(out)
    return blob


def encode_u8_host(tensors, max_code_len: int = 0, n_threads: int = 0, group_align: int = GROUP_ALIGN,
                   group_max_elems: int = GROUP_MAX_ELEMS, seg_max_bits: int = SEG_MAX_BITS,
                   coder: str = "huffman") -> np.ndarray:
    """wc_encode_u8_host over a list of uint8 code planes (numpy or torch CPU): a u8-kind
    interleaved-lane container (each byte one symbol, no raw plane), Huffman or rANS.
    max_code_len 0 selects the library's default for code planes (11 bits)."""
    arrs = [np.ascontiguousarray(t.numpy() if hasattr(t, "numpy") else t).reshape(-1).view(np.uint8)
            for t in tensors]
    nt = len(arrs)
    ptrs = (_u8p * max(nt, 1))(*[a.ctypes.data_as(_u8p) for a in arrs])
    numels = (ctypes.c_uint64 * max(nt, 1))(*[a.size for a in arrs])
    opts = EncodeOpts(max_code_len, 8, 0, n_threads, group_align, group_max_elems, LAYOUTS["lanes"], seg_max_bits,
                      CODERS[coder])
    out = _u8p()
    nbytes = ctypes.c_uint64(0)
    _check(_lib.wc_encode_u8_host(ptrs, numels, nt, ctypes.byref(opts), ctypes.byref(out), ctypes.byref(nbytes)),
           "wc_encode_u8_host")
    try:
        blob = np.empty(nbytes.value, np.uint8)
        ctypes.memmove(blob.ctypes.data, out, nbytes.value)
    finally:
        _lib.wc_free_host(out)
    return blob


class Plan:
    """wc_plan over a host container; owns the native plan until close()."""

    def __init__(self, blob_host: np.ndarray, device: int = 0):
        self._blob = np.ascontiguousarray(blob_host, dtype=np.uint8)
        h = ctypes.c_void_p()
        _check(_lib.wc_plan(self._blob.ctypes.data_as(_u8p), self._blob.size, int(device), ctypes.byref(h)),
               "wc_plan")
        self._h = h
        self.device = int(device)
        n = ctypes.c_uint64(0)
        nt = ctypes.c_uint32(0)
        _check(_lib.wc_plan_info(self._h, ctypes.byref(n), ctypes.byref(nt), None, None), "wc_plan_info")
        offs = (ctypes.c_uint64 * max(nt.value, 1))()
        nums = (ctypes.c_uint64 * max(nt.value, 1))()
        _check(_lib.wc_plan_info(self._h, None, None, offs, nums), "wc_plan_info")
        self.n_elems = n.value
        self.n_tensors = nt.value
        self.container_bytes = self.stats()["container_bytes"]
        self.tensor_offsets = [offs[i] for i in range(nt.value)]
        self.tensor_numels = [nums[i] for i in range(nt.value)]

    @property
    def handle(self):
        if self._h is None:
            raise RuntimeError("plan is closed")
        return self._h

    def format(self):
        """wc_plan_format: (container version, element kind: 0 bf16, 1 u8, coder: 0 Huffman, 1 rANS)."""
        v, k, c = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
        _check(_lib.wc_plan_format(self.handle, ctypes.byref(v), ctypes.byref(k), ctypes.byref(c)),
               "wc_plan_format")
        return v.value, k.value, c.value

    def decode_shape(self) -> dict:
        """wc_plan_decode_shape: waves per workgroup, grid and launches per call of the decode entry point."""
        w, g, n = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
        _check(_lib.wc_plan_decode_shape(self.handle, ctypes.byref(w), ctypes.byref(g), ctypes.byref(n)),
               "wc_plan_decode_shape")
        return {"waves_per_group": w.value, "grid": g.value, "launches": n.value}

    def stats(self) -> dict:
        cb, sb, ng = ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_uint64()
        kc, kd, gr, lds = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
        _check(_lib.wc_plan_stats(self.handle, ctypes.byref(cb), ctypes.byref(sb), ctypes.byref(ng),
                                  ctypes.byref(kc), ctypes.byref(kd), ctypes.byref(gr), ctypes.byref(lds)),
               "wc_plan_stats")
        return {"container_bytes": cb.value, "stream_bits": sb.value, "n_groups": ng.value,
                "count_bits": kc.value, "decode_bits": kd.value, "grid": gr.value, "lds_bytes": lds.value}

    def close(self):
        if self._h is not None:
            _lib.wc_plan_destroy(self._h)
            self._h = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def plan_debug_status(plan: Plan, reset: bool = False) -> int:
    """wc_plan_debug_status: the status word of a plan made with WC_DEBUG=1 in
    the environment (0: no invariant failed; WC_DEBUG_GROUP_COUNT: a group of
    the chunks layout decoded a codeword count other than its element count;
    WC_DEBUG_LANE_BITS: a lane of the lanes layout's decode or fused product
    did not end its string where the next lane's begins).  Waits for the
    plan's device; reset clears the word after reading it."""
    word = ctypes.c_uint32(0)
    _check(_lib.wc_plan_debug_status(plan.handle, ctypes.byref(word), 1 if reset else 0), "wc_plan_debug_status")
    return word.value


def _ptr(x) -> int:
    return int(x.data_ptr()) if hasattr(x, "data_ptr") else int(x)


def _require(t, nbytes: int, device, what: str, call: str) -> None:
    """Check a tensor argument before its pointer goes to C: a CUDA tensor on
    `device` (None: any), contiguous, holding at least `nbytes` bytes.  Raw
    integer pointers are not checked."""
    if not hasattr(t, "data_ptr"):
        return
    problem = None
    if not getattr(t, "is_cuda", False):
        problem = "is not a CUDA tensor"
    elif device is not None and t.device.index is not None and t.device.index != device:
        problem = f"is on cuda:{t.device.index}, not on cuda:{device}"
    elif not t.is_contiguous():
        problem = "is not contiguous"
    elif t.numel() * t.element_size() < nbytes:
        problem = f"holds {t.numel() * t.element_size()} bytes, fewer than the {nbytes} the call touches"
    if problem:
        raise WCError(WC_ERR_INVALID_ARG, call, f"{what} {problem}")


def decode_async(plan: Plan, blob_dev, out_dev, stream=None) -> None:
    """wc_decode_async: one launch decoding the whole container into out_dev.

    blob_dev / out_dev: torch device tensors (or raw device pointers).  stream:
    a torch.cuda.Stream, a raw hipStream_t integer, or None for torch's current
    stream."""
    _require(blob_dev, plan.container_bytes, plan.device, "blob_dev", "wc_decode_async")
    _require(out_dev, 2 * plan.n_elems, plan.device, "out_dev", "wc_decode_async")
    _check(_lib.wc_decode_async(plan.handle, ctypes.c_void_p(_ptr(blob_dev)), ctypes.c_void_p(_ptr(out_dev)),
                                ctypes.c_void_p(_stream_handle(stream))), "wc_decode_async")


def decode_u8_async(plan: Plan, blob_dev, out_dev, stream=None) -> None:
    """wc_decode_u8_async: one launch decoding a u8-kind container into out_dev (n bytes)."""
    _require(blob_dev, plan.container_bytes, plan.device, "blob_dev", "wc_decode_u8_async")
    _require(out_dev, plan.n_elems, plan.device, "out_dev", "wc_decode_u8_async")
    _check(_lib.wc_decode_u8_async(plan.handle, ctypes.c_void_p(_ptr(blob_dev)), ctypes.c_void_p(_ptr(out_dev)),
                                   ctypes.c_void_p(_stream_handle(stream))), "wc_decode_u8_async")


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        return int(torch.cuda.current_stream().cuda_stream)
    if hasattr(stream, "cuda_stream"):
        return int(stream.cuda_stream)
    return int(stream)


def gemv_bf16_async(W_dev, rows: int, cols: int, x_dev, y_dev, stream=None) -> None:
    """wc_gemv_bf16_async: y = W x (bf16 W rows x cols row-major, bf16 x, fp32 y), one launch.

    W_dev / x_dev / y_dev: torch device tensors (or raw device pointers)."""
    if rows > 0:
        dev = _current_device()
        _require(W_dev, 2 * int(rows) * int(cols), dev, "W", "wc_gemv_bf16_async")
        _require(x_dev, 2 * int(cols), dev, "x", "wc_gemv_bf16_async")
        _require(y_dev, 4 * int(rows), dev, "y", "wc_gemv_bf16_async")
    _check(_lib.wc_gemv_bf16_async(ctypes.c_void_p(_ptr(W_dev)), int(rows), int(cols), ctypes.c_void_p(_ptr(x_dev)),
                                   ctypes.c_void_p(_ptr(y_dev)), ctypes.c_void_p(_stream_handle(stream))),
           "wc_gemv_bf16_async")


def stream_reference_async(src_dev, src_bytes: int, dst_dev, dst_bytes: int, stream=None) -> None:
    """wc_stream_reference_async: the streaming yardstick (reads src_bytes once,
    writes dst_bytes; 16-byte output item j = NOT input item
    min(floor(j r / 2^32), ns - 1), r = ceil(ns 2^32 / nd)), one launch."""
    if src_bytes or dst_bytes:
        dev = _current_device()
        _require(src_dev, int(src_bytes), dev, "src", "wc_stream_reference_async")
        _require(dst_dev, int(dst_bytes), dev, "dst", "wc_stream_reference_async")
    _check(_lib.wc_stream_reference_async(ctypes.c_void_p(_ptr(src_dev)), int(src_bytes), ctypes.c_void_p(_ptr(dst_dev)),
                                          int(dst_bytes), ctypes.c_void_p(_stream_handle(stream))),
           "wc_stream_reference_async")


def _current_device():
    import torch
    return torch.cuda.current_device() if torch.cuda.is_available() else None


def _require_operands(plan: Plan, ops, call: str) -> None:
    """x and y of every operand over a non-empty tensor: cols bf16 and
    numel / cols float32 (bad tensor indexes and shapes are left to C)."""
    for i, (t, c, x, y) in enumerate(ops):
        t, c = int(t), int(c)
        if not (0 <= t < plan.n_tensors) or c <= 0 or plan.tensor_numels[t] == 0:
            continue
        _require(x, 2 * c, plan.device, f"ops[{i}].x", call)
        _require(y, 4 * (plan.tensor_numels[t] // c), plan.device, f"ops[{i}].y", call)


def _operands(ops):
    """(tensor, cols, x, y) tuples -> a ctypes array of wc_gemv_operand (x, y: device tensors or pointers)."""
    arr = (GemvOperand * max(len(ops), 1))()
    for i, (t, c, x, y) in enumerate(ops):
        arr[i] = GemvOperand(int(t), int(c), _ptr(x) if x is not None else 0, _ptr(y) if y is not None else 0)
    return arr


def decode_gemv_work_bytes(plan: Plan, ops) -> int:
    """wc_decode_gemv_work_bytes for operands [(tensor, cols, x, y), ...]."""
    _require_operands(plan, ops, "wc_decode_gemv_work_bytes")
    n = ctypes.c_uint64(0)
    _check(_lib.wc_decode_gemv_work_bytes(plan.handle, _operands(ops), len(ops), ctypes.byref(n)),
           "wc_decode_gemv_work_bytes")
    return n.value


def decode_gemv_async(plan: Plan, blob_dev, ops, work_dev, work_bytes: int, stream=None) -> None:
    """wc_decode_gemv_async: y = W x for each operand (tensor, cols, x, y) -- consecutive tensors of the
    container, decoded on chip and never written out -- in one decode launch and one row-sum launch.
    work_dev: device scratch of work_bytes >= decode_gemv_work_bytes(plan, ops), 256-byte aligned."""
    _require(blob_dev, plan.container_bytes, plan.device, "blob_dev", "wc_decode_gemv_async")
    _require_operands(plan, ops, "wc_decode_gemv_async")
    _require(work_dev, int(work_bytes), plan.device, "work_dev", "wc_decode_gemv_async")
    _check(_lib.wc_decode_gemv_async(plan.handle, ctypes.c_void_p(_ptr(blob_dev)), _operands(ops), len(ops),
                                     ctypes.c_void_p(_ptr(work_dev)), int(work_bytes),
                                     ctypes.c_void_p(_stream_handle(stream))),
           "wc_decode_gemv_async")


def decode_gemv_noalloc_async(plan: Plan, blob_dev, ops, stream=None) -> None:
    """wc_decode_gemv_noalloc_async: decode_gemv_async with the library's static device work
    array (NOALLOC_SCRATCH_BYTES) instead of a caller's buffer; allocates nothing.  Calls that
    overlap on one GPU race on that array."""
    _require(blob_dev, plan.container_bytes, plan.device, "blob_dev", "wc_decode_gemv_noalloc_async")
    _require_operands(plan, ops, "wc_decode_gemv_noalloc_async")
    _check(_lib.wc_decode_gemv_noalloc_async(plan.handle, ctypes.c_void_p(_ptr(blob_dev)), _operands(ops), len(ops),
                                             ctypes.c_void_p(_stream_handle(stream))),
           "wc_decode_gemv_noalloc_async")


def exported_symbols():
    """Names of the C ABI entry points resolvable in the loaded library."""
    return [name for name in EXPORTED if hasattr(_lib, name)]
