"""Read-only numpy view of a container's sections, for tests.

Restates the container v2 layout (256-byte header of little-endian fields,
then 256-byte-aligned sections code_len, tensors, groups, gap, stream, sm) and
the interleaved-lane layout v3 (the same header positions, with u8 lanes at
9, u16 lane block at 10, u32 segment bit cap at 12, a u16 lane-offset section
in place of the gaps and n_chunks = 0) so that tests can inspect what an
encoder wrote.  It decodes nothing.
"""
from __future__ import annotations

import struct

import numpy as np

HEADER_FIELDS = {
    "max_code_len": (8, "<B"), "chunk_bits": (9, "<B"), "chunks_per_group": (12, "<I"),
    "n_tensors": (16, "<I"), "group_align": (20, "<I"), "n_elems": (24, "<Q"), "stream_bits": (32, "<Q"), "n_chunks": (40, "<Q"),
    "n_groups": (48, "<Q"), "off_len": (56, "<Q"), "off_tens": (64, "<Q"), "off_gs": (72, "<Q"),
    "off_gap": (80, "<Q"), "off_stream": (88, "<Q"), "stream_bytes": (96, "<Q"), "off_sm": (104, "<Q"),
    "total": (112, "<Q"), "group_max_elems": (120, "<I"),
}


def header(blob: np.ndarray) -> dict:
    raw = bytes(blob[:256])
    h = {k: struct.unpack_from(fmt, raw, off)[0] for k, (off, fmt) in HEADER_FIELDS.items()}
    h["magic"] = raw[:4]
    h["version"] = struct.unpack_from("<H", raw, 4)[0]
    h["elem_kind"] = raw[124]
    h["coder"] = raw[125]
    h["gap_bits"] = 5 if (h["version"] == 2 and raw[10] == 5) else 8
    if h["version"] == 3:
        h["lanes"] = raw[9]
        h["lane_block"] = struct.unpack_from("<H", raw, 10)[0]
        h["seg_max_bits"] = struct.unpack_from("<I", raw, 12)[0]
    return h


def sections(blob: np.ndarray) -> dict:
    h = header(blob)
    n, nc, ng, nt = h["n_elems"], h["n_chunks"], h["n_groups"], h["n_tensors"]
    s = dict(h)
    if h["coder"] == 1:      # rANS: u16 frequencies in the code-length section
        s["freq"] = blob[h["off_len"]:h["off_len"] + 512].view(np.uint16)
    else:
        s["code_len"] = blob[h["off_len"]:h["off_len"] + 256]
    s["tensors"] = blob[h["off_tens"]:h["off_tens"] + 16 * nt].view(np.uint64).reshape(nt, 2)
    s["groups"] = blob[h["off_gs"]:h["off_gs"] + 16 * (ng + 1)].view(np.uint64).reshape(ng + 1, 2)
    if h["version"] == 3:
        s["lane_off"] = blob[h["off_gap"]:h["off_gap"] + 2 * 64 * ng].view(np.uint16).reshape(ng, 64)
    elif h["gap_bits"] == 5:
        # packed: gap c in bits 5c .. 5c + 4 of the section, lowest bit first
        packed = blob[h["off_gap"]:h["off_gap"] + (5 * nc + 7) // 8]
        s["gap_packed"] = packed
        bits = np.unpackbits(packed, bitorder="little")[:5 * nc].reshape(nc, 5)
        s["gap"] = (bits.astype(np.uint8) << np.arange(5, dtype=np.uint8)).sum(axis=1).astype(np.uint8)
    else:
        s["gap"] = blob[h["off_gap"]:h["off_gap"] + nc]
    s["stream"] = blob[h["off_stream"]:h["off_stream"] + h["stream_bytes"]]
    s["sm"] = blob[h["off_sm"]:h["off_sm"] + (n if h["elem_kind"] == 0 else 0)]
    return s


def expected_metadata(exps: np.ndarray, code_len: np.ndarray, chunks_per_group: int, group_align: int,
                      group_max_elems: int):
    """Auxiliary variables recomputed from first principles with numpy.

    Codeword i starts at the sum of the lengths before it.  gap[c] is the
    offset of the first start at or after bit 64c (stream end if none).  The
    group table cuts the elements into blocks of A = group_align; a group is a
    run of whole blocks (at least one), as long as possible while its
    codewords touch at most G chunks, i.e. while the run ends at a bit
    <= 64 * (first chunk + G), and while it holds at most M = group_max_elems
    elements; each entry is {first element, its start bit}, and the last one
    {n, total bits}.  Returns (total, gap, groups[n_groups + 1, 2]).
    """
    lens = code_len.astype(np.int64)[exps.astype(np.int64)]
    n = exps.size
    starts = np.zeros(n, np.int64)
    if n:
        starts[1:] = np.cumsum(lens)[:-1]
    total = int(lens.sum())
    n_chunks = -(-total // 64)
    starts_s = np.append(starts, total)          # stream end acts as a sentinel start
    c_bits = 64 * np.arange(n_chunks, dtype=np.int64)
    gap = starts_s[np.searchsorted(starts_s, c_bits, side="left")] - c_bits
    A, G = int(group_align), int(chunks_per_group)
    block_bit = np.append(starts[::A], total)     # start of every block, then the end
    nb = block_bit.size - 1
    groups = [(0, 0)]
    k = 0
    while k < nb:
        limit = 64 * (int(block_bit[k]) // 64 + G)
        end = int(np.searchsorted(block_bit, limit, side="right")) - 1   # last block end <= limit
        end = min(max(end, k + 1), nb, k + int(group_max_elems) // A)
        groups.append((min(end * A, n), int(block_bit[end])))
        k = end
    return total, gap, np.array(groups, dtype=np.uint64)


def expected_segments(exps: np.ndarray, code_len: np.ndarray, group_align: int, group_max_elems: int,
                      seg_max_bits: int) -> np.ndarray:
    """Segment table of the interleaved-lane layout, from first principles:
    runs of whole A-element blocks (at least one), as long as possible while
    they hold at most M elements and their codewords at most B bits; entries
    {first element, bits before it}, then {n, total bits}."""
    lens = code_len.astype(np.int64)[exps.astype(np.int64)]
    n = exps.size
    A = int(group_align)
    csum = np.concatenate([[0], np.cumsum(lens)])
    block_bit = csum[np.minimum(np.arange(0, n + A, A)[: -(-n // A) + 1], n)]
    nb = block_bit.size - 1
    segs = [(0, 0)]
    k = 0
    while k < nb:
        # last block end whose bits from block k stay within B, at least one block, at most M elements
        end = int(np.searchsorted(block_bit, block_bit[k] + int(seg_max_bits), side="right")) - 1
        end = min(max(end, k + 1), nb, k + int(group_max_elems) // A)
        segs.append((min(end * A, n), int(block_bit[end])))
        k = end
    return np.array(segs, dtype=np.uint64)


def lane_permutation(m: int) -> np.ndarray:
    """Element order (inside a segment of m elements) in which the
    interleaved-lane layout stores codewords: element i belongs to lane
    (i // 8) % 64; a lane's elements keep their order, lanes follow each
    other from 0 to 63."""
    idx = np.arange(m)
    lane = (idx // 8) % 64
    order = np.lexsort((idx, lane))     # by lane, then by element
    return order


RANS_P = 12          # frequency precision: frequencies sum to 2^12
RANS_STATE_BITS = 32  # every non-empty lane string starts with its 32-bit final state


def expected_rans_freqs(hist: np.ndarray) -> np.ndarray:
    """Quantized rANS frequencies from a symbol histogram, restated from the
    rule: f = max(1, floor(count * 2^12 / n)) for present symbols, 0 for the
    others; while the sum exceeds 2^12, take one unit from the largest
    frequency above 1 (the lowest symbol among equals); a shortfall goes to
    the most frequent symbol (the lowest among equal counts)."""
    hist = np.asarray(hist, dtype=np.int64)
    n = int(hist.sum())
    f = np.zeros(256, np.int64)
    if n == 0:
        return f
    present = hist > 0
    f[present] = np.maximum(1, (hist[present] << RANS_P) // n)
    total = int(f.sum())
    while total > (1 << RANS_P):
        k = int(np.argmax(np.where(f > 1, f, -1)))     # argmax takes the lowest index among equals
        f[k] -= 1
        total -= 1
    if total < (1 << RANS_P):
        f[int(np.argmax(hist))] += (1 << RANS_P) - total
    return f


def rans_cost_eighths(f: int) -> int:
    """ceil(8 (12 - log2 f)) + 1 eighths of a bit, exactly: 8 log2 f has floor
    k = bit_length(f^8) - 1, and ceil(96 - y) = 96 - floor(y) for any real y,
    so the cost is 97 - k."""
    return 97 - ((int(f) ** 8).bit_length() - 1)


def expected_rans_segment_elems(exps: np.ndarray, freq: np.ndarray, group_align: int, group_max_elems: int,
                                seg_max_bits: int) -> np.ndarray:
    """First elements of the rANS segments (then n), restated from the rule:
    runs of whole A-element blocks (at least one), as long as possible while
    they hold at most M elements and 64 * 32 + (sum of the per-symbol costs of
    their elements, in eighths) / 8 <= B."""
    table = np.array([rans_cost_eighths(f) if f else 0 for f in range(4097)], np.int64)
    cost = table[np.asarray(freq, np.int64)[exps.astype(np.int64)]]
    n = exps.size
    A = int(group_align)
    csum = np.concatenate([[0], np.cumsum(cost)])
    block_cost = csum[np.minimum(np.arange(0, n + A, A)[: -(-n // A) + 1], n)]   # eighths before each block
    nb = block_cost.size - 1
    budget = 8 * (int(seg_max_bits) - 64 * RANS_STATE_BITS)
    elems = [0]
    k = 0
    while k < nb:
        end = int(np.searchsorted(block_cost, block_cost[k] + budget, side="right")) - 1
        end = min(max(end, k + 1), nb, k + int(group_max_elems) // A)
        elems.append(min(end * A, n))
        k = end
    return np.array(elems, dtype=np.uint64)
