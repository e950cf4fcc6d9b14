#!/usr/bin/env python3
"""Benchmark: block-level decode of entropy-coded bf16 weights on one MI355X.

One step = one call of wc_decode_async: a single kernel launch that decodes
every tensor of an 8B-shape transformer block (q, k, v, o, gate, up, down and
two RMSNorm vectors; 218,112,000 bf16 with one shared codebook) from its
container in HBM into bf16 in HBM.  Inputs are resident in HBM before the
timed region; several (container, output) copies are rotated so that no step
reads what the previous one left in the 256 MB Infinity Cache.

Prints one JSON line:
  value     decompressed bf16 GB/s = 2 * n_elems * steps / elapsed
  roofline  algorithmic bytes of the decode kernel (container bytes it must
            read + 2 B per element written) / its average launch duration
            (HIP events on the launch stream), against 8 TB/s HBM3E peak;
            `traffic` = HBM bytes from rocprofv3 FETCH_SIZE/WRITE_SIZE runs
            recorded under profiles/ (null if the kernel source changed since);
            `stream_ref`: the library's streaming yardstick
            (wc_stream_reference_async: one load and one store per 16 bytes,
            workgroups in address order) reading as many bytes as the decode
            reads and writing as many as it writes, timed the same way in
            the same process; `frac_of_stream_ref` = achieved / its GB/s;
            `launch_us`: p10 / p50 / p90 of individually timed launches
  cpu_baseline  the CPU oracle's serial decode of the same container on one
            host core, repeated until about 10 s have elapsed (reported
            baseline, not a target), with the host CPU's model name
  layouts   (default run) the same block in the chunks layout, the two-phase
            count / scan / decode kernel: ms per launch and its fraction of
            8 TB/s on its own algorithmic bytes
  e2e       (default run) the 70B-shape block end to end: decode + 7 batch-1
            GEMVs (arm A), the GEMVs on resident uncompressed bf16 (arm B),
            the fused decode -> GEMV (arm C), and the decode alone

Evidence rules: every launch of a run takes the next (container, output) copy
in one rotation whose copies together exceed 1 GiB (four times the 256 MiB
Infinity Cache), so a copy's previous use is at least that much traffic back;
every output the timed launches write is first filled with a canary (or NaN)
and compared with the expected bits after the timed region.  Untimed launches
(settle, warm-up) read the same containers but write separate burn outputs,
and run both before the canary fill and for at least 10 ms after it, so the
timed launches start from the decode's own steady state.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decompressed bf16 GB/s and % of HBM roofline (1 MI355X), bit-exact"
METRIC_CODES = "decompressed 8-bit code GB/s and % of HBM roofline (1 MI355X), bit-exact"
HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 1 << 30          # rotated (container, output) bytes: 4 x the 256 MiB Infinity Cache
CANARY16 = 0x5A5A               # fills timed bf16 outputs before the timed region
CANARY8 = 0xA5
CSRC = os.path.join(ROOT, "lossless_entropy_coded_amd", "csrc")
# the files each decode kernel is compiled from (a counter record holds while
# none of them has changed)
KERNEL_SOURCES = {layout: [os.path.join(CSRC, f) for f in (src, "decode_common.h", "kernels.h")]
                  for layout, src in (("chunks", "decode.hip"), ("lanes", "decode_lanes.hip"))}
# counter records per kernel variant: layout, and the coder when not Huffman
TRAFFIC_FILES = {"chunks": os.path.join(ROOT, "profiles", "decode_chunks_block_8b_traffic.json"),
                 "lanes": os.path.join(ROOT, "profiles", "decode_lanes_block_8b_traffic.json"),
                 "lanes_rans": os.path.join(ROOT, "profiles", "decode_lanes_rans_block_8b_traffic.json")}


def variant_of(layout: str, coder: str = "huffman", gap_bits: int = 8) -> str:
    v = layout if coder == "huffman" else f"{layout}_{coder}"
    return v + "_gap5" if layout == "chunks" and gap_bits == 5 else v


def kernel_source_sha(layout: str = "chunks") -> str:
    """sha256 over the kernel's source files, in order."""
    h = hashlib.sha256()
    for path in KERNEL_SOURCES[layout]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str, layout: str = "chunks", coder: str = "huffman", gap_bits: int = 8):
    """HBM bytes per launch measured with rocprofv3 counters, if still valid
    (None for a variant with no record, such as packed gaps)."""
    try:
        with open(TRAFFIC_FILES[variant_of(layout, coder, gap_bits)]) as f:
            rec = json.load(f)
    except (OSError, ValueError, KeyError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_sha(layout) or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


def progress(msg: str) -> None:
    """One line on stderr per phase of a run (stdout carries only the JSON line)."""
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def rotation_copies(per_copy_bytes: int) -> int:
    """(container, output) copies to rotate through: together at least
    ROTATE_BYTES, so that the copy a launch reads was last touched at least
    ROTATE_BYTES - per_copy bytes of other traffic earlier."""
    return max(2, math.ceil(ROTATE_BYTES / max(1, per_copy_bytes)))


def cpu_model() -> str:
    """The host CPU's model name (the first 'model name' of /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def algorithmic_bytes(n: int, stream_bits: int, n_groups: int, layout: str, gap_bits: int, codes: bool) -> int:
    """Bytes the decode must move: the sm plane (bf16 kinds), the stream, the
    per-chunk gaps (chunks layout) or per-lane offsets (lanes layout), the
    group or segment table, and the decoded output."""
    n_chunks = -(-stream_bits // 64)
    aux = -(-gap_bits * n_chunks // 8) if layout == "chunks" else 2 * 64 * n_groups
    read = (0 if codes else n) + -(-stream_bits // 8) + aux + 16 * (n_groups + 1)
    return read + (1 if codes else 2) * n


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle-ms", type=float, default=60.0,
                    help="untimed decode launches before the warm-up steps, for at least this much GPU time: "
                         "the GPU's clocks take about 100 back-to-back launches (~15 ms) to reach steady state")
    ap.add_argument("--workload", default="block_8b",
                    help="synthetic workload (default: block_8b, the 8B-shape transformer block; "
                         "int8_codes_8b / int4_codes_8b: planes of quantized codes, decoded to bytes)")
    ap.add_argument("--cpu-baseline", choices=["on", "off"], default="on")
    ap.add_argument("--layout", choices=["lanes", "chunks"], default="lanes",
                    help="container layout: lanes (v3, interleaved lanes; the library's default) or "
                         "chunks (v2, per-chunk gaps)")
    ap.add_argument("--coder", choices=["huffman", "rans"], default="huffman",
                    help="entropy coder of the lanes layout: huffman (the default) or rans")
    ap.add_argument("--gap-bits", type=int, choices=[8, 5], default=8,
                    help="chunks layout: bits per stored gap, 8 or 5 (packed)")
    ap.add_argument("--max-code-len", type=int, default=0,
                    help="Huffman code length limit for the encoder (0: the library's default)")
    ap.add_argument("--e2e", action="store_true",
                    help="70B-shape block end to end: decode + batch-1 GEMVs against GEMVs on resident "
                         "uncompressed weights (prints its own JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="time a plain 1 GiB device copy instead (for scaling HBM counters)")
    ap.add_argument("--extras", choices=["on", "off"], default="on",
                    help="with the default workload and layout, also time the chunks layout and the 70B-block "
                         "end-to-end arms and add them to the JSON line (layouts, e2e)")
    return ap.parse_args()


def code_len_opt(args) -> dict:
    opt = {"max_code_len": args.max_code_len} if args.max_code_len else {}
    if args.gap_bits != 8:
        opt["gap_bits"] = args.gap_bits
    return opt


def aligned_device_copy(torch, blob, align=256):
    owner = torch.empty(blob.size + align, dtype=torch.uint8, device="cuda")
    off = (-owner.data_ptr()) % align
    view = owner[off:off + blob.size]
    view.copy_(torch.from_numpy(blob))
    return owner, view


def copy_calibration(args):
    """A plain streaming kernel of known traffic: reads 1 GiB, writes 1 GiB.

    (torch's same-dtype copy_ goes to a DMA engine, which kernel counters do
    not see; an elementwise bitwise-not is an ordinary copy-shaped kernel.)"""
    import torch
    nbytes = 1 << 30
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.warmup):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(args.steps):
        torch.bitwise_not(src, out=dst)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    print(json.dumps({"calibration": "copy-shaped kernel (bitwise_not)", "bytes_read_per_step": nbytes,
                      "bytes_written_per_step": nbytes, "steps": args.steps, "ms_per_step": ms,
                      "GBps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e9}), flush=True)


def stream_reference(torch, wc, read_bytes, write_bytes, steps, stream):
    """The streaming yardstick over the decode's traffic: wc_stream_reference_async
    reading `read_bytes` and writing `write_bytes` (rounded down to 16), in a
    rotation of copies exceeding 1 GiB like the decode's, settled for 60 ms,
    then `steps` back-to-back launches timed with HIP events on `stream`."""
    r16, w16 = read_bytes // 16 * 16, write_bytes // 16 * 16
    if not 0 < r16 <= w16:              # the yardstick reads at most what it writes
        return None
    copies = rotation_copies(r16 + w16)
    srcs = [torch.randint(-2**31, 2**31 - 1, (r16 // 4,), dtype=torch.int32, device="cuda") for _ in range(copies)]
    dsts = [torch.empty(w16 // 4, dtype=torch.int32, device="cuda") for _ in range(copies)]

    def launch(k):
        wc.stream_reference_async(srcs[k % copies], r16, dsts[k % copies], w16, stream)

    settle(torch, stream, launch, 60.0)
    ms = _timed(torch, stream, launch, steps)
    # spot check: the first and last output items of the last launch
    k = (steps - 1) % copies
    ns, nd = r16 // 16, w16 // 16
    rr = -(-(ns << 32) // nd)
    for j in (0, nd - 1):
        i = min((j * rr) >> 32, ns - 1)
        if not torch.equal(dsts[k][4 * j:4 * j + 4], ~srcs[k][4 * i:4 * i + 4]):
            print("bench.py: the streaming reference wrote wrong bytes", file=sys.stderr)
            sys.exit(3)
    del srcs, dsts
    torch.cuda.empty_cache()
    return {"kernel": "wc_stream_reference_async (one 16-byte load + store per lane, a workgroup per 4 KiB "
                      "of output in address order)",
            "read_bytes": r16, "write_bytes": w16, "ms": round(ms, 5),
            "GBps": round((r16 + w16) / (ms * 1e-3) / 1e9, 1), "rotating_copies": copies}


def _timed(torch, stream, fn, steps):
    """Milliseconds per call of fn over `steps` back-to-back calls (HIP events on `stream`)."""
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for k in range(steps):
        fn(k)
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def settle(torch, stream, fn, ms):
    """Untimed calls of fn until the GPU has run it for at least `ms`."""
    spent, k = 0.0, 0
    while spent < ms and k < 5000:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(10):
            fn(k)
            k += 1
        b.record(stream)
        b.synchronize()
        spent += a.elapsed_time(b)
    return k


class Scrub:
    """A 1 GiB buffer read (never written) right before a timed region: the
    canary fills leave dirty lines in the 256 MiB Infinity Cache, and reading
    4x its size writes them back before the timed launches start, not during
    them."""

    def __init__(self, torch):
        self.buf = torch.zeros(ROTATE_BYTES // 4, dtype=torch.int32, device="cuda")

    def __call__(self, torch, stream):
        with torch.cuda.stream(stream):
            self.buf.amax()


class Rotation:
    """Device copies of one container and of its output, used in turn by every
    launch of a run (one counter across settle, warm-up and timed launches)."""

    def __init__(self, torch, blob, n, out_dtype, copies):
        self.copies = copies
        self.owners, self.blobs, self.outs = [], [], []
        for _ in range(copies):
            own, view = aligned_device_copy(torch, blob)
            self.owners.append(own)
            self.blobs.append(view)
            self.outs.append(torch.empty(n, dtype=out_dtype, device="cuda"))
        self.it = 0

    def next(self):
        k = self.it % self.copies
        self.it += 1
        return k


def time_decode(torch, wc, plan, blob, raw, out_bytes, codes, args, stream):
    """Time `args.steps` back-to-back whole-container decode launches.

    Every launch takes the next copy of the rotation.  Before the timed
    launches every output copy is filled with a canary; after them each copy a
    timed launch wrote must equal the expected bits.  Returns the timing dict."""
    import numpy as np
    n = plan.n_elems
    decode = wc.decode_u8_async if codes else wc.decode_async
    out_dtype = torch.uint8 if codes else torch.int16
    copies = rotation_copies(blob.size + out_bytes * n)
    rot = Rotation(torch, blob, n, out_dtype, copies)
    ref = torch.from_numpy(np.ascontiguousarray(raw)).cuda()
    # untimed launches (settle, warm-up) read the rotation's containers but
    # write this output, so that only timed launches write the canaried copies
    burn_out = torch.empty(n, dtype=out_dtype, device="cuda")

    def launch(burn=False):
        k = rot.next()
        decode(plan, rot.blobs[k], burn_out if burn else rot.outs[k], stream)
        return k

    k = launch()
    torch.cuda.synchronize()
    if not torch.equal(rot.outs[k], ref):
        print("bench.py: decode is NOT bit-exact", file=sys.stderr)
        sys.exit(3)
    # settle: untimed launches until the GPU has run the decode for settle_ms
    settle_launches = settle(torch, stream, lambda _: launch(True), args.settle_ms)
    # canary in every output copy, the cache scrubbed, then the warm-up: W
    # launches and at least 10 ms more of them (the canary fills and the scrub
    # leave the memory system in another state than the decode's own), then
    # the timed launches: HIP events on the launch stream around K
    # back-to-back launches (a step is one launch)
    canary = CANARY8 if codes else CANARY16
    with torch.cuda.stream(stream):
        for o in rot.outs:
            o.fill_(canary)
    scrub = Scrub(torch)
    scrub(torch, stream)
    for _ in range(args.warmup):
        launch(True)
    settle_launches += args.warmup + settle(torch, stream, lambda _: launch(True), 10.0)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    written = set()
    for _ in range(args.steps):
        written.add(launch())
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    bit_exact = all(torch.equal(rot.outs[k], ref) for k in sorted(written))
    if not bit_exact:
        print("bench.py: timed outputs are NOT bit-exact", file=sys.stderr)
        sys.exit(3)
    # spread of single launches (each bracketed by its own events), after the timed region
    singles = []
    for _ in range(min(args.steps, 50)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        launch()
        b.record(stream)
        b.synchronize()
        singles.append(a.elapsed_time(b) * 1e3)
    singles.sort()

    def pct(q):
        return round(singles[min(len(singles) - 1, int(q * len(singles)))], 1)

    del rot, ref, scrub, burn_out
    torch.cuda.empty_cache()
    return {"total_ms": total_ms, "kernel_avg_ms": total_ms / args.steps, "copies": copies,
            "rotated_bytes": copies * (blob.size + out_bytes * n), "settle_launches": settle_launches,
            "timed_outputs_checked": len(written), "bit_exact": bit_exact,
            "launch_us": {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9)}}


def e2e_measure(torch, wc, name, layout, coder, steps, warmup, opts, stream):
    """The 70B-shape block: decode the whole block and run a batch-1 bf16 GEMV
    over each of its 7 matrices (arm A), against the same 7 GEMVs on resident
    uncompressed weights (arm B), and the fused decode -> GEMV of all 7
    matrices in one call, which never writes the decoded weights (arm C).
    Arms A and B run the same GEMV kernel, so their outputs must be
    bit-identical; arm C sums in another fixed order and must agree with B
    within both kernels' fp32 rounding bounds.  Every output of a timed arm is
    filled with NaN (the decoded weights with a canary) before it and checked
    after it.  Returns (record, ok)."""
    import numpy as np
    from lossless_entropy_coded_amd.synth import gemv_input, make_workload

    progress(f"{name}: generating and encoding ({layout}, {coder})")
    t_gen = time.perf_counter()
    wl = make_workload(name)
    blob = wc.encode_host(wl.tensors(), layout=layout, coder=coder, **opts)
    t_gen = time.perf_counter() - t_gen
    progress(f"{name}: timing arms A, B, C and the decode alone")
    plan = wc.Plan(blob, device=0)
    n = wl.n
    mats = [(k, s[0], s[1]) for k, s in enumerate(wl.shapes) if len(s) == 2]
    copies = rotation_copies(blob.size + 2 * n)
    rot = Rotation(torch, blob, n, torch.int16, copies)
    origs = [torch.from_numpy(wl.bits.view(np.int16)).cuda() for _ in range(copies)]
    xs = {c: torch.from_numpy(gemv_input(c).view(np.int16)).cuda() for _, _, c in mats}
    ya = [torch.empty(r, dtype=torch.float32, device="cuda") for _, r, _ in mats]
    yb = [torch.empty(r, dtype=torch.float32, device="cuda") for _, r, _ in mats]
    yc = [torch.empty(r, dtype=torch.float32, device="cuda") for _, r, _ in mats]
    ops = [(k, c, xs[c], yc[j]) for j, (k, r, c) in enumerate(mats)]
    # untimed launches write these instead, so that only timed launches
    # write the canaried (or NaN-filled) outputs
    burn_out = torch.empty(n, dtype=torch.int16, device="cuda")
    y_burn = [torch.empty(r, dtype=torch.float32, device="cuda") for _, r, _ in mats]
    ops_burn = [(k, c, xs[c], y_burn[j]) for j, (k, r, c) in enumerate(mats)]
    work_bytes = wc.decode_gemv_work_bytes(plan, ops)
    work_own = torch.empty(work_bytes // 4 + 64, dtype=torch.float32, device="cuda")
    work = work_own[(-work_own.data_ptr()) % 256 // 4:]

    def gemvs(src, ys):
        for j, (k, r, c) in enumerate(mats):
            off = plan.tensor_offsets[k]
            wc.gemv_bf16_async(src[off:off + r * c], r, c, xs[c], ys[j], stream)

    touched = set()

    def arm_a(_, burn=False):
        k = rot.next()
        out = burn_out if burn else rot.outs[k]
        if not burn:
            touched.add(k)
        wc.decode_async(plan, rot.blobs[k], out, stream)
        gemvs(out, y_burn if burn else ya)

    def arm_b(i, burn=False):
        gemvs(origs[i % copies], y_burn if burn else yb)

    def decode_only(_, burn=False):
        k = rot.next()
        if not burn:
            touched.add(k)
        wc.decode_async(plan, rot.blobs[k], burn_out if burn else rot.outs[k], stream)

    def arm_c(_, burn=False):
        wc.decode_gemv_async(plan, rot.blobs[rot.next()], ops_burn if burn else ops, work, work_bytes, stream)

    def fill(tensors, value):
        with torch.cuda.stream(stream):
            for t in tensors:
                t.fill_(value)

    def outs_exact():
        ok = all(torch.equal(rot.outs[k], origs[0]) for k in sorted(touched))
        touched.clear()
        return ok

    # each arm: settled for at least 60 ms of its own launches (the GPU's
    # clocks follow the load), its outputs filled with canaries, the cache
    # scrubbed, 10 ms more of its launches, and `steps` launches timed; the
    # untimed launches write the burn outputs
    scrub = Scrub(torch)
    warm = {}

    def timed_arm(name, fn, fills):
        warm[name] = settle(torch, stream, lambda i: fn(i, True), 60.0)
        for tensors, value in fills:
            fill(tensors, value)
        scrub(torch, stream)
        warm[name] += settle(torch, stream, lambda i: fn(i, True), 10.0)
        touched.clear()
        return _timed(torch, stream, fn, steps)

    ms_a = timed_arm("a", arm_a, [(rot.outs, CANARY16), (ya, float("nan"))])
    exact_a = outs_exact()
    ms_b = timed_arm("b", arm_b, [(yb, float("nan"))])
    ms_c = timed_arm("c", arm_c, [(yc, float("nan"))])
    ms_dec = timed_arm("decode", decode_only, [(rot.outs, CANARY16)])
    exact_dec = outs_exact()
    identical = all(torch.equal(a.view(torch.int32), b.view(torch.int32)) for a, b in zip(ya, yb))
    finite = all(bool(torch.isfinite(y).all()) for y in ya + yb + yc)
    # arm C against arm B: |yc - yb| <= (fused bound + GEMV bound) * 2^-24 * sum |w x|,
    # with sum |w x| from the GEMV kernel on the magnitudes (sign bits cleared)
    fused_ok = True
    for j, (t, r, c) in enumerate(mats):
        off = plan.tensor_offsets[t]
        mag = torch.empty(r, dtype=torch.float32, device="cuda")
        wc.gemv_bf16_async((origs[0][off:off + r * c] & 0x7FFF).contiguous(), r, c, (xs[c] & 0x7FFF).contiguous(),
                           mag, stream)
        terms = (12 + 8 + 6 + c // wc.GROUP_ALIGN + 2) + (c // 64 + 14)
        fused_ok &= bool(((yc[j] - yb[j]).abs() <= 1.05 * terms * 2.0 ** -24 * mag).all().item())
    ok = identical and exact_a and exact_dec and finite and fused_ok
    weight_bytes = 2 * sum(r * c for _, r, c in mats)
    rec = {
        "workload": f"{name}: decode of the whole block, then q,k,v,o,gate,up,down batch-1 GEMVs "
                    f"(x length = each matrix's in-dimension)",
        "layout": layout, "coder": coder, "n_elems": n, "container_bytes": int(blob.size),
        "weight_bytes": weight_bytes, "steps": steps, "settle_launches": warm, "rotating_copies": copies,
        "arm_a_decode_plus_gemv_ms": round(ms_a, 4),
        "arm_b_uncompressed_gemv_ms": round(ms_b, 4),
        "arm_c_fused_decode_gemv_ms": round(ms_c, 4),
        "decode_only_ms": round(ms_dec, 4),
        "ratio_a_over_b": round(ms_a / ms_b, 3),
        "ratio_c_over_b": round(ms_c / ms_b, 3),
        "fused_container_GBps": round(blob.size / (ms_c * 1e-3) / 1e9, 1),
        "fused_frac_of_hbm_peak": round(blob.size / (ms_c * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "gemv_weight_GBps": round(weight_bytes / (ms_b * 1e-3) / 1e9, 1),
        "decode_roofline_frac": round((blob.size + 2 * n) / (ms_dec * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "outputs_bit_identical_a_b": identical,
        "decoded_weights_bit_exact": exact_a and exact_dec,
        "fused_within_bound": fused_ok,
        "host_prep_s": round(t_gen, 2),
    }
    plan.close()
    del rot, origs, work_own, scrub, burn_out
    torch.cuda.empty_cache()
    # the streaming yardstick over the whole-block decode's traffic
    sref = stream_reference(torch, wc, int(blob.size), 2 * n, steps, stream)
    if sref:
        rec["decode_stream_ref"] = sref
        rec["decode_frac_of_stream_ref"] = round((blob.size + 2 * n) / (ms_dec * 1e-3) / 1e9 / sref["GBps"], 4)
    return rec, ok


def end_to_end(args):
    """--e2e: the 70B-block arms as a JSON line of their own."""
    import torch
    from lossless_entropy_coded_amd import wc
    name = args.workload if args.workload != "block_8b" else "block_70b"
    rec, ok = e2e_measure(torch, wc, name, args.layout, args.coder, args.steps, args.warmup, code_len_opt(args),
                          torch.cuda.current_stream())
    if not ok:
        print(f"bench.py --e2e: outputs disagree: {json.dumps(rec)}", file=sys.stderr)
        sys.exit(3)
    line = {
        "metric": "end-to-end batch-1 bf16 GEMV over a 70B-shape block: decode + GEMV vs GEMV on uncompressed weights",
        "value": rec["arm_a_decode_plus_gemv_ms"], "unit": "ms", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "higher_is_better": False, "vs_baseline": None, "dtype": "bf16 in, fp32 accumulate",
        "data": "synthetic: seeded bf16 weights (70B-block shapes, N(0, 0.015)), x ~ N(0, 1) in bf16",
        "config": {"workload": rec["workload"], "layout": args.layout, "coder": args.coder},
        **{k: v for k, v in rec.items() if k not in ("workload", "layout", "coder")},
    }
    print(json.dumps(line), flush=True)


def layout_record(torch, wc, wl, layout, args, stream):
    """The same workload in another layout, timed like the headline."""
    t = time.perf_counter()
    blob = wc.encode_host(wl.tensors(), layout=layout)
    t = time.perf_counter() - t
    plan = wc.Plan(blob, device=0)
    st = plan.stats()
    alg = algorithmic_bytes(wl.n, st["stream_bits"], st["n_groups"], layout, 8, False)
    tm = time_decode(torch, wc, plan, blob, wl.bits.view("int16"), 2, False, args, stream)
    plan.close()
    frac = alg / (tm["kernel_avg_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS
    return {"kernel": "decode_kernel (per-chunk gaps; count, DPP scan, decode)" if layout == "chunks" else
            "decode_lanes_kernel", "container_bytes": int(blob.size), "algorithmic_bytes_per_launch": alg,
            "ms": round(tm["kernel_avg_ms"], 5), "decompressed_GBps": round(2 * wl.n / (tm["kernel_avg_ms"] * 1e-3)
                                                                            / 1e9, 1),
            "frac": round(frac, 4), "bit_exact": tm["bit_exact"], "launch_us": tm["launch_us"],
            "rotating_copies": tm["copies"], "traffic": recorded_traffic(args.workload, layout),
            "host_prep_s": round(t, 2)}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: the decode runs on one GPU only (it is per-GPU and needs no collectives); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(args)
        return
    if args.e2e:
        end_to_end(args)
        return

    from lossless_entropy_coded_amd import wc
    from lossless_entropy_coded_amd.synth import CODE_WORKLOADS, make_code_workload, make_workload, workload_spec

    # bf16 weights (the exponent coded, sm raw) or a plane of 8-bit quantized
    # codes (every byte coded; lanes layout only)
    codes = args.workload in CODE_WORKLOADS
    if (codes or args.coder != "huffman") and args.layout != "lanes":
        print("bench.py: code planes and the rANS coder use the lanes layout", file=sys.stderr)
        sys.exit(2)
    if args.gap_bits != 8 and args.layout != "chunks":
        print("bench.py: --gap-bits applies to the chunks layout", file=sys.stderr)
        sys.exit(2)
    progress(f"{args.workload}: generating and encoding ({args.layout}, {args.coder})")
    t_gen = time.perf_counter()
    if codes:
        wl = make_code_workload(args.workload)
        blob = wc.encode_u8_host(wl.tensors(), coder=args.coder, **code_len_opt(args))
        raw, out_bytes = wl.codes, 1
    else:
        wl = make_workload(args.workload)
        blob = wc.encode_host(wl.tensors(), layout=args.layout, coder=args.coder, **code_len_opt(args))
        raw, out_bytes = wl.bits.view(np.int16), 2
    t_gen = time.perf_counter() - t_gen
    n = wl.n
    plan = wc.Plan(blob, device=0)
    st = plan.stats()
    stream_bits = st["stream_bits"]
    alg_bytes = algorithmic_bytes(n, stream_bits, st["n_groups"], args.layout, args.gap_bits, codes)
    stream = torch.cuda.current_stream()
    progress(f"{args.workload}: timing {args.steps} decode launches")
    tm = time_decode(torch, wc, plan, blob, raw, out_bytes, codes, args, stream)
    total_ms = tm["total_ms"]
    # the decode entry point's launches per call (the library's own split: a
    # large bf16 container takes several launches of whole grid rounds);
    # bytes and time per launch are the step's shares
    launches = max(1, plan.decode_shape()["launches"])
    kernel_avg_ms = tm["kernel_avg_ms"] / launches
    alg_bytes_launch = alg_bytes // launches
    ms_per_step = total_ms / args.steps
    value = out_bytes * n / (ms_per_step * 1e-3) / 1e9
    achieved = alg_bytes_launch / (kernel_avg_ms * 1e-3) / 1e9
    progress(f"{args.workload}: timing the streaming reference")
    sref = stream_reference(torch, wc, alg_bytes - out_bytes * n, out_bytes * n, args.steps, stream)

    extras = (args.extras == "on" and args.workload == "block_8b" and args.layout == "lanes"
              and args.coder == "huffman" and not args.max_code_len)
    layouts = e2e = None
    if extras:
        progress(f"{args.workload}: timing the chunks layout")
        layouts = {"chunks": layout_record(torch, wc, wl, "chunks", args, stream)}
        rec, ok = e2e_measure(torch, wc, "block_70b", "lanes", "huffman", args.steps, args.warmup, {}, stream)
        if not ok:
            print(f"bench.py: 70B-block arms disagree: {json.dumps(rec)}", file=sys.stderr)
            sys.exit(3)
        e2e = rec

    cpu = None
    if args.cpu_baseline == "on":
        progress(f"{args.workload}: timing the CPU oracle")
        import oracle
        reps, spent = 0, 0.0
        while reps < 1 or (spent < 10.0 and reps < 8):
            t = time.perf_counter()
            dec = oracle.decode_u8(blob) if codes else oracle.decode(blob)
            spent += time.perf_counter() - t
            reps += 1
            assert np.array_equal(dec, wl.codes if codes else wl.bits)
        cpu = {"value": round(out_bytes * n * reps / spent / 1e9, 4), "unit": "GB/s", "cores": 1,
               "cpu_model": cpu_model(), "kind": "oracle",
               "sample": f"the whole {args.workload} container ({n} elements) decoded {reps} times by the serial "
                         f"{'rANS decoder (linear slot search)' if args.coder == 'rans' else 'bit-by-bit trie decoder'} "
                         f"with every container check: {spent:.1f} s on one host core"}

    desc = CODE_WORKLOADS[args.workload][0] if codes else workload_spec(args.workload)[0]
    line = {
        "metric": METRIC_CODES if codes else METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32",
        "data": ("synthetic: seeded quantized-code planes (rounded, clipped Gaussians), 8B-block matrix shapes"
                 if codes else "synthetic: seeded bf16 weights, transformer-block shapes and distributions"),
        "config": {
            "workload": f"{args.workload}: {desc}",
            "layout": args.layout,
            "coder": args.coder,
            "max_code_len": args.max_code_len or None,
            "gap_bits": args.gap_bits if args.layout == "chunks" else None,
            "n_elems": n,
            "n_tensors": len(wl.numels),
            "container_bytes": int(blob.size),
            "compression_ratio": round(out_bytes * n / blob.size, 4),
            "mean_code_bits": round(stream_bits / n, 4),
            "launches_per_step": launches,
            "count_bits": st["count_bits"],
            "decode_bits": st["decode_bits"],
            "grid": st["grid"],
            "lds_bytes": st["lds_bytes"],
            "rotating_copies": tm["copies"],
            "rotated_bytes": tm["rotated_bytes"],
            "settle_launches": tm["settle_launches"],
            "timed_outputs_checked": tm["timed_outputs_checked"],
            "bit_exact": tm["bit_exact"],
            "host_prep_s": round(t_gen, 2),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(args.workload, args.layout, args.coder, args.gap_bits),
            "algorithmic_bytes_per_launch": alg_bytes_launch,
            "kernel_avg_ms": round(kernel_avg_ms, 5),
            "launch_us": tm["launch_us"],
            "stream_ref": sref,
            "frac_of_stream_ref": round(achieved / sref["GBps"], 4) if sref else None,
        },
        "cpu_baseline": cpu,
    }
    if layouts is not None:
        if sref:
            for rec in layouts.values():
                rec["frac_of_stream_ref"] = round(rec["algorithmic_bytes_per_launch"] / (rec["ms"] * 1e-3) / 1e9
                                                  / sref["GBps"], 4)
        line["layouts"] = layouts
    if e2e is not None:
        line["e2e"] = e2e
    print(json.dumps(line), flush=True)
    plan.close()


if __name__ == "__main__":
    main()
