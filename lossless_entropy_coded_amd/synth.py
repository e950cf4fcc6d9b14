"""Seeded synthetic bf16 weight generators.

This module holds no part of the codec: it only draws random weights with the
shapes and value distributions of the workloads below and rounds them to bf16
bit patterns.  Both the HIP path's tests/bench and the CPU oracle's tests take
their inputs from here, so that neither side generates data for the other.

The trained checkpoints that the pages measure on (Llama2-7B in "From a
Lossless (~1.5:1) Compression Algorithm for Llama2 7B Weights ...", abstract;
Llama-3.1 / Qwen-2.5 / Gemma-3 in "70% Size, 100% Accuracy: Lossless LLM
Compression ... Dynamic-Length Float", abstract) are not available, so seeded
Gaussian / Student-t tensors of the same transformer shapes stand in for them.

Recipe (fixed, so that every run reproduces the same bits):
  * ``numpy.random.default_rng(seed)``;
  * float32 draws: ``standard_normal(dtype=float32) * float32(sigma)`` (+ mean);
    Student-t draws come from ``standard_t`` in float64 and are cast to float32;
  * float32 -> bf16 by round-to-nearest-even on the integer bit pattern;
  * tensors are generated in the listed order, each row-major (out x in), and
    concatenated into one flat uint16 array (the element space of a block).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_rne",
    "gemv_input",
    "Workload",
    "WORKLOADS",
    "make_workload",
    "workload_spec",
]


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (round to nearest, ties to even).

    Works on the integer bit pattern: add 0x7FFF plus the lowest kept bit, then
    drop the low 16 bits.  Inputs here are finite, so no NaN special case is
    needed (a NaN input would still map to a NaN or inf pattern).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


@dataclass(frozen=True)
class TensorSpec:
    name: str
    shape: tuple
    mean: float = 0.0
    sigma: float = 0.02

    @property
    def numel(self) -> int:
        n = 1
        for d in self.shape:
            n *= int(d)
        return n


@dataclass
class Workload:
    """A generated workload: flat bf16 bits plus the tensor partition."""

    name: str
    bits: np.ndarray                      # uint16[n], all tensors concatenated
    names: list = field(default_factory=list)
    shapes: list = field(default_factory=list)
    numels: list = field(default_factory=list)

    @property
    def n(self) -> int:
        return int(self.bits.size)

    def tensors(self):
        """Views of the flat array, one per tensor, in order."""
        out, off = [], 0
        for k in self.numels:
            out.append(self.bits[off:off + k])
            off += k
        return out


def _block_8b():
    d, kv, ff = 4096, 1024, 14336
    return [
        TensorSpec("q_proj", (d, d)),
        TensorSpec("k_proj", (kv, d)),
        TensorSpec("v_proj", (kv, d)),
        TensorSpec("o_proj", (d, d)),
        TensorSpec("gate_proj", (ff, d)),
        TensorSpec("up_proj", (ff, d)),
        TensorSpec("down_proj", (d, ff)),
        TensorSpec("attn_norm", (d,), mean=1.0, sigma=0.05),
        TensorSpec("mlp_norm", (d,), mean=1.0, sigma=0.05),
    ]


def _block_70b():
    d, kv, ff = 8192, 1024, 28672
    s = 0.015
    return [
        TensorSpec("q_proj", (d, d), sigma=s),
        TensorSpec("k_proj", (kv, d), sigma=s),
        TensorSpec("v_proj", (kv, d), sigma=s),
        TensorSpec("o_proj", (d, d), sigma=s),
        TensorSpec("gate_proj", (ff, d), sigma=s),
        TensorSpec("up_proj", (ff, d), sigma=s),
        TensorSpec("down_proj", (d, ff), sigma=s),
    ]


# name -> (description, seed, tensor specs, extra structure)
WORKLOADS = {
    "matrix_1k": ("single 1024x1024 matrix, N(0, 0.02)", 0,
                  [TensorSpec("w", (1024, 1024))], None),
    "attn_4k_zeros": ("4096x4096 attention projection, N(0, 0.02) with 0.5% exact +0", 1,
                      [TensorSpec("w", (4096, 4096))], "zeros_0.5pct"),
    "block_8b": ("8B-shape transformer block: q,k,v,o,gate,up,down + 2 RMSNorm vectors", 2,
                 _block_8b(), None),
    "heavy_tail_14k": ("14336x4096 Student-t(3)*0.01 with 1% +0, 0.01% subnormals, 0.1% x50 outliers", 3,
                       [TensorSpec("w", (14336, 4096), sigma=0.01)], "heavy_tail"),
    "block_70b": ("70B-shape transformer block: q,k,v,o,gate,up,down, N(0, 0.015)", 4,
                  _block_70b(), None),
}


def workload_spec(name: str):
    desc, seed, specs, extra = WORKLOADS[name]
    return desc, seed, specs, extra


def _heavy_tail(rng, spec: TensorSpec) -> np.ndarray:
    n = spec.numel
    t = rng.standard_t(3.0, size=n).astype(np.float32) * np.float32(spec.sigma)
    perm = rng.permutation(n)
    n_zero, n_sub, n_out = n // 100, n // 10000, n // 1000
    zero_idx = perm[:n_zero]
    sub_idx = perm[n_zero:n_zero + n_sub]
    out_idx = perm[n_zero + n_sub:n_zero + n_sub + n_out]
    t[out_idx] *= np.float32(50.0)
    bits = f32_to_bf16_rne(t)
    bits[zero_idx] = 0
    sign = rng.integers(0, 2, size=n_sub, dtype=np.uint16) << np.uint16(15)
    mant = rng.integers(1, 128, size=n_sub, dtype=np.uint16)
    bits[sub_idx] = sign | mant          # exponent field 0, mantissa 1..127
    return bits


def gemv_input(cols: int, seed: int = 4) -> np.ndarray:
    """The batch-1 input of a GEMV over a block's matrix with `cols` columns:
    x ~ N(0, 1) in float32, rounded to bf16 (RNE); drawn from
    ``numpy.random.default_rng([seed, cols])`` so that every in-dimension has
    its own fixed vector."""
    rng = np.random.default_rng([seed, cols])
    return f32_to_bf16_rne(rng.standard_normal(cols, dtype=np.float32))


def make_workload(name: str, scale_rows: int | None = None) -> Workload:
    """Generate workload ``name``.

    ``scale_rows`` (optional) truncates every 2-D tensor to at most that many
    rows; it is used only to build small cases with the same distributions.
    """
    desc, seed, specs, extra = WORKLOADS[name]
    rng = np.random.default_rng(seed)
    parts, names, shapes, numels = [], [], [], []
    for spec in specs:
        shape = spec.shape
        if scale_rows is not None and len(shape) == 2:
            shape = (min(shape[0], scale_rows), shape[1])
        spec = TensorSpec(spec.name, shape, spec.mean, spec.sigma)
        n = spec.numel
        if extra == "heavy_tail":
            b = _heavy_tail(rng, spec)
        else:
            x = rng.standard_normal(n, dtype=np.float32) * np.float32(spec.sigma)
            if spec.mean != 0.0:
                x += np.float32(spec.mean)
            b = f32_to_bf16_rne(x)
            if extra == "zeros_0.5pct":
                idx = rng.choice(n, size=n // 200, replace=False)
                b[idx] = 0
        parts.append(b)
        names.append(spec.name)
        shapes.append(shape)
        numels.append(n)
    bits = np.concatenate(parts) if len(parts) > 1 else parts[0]
    return Workload(name=name, bits=bits, names=names, shapes=shapes, numels=numels)


# ---------------------------------------------------------------------------
# Planes of quantized integer codes (the setting of the LazyWeights page:
# Huffman codes for the already-quantized weights of a model).  No quantized
# model is available, so seeded stand-ins with the 8B-shape block's matrix
# shapes are drawn: a quantizer maps a weight to round(w / scale) and clips it
# to the code range; with the weights roughly Gaussian, a code is
# round(N(0, sigma)) clipped, sigma being the weights' spread in units of the
# scale (smaller sigma: more skewed codes).  Codes are stored unsigned with a
# zero point (code + 2^(bits - 1)); int4 codes are packed two per byte, the
# first in the low nibble.
# ---------------------------------------------------------------------------

# name -> (description, seed, bits per code, sigma)
CODE_WORKLOADS = {
    "int8_codes_8b": ("8B-shape block's 7 matrices as int8 codes: round(N(0, 20)) clipped to [-128, 127], "
                      "zero point 128, one byte per weight", 5, 8, 20.0),
    "int4_codes_8b": ("8B-shape block's 7 matrices as int4 codes: round(N(0, 1.5)) clipped to [-8, 7], "
                      "zero point 8, two per byte (low nibble first)", 6, 4, 1.5),
}


@dataclass
class CodeWorkload:
    """A generated plane of 8-bit symbols and its tensor partition."""

    name: str
    codes: np.ndarray                     # uint8[n], all tensors concatenated
    bits: int                             # bits per quantized code (8, or 4 packed in pairs)
    sigma: float
    names: list = field(default_factory=list)
    shapes: list = field(default_factory=list)   # byte shapes
    numels: list = field(default_factory=list)   # bytes per tensor

    @property
    def n(self) -> int:
        return int(self.codes.size)

    def tensors(self):
        out, off = [], 0
        for k in self.numels:
            out.append(self.codes[off:off + k])
            off += k
        return out


def quantized_codes(rng, n: int, bits: int, sigma: float) -> np.ndarray:
    """n codes of `bits` bits: round(N(0, sigma)) clipped to the signed range,
    plus the zero point 2^(bits - 1), as uint8."""
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    z = rng.standard_normal(n, dtype=np.float32) * np.float32(sigma)
    return (np.clip(np.rint(z), lo, hi).astype(np.int16) + (1 << (bits - 1))).astype(np.uint8)


def make_code_workload(name: str, scale_rows: int | None = None) -> CodeWorkload:
    desc, seed, bits, sigma = CODE_WORKLOADS[name]
    rng = np.random.default_rng(seed)
    parts, names, shapes, numels = [], [], [], []
    for spec in _block_8b():
        if len(spec.shape) != 2:
            continue
        rows, cols = spec.shape
        if scale_rows is not None:
            rows = min(rows, scale_rows)
        q = quantized_codes(rng, rows * cols, bits, sigma)
        if bits == 4:
            q = (q[0::2] | (q[1::2] << 4)).astype(np.uint8)
            shape = (rows, cols // 2)
        else:
            shape = (rows, cols)
        parts.append(q)
        names.append(spec.name)
        shapes.append(shape)
        numels.append(q.size)
    return CodeWorkload(name=name, codes=np.concatenate(parts), bits=bits, sigma=sigma, names=names,
                        shapes=shapes, numels=numels)
