"""Helpers for the GPU parity tests: device buffers with guard bands."""
from __future__ import annotations

import sys

import numpy as np

CANARY = 0x5A5A
GUARD = 256          # guard elements on each side of the output (512 B)


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device_aligned(blob: np.ndarray, align: int = 256):
    """Copy host bytes to a device uint8 tensor whose data starts 256-byte aligned.

    Returns (owner, view); keep `owner` alive while `view` is used."""
    import torch
    owner = torch.empty(blob.size + align, dtype=torch.uint8, device="cuda")
    off = (-owner.data_ptr()) % align
    view = owner[off:off + blob.size]
    if blob.size:
        view.copy_(torch.from_numpy(np.ascontiguousarray(blob)))
    assert view.data_ptr() % align == 0
    return owner, view


class GuardedOutput:
    """n bf16 words on the device framed by canary guard bands."""

    def __init__(self, n: int):
        import torch
        self.n = n
        self.buf = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.int16, device="cuda")
        self.out = self.buf[GUARD:GUARD + n]
        assert self.out.data_ptr() % 16 == 0

    def guards_intact(self) -> bool:
        import torch
        return bool((self.buf[:GUARD] == CANARY).all().item() and (self.buf[GUARD + self.n:] == CANARY).all().item())

    def host(self) -> np.ndarray:
        return self.out.cpu().numpy().view(np.uint16)


def gpu_decode(wc, blob: np.ndarray, plan=None, stream=None) -> np.ndarray:
    """Plan (if needed), upload, decode in one launch, check the guards, return host uint16."""
    import torch
    own = plan is None
    if own:
        plan = wc.Plan(blob)
    try:
        _, dblob = to_device_aligned(blob)
        out = GuardedOutput(plan.n_elems)
        wc.decode_async(plan, dblob, out.out, stream=stream)
        torch.cuda.synchronize()
        assert out.guards_intact(), "decode wrote outside its output range"
        return out.host()
    finally:
        if own:
            plan.close()
