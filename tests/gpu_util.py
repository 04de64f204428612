"""Host <-> device helpers for the GPU parity tests (marshalling only)."""

from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

DEV = "cuda:0"
GUARD = 4096            # bytes of canary on each side of an output buffer
CANARY = 0xA5


def announce(case: str) -> None:
    """Name the case about to run on the GPU, flushed, so that a run that
    dies on the device still says which case it was in."""
    print(f"\n[gpu case] {case}", flush=True)
    sys.stdout.flush()


def bits_to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> int16 CUDA tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV)


def u8_to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(DEV)


def i8_to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int8)).to(DEV)


def f32_to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


class Guarded:
    """An output tensor inside a larger byte buffer whose margins hold a
    canary pattern; ``intact()`` reports whether the kernel wrote outside."""

    def __init__(self, shape, dtype):
        self.shape, self.dtype = tuple(shape), dtype
        n = int(np.prod(self.shape)) * torch.empty((), dtype=dtype).element_size()
        self.nbytes = n
        self.buf = torch.full((GUARD + n + GUARD,), CANARY, dtype=torch.uint8, device=DEV)
        self.t = self.buf[GUARD:GUARD + n].view(dtype).view(self.shape)

    def intact(self) -> bool:
        b = self.buf.cpu().numpy()
        return bool(np.all(b[:GUARD] == CANARY) and np.all(b[GUARD + self.nbytes:] == CANARY))


def oracle_workers() -> int:
    """Threads for running the oracle over bands of a large input (numpy
    releases the interpreter lock inside its array operations)."""
    return max(1, min(16, os.cpu_count() or 1))


def oracle_by_rows(fn, bits: np.ndarray, band: int):
    """fn applied to consecutive bands of `band` rows of `bits`, in parallel
    threads, with the bands' outputs concatenated along the rows.  fn returns
    (codes, scales); every row-wise quantizer, and the block quantizer with
    `band` a multiple of 128, is a function of its band alone (the oracle's
    shard-commutation pin), so the result is fn(bits)."""
    starts = list(range(0, bits.shape[0], band))
    with ThreadPoolExecutor(oracle_workers()) as ex:
        parts = list(ex.map(lambda r: fn(bits[r:r + band]), starts))
    return (np.concatenate([p[0] for p in parts], axis=0),
            np.concatenate([p[1] for p in parts], axis=0))
