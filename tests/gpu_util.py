"""Helpers for the GPU parity tests: moving seeded inputs to the device."""
import os
import sys
import time

import numpy as np
import pytest


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def to_dev_bf16(bits: np.ndarray, lda: int | None = None):
    """uint16 bf16 bit patterns [T x n] -> device bfloat16 tensor (optionally row-padded to lda)."""
    torch = torch_cuda()
    T, n = bits.shape
    if lda is None or lda == n:
        h = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
        return h.to("cuda").view(torch.bfloat16)
    buf = np.zeros((T, lda), dtype=np.uint16)
    buf[:, :n] = bits
    h = torch.from_numpy(buf.view(np.int16)).to("cuda").view(torch.bfloat16)
    return h[:, :n]


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


_PROGRESS = os.environ.get("KQ_TEST_PROGRESS", "")


def announce(msg: str) -> None:
    """Name the case on stdout (shown with -s) and, when KQ_TEST_PROGRESS names a file, append
    it there too: a captured run still writes that file as it goes."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
    if not _PROGRESS:
        return
    try:
        os.makedirs(os.path.dirname(os.path.abspath(_PROGRESS)), exist_ok=True)
        with open(_PROGRESS, "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")
    except OSError:
        pass
