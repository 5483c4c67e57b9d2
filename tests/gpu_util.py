"""Shared helpers of the GPU parity tests (comparators and device checks)."""
import sys

import numpy as np
import pytest
import torch

TOL = 2e-2  # max |gpu - oracle| / max |oracle| per slice


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from speech_recognition_amd import _lib
    _lib.lib()  # fails loudly if the library is not built


def say(*a):
    print("[gpu]", *a, flush=True)
    sys.stdout.flush()


def rel_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.abs(g - o).max() / max(np.abs(o).max(), 1e-30))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy()
