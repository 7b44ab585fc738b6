"""Helpers for the GPU tests (device transfer, tolerance checks)."""

import sys

import numpy as np
import pytest

# Bars: normwise relative error of fp16 outputs and of the fp32 intermediate
# before rounding against the oracle.
TOL_FP16 = 2e-2
TOL_FP32_PRE = 1e-3


def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def to_dev(a):
    torch = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_np(t):
    return t.detach().cpu().numpy()


def bits(t):
    return to_np(t).view(np.uint16)


def note(msg):
    """Name the case on stdout before a GPU step (flushed)."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()
