"""Helpers shared by the GPU tests: device copies of seeded inputs and error measures."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

TOL = 2e-3   # max normwise relative error against the fp64 oracle

_records = []


def dev():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU (gfx950)"
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, bf16_bits: bool = False) -> torch.Tensor:
    if bf16_bits:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def normwise(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref| (0 when both are all zero)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(got - ref)) if ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)


def rms_rel(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    return float(np.sqrt(np.mean((got - ref) ** 2)) / den) if den > 0 else 0.0


def record(**kw):
    """Keep a parity figure (test, case, error); appended at the end of the session, one JSON object per
    line, to the file that the environment variable AQD_PARITY_REPORT names, if it names one."""
    _records.append(kw)


def flush_records():
    path = os.environ.get("AQD_PARITY_REPORT")
    if _records and path and os.path.isdir(os.path.dirname(os.path.abspath(path))):
        with open(path, "a") as f:
            for r in _records:
                f.write(json.dumps(r) + "\n")
    _records.clear()
