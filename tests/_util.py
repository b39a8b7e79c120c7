"""Shared helpers of the test suite (no method arithmetic here)."""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_mi355x.h")


def header_functions():
    """Names of the functions the headers under ``include/`` declare."""
    import glob
    src = "\n".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\*?(moe_\w+)\s*\(", src, flags=re.M)))


def to_dev(a, device="cuda", dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def bf16_dev(bits, device="cuda"):
    import torch
    return to_dev(np.asarray(bits, dtype=np.uint16), device, torch.bfloat16)


def bf16_host(t):
    """bf16 device tensor -> fp64 numpy values."""
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16).astype(np.uint32).__lshift__(16) \
        .view(np.float32).astype(np.float64)


def bits_host(t):
    import torch
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def row_rel_err(got, ref):
    """Per-row relative L2 error ||got - ref|| / ||ref|| (rows of a 2-D array)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return num / np.maximum(den, 1e-300)


def assert_close_rows(got, ref, tol=2e-2, what=""):
    e = row_rel_err(got, ref)
    tot = np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    worst = int(np.argmax(e)) if e.size else -1
    assert e.size == 0 or e.max() <= tol, f"{what}: worst row {worst} rel err {e.max():.3e} > {tol}"
    assert tot <= tol, f"{what}: whole-tensor rel err {tot:.3e} > {tol}"
    return float(e.max()) if e.size else 0.0, float(tot)


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place between two arrays of finite bf16 bit patterns."""
    def key(b):
        b = np.asarray(b, np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))
