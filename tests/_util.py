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


BF16_ELEM_ALLOWANCE = 2.0 ** -8   # one bf16 ulp of the element: the output is a bf16 rounding


def elem_rms_ratio(got, ref, allowance=0.0):
    """Per row: max_j (|got - ref| - allowance * |ref|)+ / rms(ref row) (rows whose reference is all
    zero give 0 when got matches them exactly, else inf)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return np.zeros(ref.shape[:1])
    dev = np.max(np.maximum(np.abs(got - ref) - allowance * np.abs(ref), 0.0), axis=1)
    rms = np.sqrt(np.mean(ref * ref, axis=1))
    return np.where(rms > 0, dev / np.maximum(rms, 1e-300), np.where(dev == 0, 0.0, np.inf))


def close_rows_report(got, ref):
    """(worst row relative L2 error, whole-tensor relative error, worst elementwise |diff| / rms(row))."""
    e = row_rel_err(got, ref)
    tot = np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    el = elem_rms_ratio(got, ref)
    return (float(e.max()) if e.size else 0.0), float(tot), (float(el.max()) if el.size else 0.0)


def assert_close_rows(got, ref, tol=2e-2, what="", ulps=1):
    """Every row within ``tol`` in relative L2 error, the whole tensor too, and every element within
    ``tol`` of its row's rms beyond ``ulps`` bf16 ulps of itself:
    |got - ref| <= tol * rms(row) + ulps * 2^-8 * |ref|.  The outputs are bf16 roundings, so an element
    far above its row's rms carries that much rounding by itself (ulps = 1); a path with more bf16
    roundings that the two sides may take differently (the gate/up LoRA: gate, up, their folds and
    SiLU * up) allows one ulp per rounding.  A dropped or wrong element is off by about |ref| and is
    caught, not averaged away.  Prints the figures, the elementwise one with and without the allowance."""
    e = row_rel_err(got, ref)
    tot = np.linalg.norm(np.asarray(got, np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    raw = elem_rms_ratio(got, ref)
    el = elem_rms_ratio(got, ref, ulps * BF16_ELEM_ALLOWANCE)
    worst = int(np.argmax(e)) if e.size else -1
    print(f"  [{what}] rows {e.size}: worst row rel err {e.max() if e.size else 0:.3e}, tensor {tot:.3e}, "
          f"worst |diff|/rms(row) {raw.max() if raw.size else 0:.3e} "
          f"({el.max() if el.size else 0:.3e} beyond {ulps} bf16 ulp(s) of the element)", flush=True)
    assert e.size == 0 or e.max() <= tol, f"{what}: worst row {worst} rel err {e.max():.3e} > {tol}"
    assert tot <= tol, f"{what}: whole-tensor rel err {tot:.3e} > {tol}"
    if el.size:
        we = int(np.argmax(el))
        assert el.max() <= tol, (f"{what}: row {we} has an element {el.max():.3e} x rms(row) off beyond {ulps} "
                                 f"bf16 ulp(s) of itself (> {tol})")
    return float(e.max()) if e.size else 0.0, float(tot)


def bf16_ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place between two arrays of finite bf16 bit patterns."""
    def key(b):
        b = np.asarray(b, np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(key(a_bits) - key(b_bits))
