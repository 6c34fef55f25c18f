"""Shared helpers for the GPU parity tests (no method arithmetic here)."""

import dataclasses
import math
import sys

import numpy as np
import torch

# Tolerances: bf16 in, fp32 accumulate.
O_TOL = 2e-2
LSE_TOL = 1e-3


def say(msg):
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(case, dev):
    kw = {}
    for f in dataclasses.fields(case):
        v = getattr(case, f.name)
        kw[f.name] = v.to(dev) if isinstance(v, torch.Tensor) else v
    return type(case)(**kw)


def np_i(t):
    return t.detach().cpu().numpy().astype(np.int64)


def np_f(t):
    return t.detach().to("cpu", torch.float64).numpy()


def max_err(got, ref):
    """Max |got - ref| treating matching infinities as equal and NaN as infinite error."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.shape != ref.shape:
        raise AssertionError(f"shape {got.shape} vs {ref.shape}")
    if np.isnan(got).any() or np.isnan(ref).any():
        return math.inf
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    with np.errstate(invalid="ignore"):
        d = np.where(both_inf, 0.0, np.abs(got - ref))
    return float(d.max()) if d.size else 0.0


def assert_close(name, got, ref, tol):
    e = max_err(got, ref)
    print(f"[err] {name}: max abs error {e:.3e} (tol {tol:.1e})", flush=True)
    assert e <= tol, f"{name}: max abs error {e:.3e} > {tol:.1e}"
    return e


def compact_pages(cache, page_table_np, kv_lens_np, page_size, rows):
    """Copy to the host only the pages that the given requests use.

    Returns (small cache as float64 numpy, page table rows renumbered into it).
    Values and the logical token order are unchanged, so the oracle sees the
    same keys as the GPU did.
    """
    used = []
    for b in rows:
        n = -(-int(kv_lens_np[b]) // page_size)
        used.append(page_table_np[b, :n])
    uniq = np.unique(np.concatenate(used)) if used else np.zeros(0, dtype=np.int64)
    small = np_f(cache[torch.as_tensor(uniq, device=cache.device)])
    remap = {int(p): i for i, p in enumerate(uniq)}
    width = page_table_np.shape[1]
    pt = np.zeros((len(rows), width), dtype=np.int64)
    for i, b in enumerate(rows):
        n = -(-int(kv_lens_np[b]) // page_size)
        pt[i, :n] = [remap[int(p)] for p in page_table_np[b, :n]]
    return small, pt
