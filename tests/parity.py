"""Shared helpers of the GPU parity tests (not a test module).

Bars: O, dQ, dK, dV within max-abs <= 1e-2 and relative L2 <= 5e-3 of the fp64
oracle (fp32 outputs compared, before any bf16 cast); LSE within 1e-3 where
finite, with -inf matching exactly.
"""
import math

import numpy as np
import torch

MAX_ABS = 1e-2
REL_L2 = 5e-3
LSE_ABS = 1e-3


def to_np(x):
    if isinstance(x, torch.Tensor):
        return x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def report(name, got, ref):
    got, ref = to_np(got), to_np(ref)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got - ref))
    return mx, rel


def assert_close(name, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2):
    mx, rel = report(name, got, ref)
    print(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e}", flush=True)
    assert mx <= max_abs, f"{name}: max-abs {mx:.3e} > {max_abs}"
    assert rel <= rel_l2, f"{name}: rel-L2 {rel:.3e} > {rel_l2}"


def assert_lse(name, got, ref, tol=LSE_ABS):
    got, ref = to_np(got), to_np(ref)
    ninf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf_ref), f"{name}: -inf pattern differs"
    fin = ~ninf_ref
    assert np.all(np.isfinite(got[fin])), f"{name}: non-finite where finite expected"
    mx = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    print(f"  {name}: max_abs={mx:.3e} (finite rows {int(fin.sum())}/{fin.size})", flush=True)
    assert mx <= tol, f"{name}: {mx:.3e} > {tol}"


def seg_positions(seg):
    """Positions of the rows described by (start0, len0[, start1, len1])."""
    parts = [seg[i] + np.arange(seg[i + 1], dtype=np.int64) for i in range(0, len(seg), 2)]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)


def banner(msg):
    print(f"\n[case] {msg}", flush=True)


def scale_of(D):
    return 1.0 / math.sqrt(D)
