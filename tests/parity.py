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


# ---- per-element bound of the kernels' rounding ------------------------------------------------------------
# The bars above are stated for the configured workloads.  Where a gradient element sums many large terms (a
# few keys seen by hundreds of queries), the bf16 rounding of P and dS that the path prescribes (the
# probabilities and dS enter the matrix products as bf16, products and sums in fp32) can by itself move an
# element by more than 1e-2.  A forward error analysis of that arithmetic bounds each element:
#   O_id      (u + g) sum_j P_ij |v_jd|                        (P rounded to bf16 in P V)
#   Delta_i   (u + g) sum_j P_ij |dP_ij| + g sum_d |dO_id O_id| (from the computed O, in fp32: P_ij rounds once
#                                                              for all d, so its error reaches Delta as dP_ij)
#   dS_ij     (u + h + g) |dS_ij| + P_ij (g sum_d |dO_id v_jd| + eDelta_i)
#                                                              (bf16 dS, the fp16 hand-over of P, fp32 dP - Delta)
#   dV_jd     (u + g) sum_i P_ij |dO_id|;  dK_jd  s sum_i edS_ij |q_id|;  dQ_id  s sum_j edS_ij |k_jd|
# with u = 2^-8 and h = 2^-11 the unit roundoffs of bf16 and fp16 and g = 2^-14 for the fp32 sums of at most a
# few thousand terms, the fp32 exponential and the fp32 row statistics (each below 1e-5 relative).
U_BF16 = 2.0 ** -8
U_F16 = 2.0 ** -11
G_FP32 = 2.0 ** -14


def rounding_bounds(q, k, v, do, pos_q, pos_k, causal, scale, ref):
    """Per-element bounds for O, dQ, dK, dV ([B,S,H,D] arrays) from the oracle's result `ref` on the same inputs."""
    Q, K, V, dO = (to_np(x) for x in (q, k, v, do))
    pos_q, pos_k = np.asarray(pos_q, dtype=np.int64), np.asarray(pos_k, dtype=np.int64)
    allowed = pos_k[None, :] <= pos_q[:, None] if causal else np.ones((len(pos_q), len(pos_k)), dtype=bool)
    out = {n: np.zeros(np.shape(ref[n])) for n in ("o", "dq", "dk", "dv")}
    B, _, H, _ = Q.shape
    for b in range(B):
        for h in range(H):
            lse = np.asarray(ref["lse"])[b, :, h]
            live = allowed & np.isfinite(lse)[:, None]
            S = scale * Q[b, :, h] @ K[b, :, h].T
            P = np.where(live, np.exp(np.where(live, S - np.where(np.isfinite(lse), lse, 0.0)[:, None], 0.0)), 0.0)
            aV, adO, aQ, aK = (np.abs(x[b, :, h]) for x in (V, dO, Q, K))
            eO = (U_BF16 + G_FP32) * (P @ aV)
            dP = dO[b, :, h] @ V[b, :, h].T
            eD = (U_BF16 + G_FP32) * (P * np.abs(dP)).sum(1) + G_FP32 * (adO * np.abs(np.asarray(ref["o"])[b, :, h])).sum(1)
            dS = P * (dP - np.asarray(ref["delta"])[b, :, h][:, None])
            edS = (U_BF16 + U_F16 + G_FP32) * np.abs(dS) + P * (G_FP32 * (adO @ aV.T) + eD[:, None])
            out["o"][b, :, h] = eO
            out["dv"][b, :, h] = (U_BF16 + G_FP32) * (P.T @ adO)
            out["dq"][b, :, h] = scale * (edS @ aK)
            out["dk"][b, :, h] = scale * (edS.T @ aQ)
    return out


def assert_within(name, got, ref, bound, max_abs=MAX_ABS, rel_l2=REL_L2):
    """rel-L2 <= rel_l2, and each element within max(max_abs, its rounding bound)."""
    mx, rel = report(name, got, ref)
    err = np.abs(to_np(got) - to_np(ref))
    lim = np.maximum(max_abs, bound)
    worst = float((err / lim).max()) if err.size else 0.0
    over = int((err > max_abs).sum())
    print(f"  {name}: max_abs={mx:.3e} rel_l2={rel:.3e} max err/limit={worst:.3f} (elements above {max_abs:g}: "
          f"{over}, max bound {float(np.max(bound)) if err.size else 0.0:.3e})", flush=True)
    assert worst <= 1.0, f"{name}: an element exceeds max({max_abs}, its rounding bound) by {worst:.3f}x"
    assert rel <= rel_l2, f"{name}: rel-L2 {rel:.3e} > {rel_l2}"
