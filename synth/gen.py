"""Seeded Gaussian draws rounded once to bf16.

Every tensor is drawn in fp32 from its own ``torch.Generator`` (seed =
``cfg.seed + 1000 * tensor_id + 10 * rank``; tensor ids Q=0, K=1, V=2, dO=3),
scaled by ``cfg.std`` and rounded once to bf16 (nearest even).  Q and K are the
unrotated projections: a workload with a rotary base has its rotation applied by
the code under test and, independently, by the oracle.

Tensors are laid out [B, S, H, D] (D contiguous).  Draws happen on ``device``:
CPU and GPU generators give different (each reproducible) streams, so a test
that compares two implementations always feeds both the same tensors.
"""
import torch

Q_ID, K_ID, V_ID, DO_ID = 0, 1, 2, 3


def normal_draw(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def make_dense_case(cfg, device="cpu", with_grad_input=True, S=None, H=None):
    """Q, K, V, dO for a whole-sequence causal workload (positions 0..S-1)."""
    S = cfg.S if S is None else S
    H = cfg.H if H is None else H
    shape = (cfg.B, S, H, cfg.D)
    out = {}
    for name, tid in (("q", Q_ID), ("k", K_ID), ("v", V_ID), ("do", DO_ID)):
        if name == "do" and not with_grad_input:
            continue
        x = normal_draw(shape, cfg.seed + 1000 * tid, cfg.std, device)
        out[name] = _bf16(x)
        del x
    return out


def make_ring_case(cfg, device="cpu", C=None, H=None, rank=None):
    """One rank's local Q and dO ([B, 2C, H, D]) and the global K and V ([B, 2WC, H, D]).

    The local rows are drawn directly (they stand for the rank's two chunks); which
    global positions they occupy is left to the code under test and to the oracle.
    """
    C = cfg.C if C is None else C
    H = cfg.H if H is None else H
    r = cfg.rank if rank is None else rank
    sq, sk = 2 * C, 2 * cfg.W * C
    out = {}
    out["q"] = _bf16(normal_draw((cfg.B, sq, H, cfg.D), cfg.seed + 1000 * Q_ID + 10 * r, cfg.std, device))
    out["k"] = _bf16(normal_draw((cfg.B, sk, H, cfg.D), cfg.seed + 1000 * K_ID, cfg.std, device))
    out["v"] = _bf16(normal_draw((cfg.B, sk, H, cfg.D), cfg.seed + 1000 * V_ID, cfg.std, device))
    out["do"] = _bf16(normal_draw((cfg.B, sq, H, cfg.D), cfg.seed + 1000 * DO_ID + 10 * r, cfg.std, device))
    return out
