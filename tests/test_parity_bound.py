"""The per-element rounding bound of tests/parity.py against an explicit emulation of the rounding it covers.

The emulation applies, in fp64, exactly the roundings the bound accounts for: probabilities relative to the row
maximum rounded to bf16 in P V (the row sum from the unrounded values), Delta from that O, P rounded to bf16 for
dV, P handed over in fp16 (scaled by 2^14) and dS = P (dP - Delta) rounded to bf16 for dK, dS from the fp32 P
rounded to bf16 for dQ.  Its deviation from the oracle must lie inside the bound everywhere, and reach a
noticeable share of it somewhere (a bound that is never approached would pin nothing).
"""
import numpy as np
import pytest

import oracle
import synth
from oracle.rope import round_bf16
from tests.parity import rounding_bounds


def _bf16_inputs(shape, seed, std=1.0):
    return round_bf16(synth.normal_draw(shape, seed, std).double().numpy())


def _emulate_head(q, k, v, do, pos_q, pos_k, causal, scale):
    allowed = pos_k[None, :] <= pos_q[:, None] if causal else np.ones((len(pos_q), len(pos_k)), dtype=bool)
    S = np.where(allowed, scale * q @ k.T, -np.inf)
    has = allowed.any(1)
    m = np.where(has, S.max(1, initial=-np.inf), 0.0)
    pt = np.where(allowed, np.exp(np.where(allowed, S - m[:, None], 0.0)), 0.0)
    l = pt.sum(1)
    o = np.where(has[:, None], (round_bf16(pt) @ v) / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    delta = (do * o).sum(1)
    p = np.where(allowed, np.exp(np.where(allowed, S - np.where(has, lse, 0.0)[:, None], 0.0)), 0.0)
    dpm = do @ v.T - delta[:, None]
    p16 = (p * 2.0 ** 14).astype(np.float16).astype(np.float64) / 2.0 ** 14
    return {"o": o, "dv": round_bf16(p).T @ do, "dk": scale * round_bf16(p16 * dpm).T @ q,
            "dq": scale * round_bf16(p * dpm) @ k}


CASES = [
    # Sq, Sk, D, causal, q positions, k positions, std of v and dO
    (200, 12, 64, False, None, None, 1.0),      # a few keys seen by many queries: the largest gradients
    (150, 170, 64, True, (40, 150), (0, 170), 1.0),
    (96, 64, 128, True, (500, 96), (480, 64), 2.0),
    (64, 300, 64, True, (1000, 64), (700, 300), 1.0),  # many keys per query
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_bound_covers_emulated_rounding(case):
    sq, sk, D, causal, qp, kp, std = case
    pos_q = np.arange(sq) + (qp[0] if qp else 0)
    pos_k = np.arange(sk) + (kp[0] if kp else 0)
    seed = 31 * sq + sk
    q, k = _bf16_inputs((1, sq, 1, D), seed), _bf16_inputs((1, sk, 1, D), seed + 1)
    v, do = _bf16_inputs((1, sk, 1, D), seed + 2, std), _bf16_inputs((1, sq, 1, D), seed + 3, std)
    scale = D ** -0.5
    ref = oracle.attn_bwd_heads(q, k, v, do, pos_q, pos_k, causal, scale)
    bound = rounding_bounds(q, k, v, do, pos_q, pos_k, causal, scale, ref)
    em = _emulate_head(q[0, :, 0], k[0, :, 0], v[0, :, 0], do[0, :, 0], pos_q, pos_k, causal, scale)
    ratios = {}
    for name in ("o", "dq", "dk", "dv"):
        err = np.abs(em[name] - ref[name][0, :, 0])
        b = bound[name][0, :, 0]
        assert np.all(err <= b), f"{name}: emulated rounding exceeds the bound ({float((err / (b + 1e-300)).max()):.3f}x)"
        ratios[name] = float((err / (b + 1e-300)).max())
    print(ratios)
    assert max(ratios.values()) > 0.05, "the bound is never approached"


def test_bound_is_zero_without_rounded_terms():
    """Rows with no allowed key carry no error, and neither do keys no query sees."""
    sq, sk, D = 8, 8, 64
    q, k = _bf16_inputs((1, sq, 1, D), 1), _bf16_inputs((1, sk, 1, D), 2)
    v, do = _bf16_inputs((1, sk, 1, D), 3), _bf16_inputs((1, sq, 1, D), 4)
    pos_q, pos_k = np.arange(sq), np.arange(sk) + 4  # rows 0..3 see no key; keys 4..7 only some
    ref = oracle.attn_bwd_heads(q, k, v, do, pos_q, pos_k, True, D ** -0.5)
    bound = rounding_bounds(q, k, v, do, pos_q, pos_k, True, D ** -0.5, ref)
    assert np.all(bound["o"][0, :4] == 0) and np.all(bound["dq"][0, :4] == 0)
    assert np.all(bound["dk"] >= 0) and np.all(bound["dv"] >= 0)
