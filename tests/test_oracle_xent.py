"""Pins of the cross-entropy oracle (CPU).

Independent checks: a hand-derived fixture, torch's fp64 cross_entropy and its
autograd (a library routine), closed forms (uniform logits, two classes) and
invariants (rows of the gradient sum to zero, a per-row shift leaves loss and
gradient unchanged, ignored rows are zero).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.xent import xent_fwd_bwd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_two_classes():
    case = json.load(open(os.path.join(GOLDEN, "xent_two_classes.json")))
    out = xent_fwd_bwd(np.array(case["logits"]), np.array(case["labels"]), case["grad_scale"])
    for k in ("lse", "loss", "grad"):
        np.testing.assert_allclose(out[k], np.array(case["expect"][k]), rtol=0, atol=1e-14)


@pytest.mark.parametrize("seed,n,v", [(0, 7, 5), (1, 16, 1000), (2, 3, 32000)])
def test_matches_torch_cross_entropy(seed, n, v):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 3.0, size=(n, v))
    y = rng.integers(0, v, size=n)
    y[::3] = -100
    g = 1.0 / max(1, int((y != -100).sum()))
    out = xent_fwd_bwd(x, y, g)
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    yt = torch.tensor(y)
    loss = torch.nn.functional.cross_entropy(xt, yt, reduction="none", ignore_index=-100)
    (loss.sum() * g).backward()
    np.testing.assert_allclose(out["loss"], loss.detach().numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out["grad"], xt.grad.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(out["lse"], torch.logsumexp(xt, dim=1).detach().numpy(), rtol=1e-13)


def test_uniform_logits_closed_form():
    v = 50
    x = np.full((2, v), 3.5)
    out = xent_fwd_bwd(x, np.array([7, 0]), 0.5)
    np.testing.assert_allclose(out["loss"], [math.log(v)] * 2, rtol=1e-14)
    np.testing.assert_allclose(out["lse"], [3.5 + math.log(v)] * 2, rtol=1e-14)
    expect = np.full((2, v), 0.5 / v)
    expect[0, 7] -= 0.5
    expect[1, 0] -= 0.5
    np.testing.assert_allclose(out["grad"], expect, atol=1e-15)


@pytest.mark.parametrize("a,b", [(0.3, -1.2), (-4.0, 6.0), (20.0, 20.0)])
def test_two_classes_softplus(a, b):
    out = xent_fwd_bwd(np.array([[a, b]]), np.array([0]))
    sp = max(b - a, 0.0) + math.log1p(math.exp(-abs(b - a)))
    sig = 1.0 / (1.0 + math.exp(-(b - a)))
    np.testing.assert_allclose(out["loss"][0], sp, rtol=1e-13)
    np.testing.assert_allclose(out["grad"][0], [-sig, sig], rtol=1e-12, atol=1e-15)


def test_invariants():
    rng = np.random.default_rng(5)
    x = rng.normal(0, 2, size=(9, 77))
    y = rng.integers(0, 77, size=9)
    y[4] = -100
    out = xent_fwd_bwd(x, y, 0.25)
    keep = y != -100
    np.testing.assert_allclose(out["grad"][keep].sum(axis=1), 0.0, atol=1e-14)
    assert np.all(out["grad"][~keep] == 0) and np.all(out["loss"][~keep] == 0)
    c = rng.normal(0, 10, size=(9, 1))
    sh = xent_fwd_bwd(x + c, y, 0.25)
    np.testing.assert_allclose(sh["loss"], out["loss"], atol=1e-12)
    np.testing.assert_allclose(sh["grad"], out["grad"], atol=1e-14)
    np.testing.assert_allclose(sh["lse"], out["lse"] + c[:, 0], rtol=1e-13)


def test_out_of_range_label_rejected():
    with pytest.raises(ValueError):
        xent_fwd_bwd(np.zeros((1, 4)), np.array([4]))
