"""Pins of the rotary-embedding oracle (oracle/rope.py) against things other than itself."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle.rope import attn_bwd_rope, inv_freq, rope, round_bf16
from oracle.attention import attn_bwd

HERE = os.path.dirname(os.path.abspath(__file__))


def test_golden_quarter_turn():
    fx = json.load(open(os.path.join(HERE, "golden", "rope_d4_quarter_turn.json")))
    x = np.array(fx["x"], dtype=np.float64)[:, None, :]        # [S, H=1, D=4]
    got = rope(x, np.array(fx["positions"]), fx["theta"])[:, 0, :]
    np.testing.assert_allclose(got, np.array(fx["expect"]), rtol=0, atol=1e-12)
    back = rope(got[:, None, :], np.array(fx["positions"]), fx["theta"], inverse=True)[:, 0, :]
    np.testing.assert_allclose(back, np.array(fx["x"]), rtol=0, atol=1e-12)


def test_d2_is_complex_rotation():
    """D = 2: the pair (x0, x1) is the complex number x0 + i x1 multiplied by e^{i p} (frequency theta^0 = 1)."""
    rng = np.random.default_rng(0)
    pos = np.array([0, 1, 5, 1000, 2 ** 20 + 3])
    x = rng.standard_normal((len(pos), 3, 2))
    got = rope(x, pos, theta=123.0)
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos.astype(np.float64))[:, None]
    np.testing.assert_allclose(got[..., 0], z.real, atol=1e-12)
    np.testing.assert_allclose(got[..., 1], z.imag, atol=1e-12)


@pytest.mark.parametrize("D,theta", [(64, 1e4), (128, 1e6), (128, 1e9)])
def test_matches_transformers_llama(D, theta):
    """The Llama rotary embedding of the transformers library (fp32 angles, so small positions only)."""
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding, apply_rotary_pos_emb

    H, S = 2, 48
    cfg = LlamaConfig(hidden_size=H * D, num_attention_heads=H, rope_theta=theta, max_position_embeddings=4096)
    emb = LlamaRotaryEmbedding(config=cfg)
    g = torch.Generator().manual_seed(D)
    q = torch.randn((1, S, H, D), generator=g, dtype=torch.float64)
    k = torch.randn((1, S, H, D), generator=g, dtype=torch.float64)
    pos = torch.arange(7, 7 + S)
    cos, sin = emb(q, pos[None])
    qr, kr = apply_rotary_pos_emb(q, k, cos, sin, unsqueeze_dim=2)   # [B, S, H, D] layout
    np.testing.assert_allclose(rope(q.numpy(), pos.numpy(), theta), qr.numpy(), rtol=0, atol=2e-5)
    np.testing.assert_allclose(rope(k.numpy(), pos.numpy(), theta), kr.numpy(), rtol=0, atol=2e-5)


def test_orthogonal_and_inverse():
    rng = np.random.default_rng(1)
    pos = rng.integers(0, 2 ** 31 - 1, size=40)
    x = rng.standard_normal((2, 40, 3, 128))
    y = rope(x, pos, 1e9)
    # each (x_k, x_{k+D/2}) pair keeps its length
    n0 = x[..., :64] ** 2 + x[..., 64:] ** 2
    n1 = y[..., :64] ** 2 + y[..., 64:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    np.testing.assert_allclose(rope(y, pos, 1e9, inverse=True), x, atol=1e-12)
    np.testing.assert_allclose(rope(x, np.zeros(40, dtype=np.int64), 1e9), x, atol=0)


def test_scores_depend_on_position_difference_only():
    """<R(p) q, R(p') k> is unchanged when both positions move by the same amount."""
    rng = np.random.default_rng(2)
    q = rng.standard_normal((16, 1, 128))
    k = rng.standard_normal((16, 1, 128))
    pq = rng.integers(0, 10 ** 6, size=16)
    pk = rng.integers(0, 10 ** 6, size=16)
    for shift in (1, 977, 123456):
        a = np.einsum("ihd,jhd->ij", rope(q, pq, 1e6), rope(k, pk, 1e6))
        b = np.einsum("ihd,jhd->ij", rope(q, pq + shift, 1e6), rope(k, pk + shift, 1e6))
        np.testing.assert_allclose(a, b, atol=1e-8)


def test_inv_freq_closed_form():
    f = inv_freq(8, 1e4)
    np.testing.assert_allclose(f, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)


def test_round_bf16_against_torch_and_ties():
    # fp32-representable inputs: torch's fp32 -> bf16 cast (round to nearest even) is a single rounding
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * 10.0 ** rng.integers(-3, 4, 100000)).astype(np.float32).astype(np.float64)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(round_bf16(x), ref)
    # exact ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> the even one, 1
    assert round_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 1.0
    assert round_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert round_bf16(np.array([-(1.0 + 2.0 ** -8 + 2.0 ** -30)]))[0] == -(1.0 + 2.0 ** -7)
    assert round_bf16(np.array([0.0, -0.0, np.inf]))[2] == np.inf


def test_attention_gradient_through_rotation():
    """torch fp64 autograd through the rotation (as matrices) and softmax attention."""
    rng = np.random.default_rng(4)
    S, D, theta, scale = 12, 8, 100.0, 8 ** -0.5
    q, k, v, do = (round_bf16(rng.standard_normal((S, D))) for _ in range(4))
    pos = np.arange(40, 40 + S)
    out = attn_bwd_rope(q, k, v, do, pos, pos, True, scale, theta)

    def rot_mats(p):
        R = np.zeros((S, D, D))
        f = inv_freq(D, theta)
        h = D // 2
        for i in range(S):
            for kk in range(h):
                c, s = math.cos(p[i] * f[kk]), math.sin(p[i] * f[kk])
                R[i, kk, kk], R[i, kk, kk + h] = c, -s
                R[i, kk + h, kk + h], R[i, kk + h, kk] = c, s
        return torch.from_numpy(R)

    R = rot_mats(pos)
    # the oracle rounds the rotated rows to bf16; use the same rotated values, so the
    # gradient of the rounding (treated as identity) is what is compared
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    qr = torch.einsum("iab,ib->ia", R, tq)
    kr = torch.einsum("iab,ib->ia", R, tk)
    qr = qr + (torch.from_numpy(out["q_rot"]) - qr).detach()
    kr = kr + (torch.from_numpy(out["k_rot"]) - kr).detach()
    s = scale * qr @ kr.T
    mask = torch.from_numpy(pos[None, :] <= pos[:, None])
    p = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1)
    o = p @ torch.from_numpy(v)
    o.backward(torch.from_numpy(do))
    np.testing.assert_allclose(out["o"], o.detach().numpy(), atol=1e-12)
    np.testing.assert_allclose(out["dq"], tq.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(out["dk"], tk.grad.numpy(), atol=1e-10)
    # at position 0 nothing rotates: plain attention
    plain = attn_bwd(q, k, v, do, pos * 0, pos * 0, False, scale)
    zero = attn_bwd_rope(q, k, v, do, pos * 0, pos * 0, False, scale, theta)
    np.testing.assert_allclose(zero["dq"], plain["dq"], atol=1e-12)
