"""GPU parity of the rotary embedding (ea_rope) and of the drivers that apply it, against the fp64 oracle.

Bars, from the arithmetic: angles are formed in fp64 on both sides, the GPU
rotates in fp32 and rounds once.  bf16 outputs must be within one bf16 rounding
of the fp64 value plus the fp32 error (|gpu - ref| <= 2^-8 |ref| + 1e-6 times
the length of the element's (x_k, x_{k+D/2}) pair, which bounds the error of a
result that cancels) and equal to the
oracle's own bf16 rounding except where the fp32 and fp64 values straddle a
rounding boundary (at most 0.1 % of elements); fp32 outputs within 1e-6 of the
length of their (x_k, x_{k+D/2}) pair.  The drivers with RoPE are held to the
attention bars (max-abs 1e-2, rel-L2 5e-3 on O, dQ, dK, dV; LSE 1e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea
import synth
from oracle.rope import rope, round_bf16
from tests.parity import assert_close, assert_lse, banner, scale_of, seg_positions

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _check_rotation(name, x, y, pos, theta, inverse):
    ref = rope(x, pos, theta, inverse=inverse)        # [B, S, H, D] fp64
    got = y.double().cpu().numpy()
    half = ref.shape[-1] // 2
    pair = np.sqrt(ref[..., :half] ** 2 + ref[..., half:] ** 2)
    pair = np.concatenate([pair, pair], axis=-1) + 1e-30
    if y.dtype == torch.bfloat16:
        # one rounding of the fp32 value, whose own error is relative to the pair length (cancellation)
        bound = 2.0 ** -8 * np.abs(ref) + 1e-6 * pair
        worst = float((np.abs(got - ref) / bound).max())
        mism = float(np.mean(got != round_bf16(ref)))
        print(f"  {name}: max err / bf16 bound {worst:.3f}, differs from oracle rounding in {mism:.2e}", flush=True)
        assert worst <= 1.0 and mism <= 1e-3
    else:
        worst = float((np.abs(got - ref) / pair).max())
        print(f"  {name}: max err / pair length {worst:.2e}", flush=True)
        assert worst <= 1e-6


CASES = [
    # B, S, H, D, dtype, seg, theta, inverse, in_place, batch_rows
    (1, 300, 3, 128, torch.bfloat16, [0, 300], 1e4, False, False, None),
    (2, 257, 4, 64, torch.bfloat16, [1000, 257], 1e6, False, True, 300),
    (1, 200, 2, 128, torch.bfloat16, [2 ** 31 - 150, 100, 5, 100], 1e9, False, False, None),
    (1, 129, 40, 128, torch.float32, [7, 129], 1e6, True, True, None),
    (3, 33, 1, 64, torch.float32, [0, 33], 1e4, False, False, 40),
    (1, 1, 32, 128, torch.bfloat16, [123456, 1], 1e6, False, False, None),
    (1, 1000, 32, 128, torch.float32, [600000, 500, 90000, 500], 1e9, True, False, None),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_rope_matches_oracle(case):
    B, S, H, D, dtype, seg, theta, inverse, in_place, br = case
    br = S if br is None else br
    banner(f"rope B={B} S={S} H={H} D={D} {dtype} seg={seg} theta={theta:g} inverse={inverse} in_place={in_place}")
    g = torch.Generator().manual_seed(S * 7 + H)
    parent = (torch.randn((B, br, H, D), generator=g) * 2.0).to(dtype)
    x_cpu = parent[:, :S].clone()
    xp = parent.to(DEV)
    x = xp[:, :S]
    if in_place:
        y, yp = x, xp
    else:
        yp = torch.full((B, br, H, D), float("nan"), dtype=dtype, device=DEV)
        y = yp[:, :S]
    ea.ea_rope(x, y, seg, theta, inverse=inverse)
    torch.cuda.synchronize()
    _check_rotation("rope", x_cpu, y, seg_positions(seg), theta, inverse)
    if br > S:  # rows of the parent outside the view are untouched
        pad = yp[:, S:].cpu()
        if in_place:
            assert torch.equal(pad, parent[:, S:])
        else:
            assert torch.isnan(pad.float()).all()
    if not in_place:
        assert torch.equal(x.cpu(), x_cpu)


def test_rope_inverse_undoes_forward():
    banner("rope inverse after forward, fp32")
    g = torch.Generator().manual_seed(5)
    x = torch.randn((1, 640, 8, 128), generator=g).to(DEV)
    y = x.clone()
    seg = [3, 320, 100000, 320]
    ea.ea_rope(y, y, seg, 1e6)
    ea.ea_rope(y, y, seg, 1e6, inverse=True)
    torch.cuda.synchronize()
    assert float((y - x).abs().max()) <= 2e-6 * float(x.abs().max())


def test_dense_causal_with_rope():
    B, S, H, D, theta = 1, 300, 2, 128, 1e6
    banner(f"DenseCausal rope theta={theta:g} S={S}")
    q, k, v, do = (synth.normal_draw((B, S, H, D), 900 + i, 1.0, DEV).to(torch.bfloat16) for i in range(4))
    drv = ea.DenseCausal(q, k, v, causal=True, rope_theta=theta)
    drv.step(do)
    torch.cuda.synchronize()
    pos = np.arange(S)
    ref = oracle.attn_bwd_rope_heads(q, k, v, do, pos, pos, True, scale_of(D), theta)
    assert_close("O", drv.o, ref["o"])
    assert_lse("LSE", drv.lse, ref["lse"])
    assert_close("dQ", drv.dq, ref["dq"])
    assert_close("dK", drv.dk, ref["dk"])
    assert_close("dV", drv.dv, ref["dv"])
    # the inputs are left unrotated
    assert torch.equal(drv.q_in, q) and torch.equal(drv.k_in, k)


@pytest.mark.parametrize("rank", [1, 2])
def test_zigzag_ring_with_rope(rank):
    W, C, H, D, theta = 4, 48, 2, 128, 1e9
    banner(f"zigzag ring rope W={W} C={C} rank={rank}")
    t = {n: synth.normal_draw((1, s, H, D), 950 + i, 1.0, DEV).to(torch.bfloat16) for i, (n, s) in
         enumerate((("q", 2 * C), ("k", 2 * W * C), ("v", 2 * W * C), ("do", 2 * C)))}
    drv = ea.ZigzagRingRank(t["q"], t["k"], t["v"], W, rank, rope_theta=theta)
    drv.step(t["do"])
    torch.cuda.synchronize()
    S = 2 * W * C
    pq = oracle.zigzag_positions(S, W, rank)
    pk = np.concatenate([oracle.zigzag_positions(S, W, s) for s in range(W)])
    ref = oracle.attn_bwd_rope_heads(t["q"], t["k"], t["v"], t["do"], pq, pk, True, scale_of(D), theta)
    assert_close("O", drv.o, ref["o"])
    assert_lse("LSE", drv.lse, ref["lse"])
    assert_close("dQ", drv.dq, ref["dq"])
    assert_close("dK", drv.dk, ref["dk"])
    assert_close("dV", drv.dv, ref["dv"])


FUSED_CASES = [
    # B, Sq, Sk, H, D, q_seg, k_seg, theta, causal
    (1, 300, 300, 2, 128, [0, 300], [0, 300], 1e6, True),
    (2, 257, 190, 3, 64, [5000, 257], [4900, 190], 1e4, True),
    (1, 200, 260, 2, 128, [2 ** 31 - 300, 100, 70000, 100], [2 ** 31 - 400, 130, 69990, 130], 1e9, True),
    (1, 96, 64, 1, 128, [640, 96], [0, 64], 1e6, False),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[f"fused{i}" for i in range(len(FUSED_CASES))])
def test_fused_rope_matches_separate_rotation(case):
    """ea_attn_fwd_rope / ea_attn_bwd_rope against ea_rope around ea_attn_fwd / ea_attn_bwd on the same inputs.

    The forward turns q with the same arithmetic as ea_rope, so q_rot, O and LSE must agree bit for bit (also
    merged into an accumulator).  The backward turns dQ, dK before adding them instead of after: dV and Delta are
    bit-identical, dQ and dK agree to fp32 rounding (1e-6 of the pair length), also after a second accumulating
    call."""
    B, sq, sk, H, D, qs, ks, theta, causal = case
    banner(f"fused rope B={B} Sq={sq} Sk={sk} H={H} D={D} q_seg={qs} k_seg={ks} theta={theta:g} causal={causal}")
    draw = lambda shape, seed: synth.normal_draw(shape, seed, 1.0, DEV).to(torch.bfloat16)
    q, do = draw((B, sq, H, D), 21), draw((B, sq, H, D), 22)
    k, v = draw((B, sk, H, D), 23), draw((B, sk, H, D), 24)
    qr, kr = torch.empty_like(q), torch.empty_like(k)
    ea.ea_rope(q, qr, qs, theta)
    ea.ea_rope(k, kr, ks, theta)
    f32 = lambda *s: torch.zeros(*s, device=DEV)
    o1, lse1, o2, lse2 = f32(B, sq, H, D), f32(B, sq, H), f32(B, sq, H, D), f32(B, sq, H)
    q_rot = torch.full_like(q, float("nan"))
    ea.ea_attn_fwd(qr, kr, v, o1, lse1, qs, ks, causal)
    ea.ea_attn_fwd_rope(q, kr, v, o2, lse2, qs, ks, theta, q_rot=q_rot, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(q_rot, qr), "q_rot differs from ea_rope"
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2), "fused forward differs from rotate-then-forward"
    # merged into an accumulator holding the first result: both paths again bit for bit
    ea.ea_attn_fwd_merge(qr, kr, v, o1, lse1, qs, ks, causal)
    ea.ea_attn_fwd_rope(q, kr, v, o2, lse2, qs, ks, theta, merge=True, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(lse1, lse2), "fused merging forward differs"
    # backward from the first forward's statistics
    ea.ea_attn_fwd(qr, kr, v, o1, lse1, qs, ks, causal)
    grads = [[f32(B, sq, H, D), f32(B, sk, H, D), f32(B, sk, H, D), f32(B, sq, H)] for _ in range(2)]
    for calls in (1, 2):
        for _ in range(calls if calls == 1 else 1):
            ea.ea_attn_bwd(qr, kr, v, o1, do, lse1, grads[0][3], grads[0][0], grads[0][1], grads[0][2], qs, ks,
                           causal)
            ea.ea_attn_bwd_rope(qr, kr, v, o1, do, lse1, grads[1][3], grads[1][0], grads[1][1], grads[1][2], qs, ks,
                                theta, causal)
        dq_sep, dk_sep = grads[0][0].clone(), grads[0][1].clone()
        ea.ea_rope(dq_sep, dq_sep, qs, theta, inverse=True)
        ea.ea_rope(dk_sep, dk_sep, ks, theta, inverse=True)
        torch.cuda.synchronize()
        assert torch.equal(grads[0][2], grads[1][2]) and torch.equal(grads[0][3], grads[1][3]), "dV or Delta differs"
        for name, sep, fused in (("dQ", dq_sep, grads[1][0]), ("dK", dk_sep, grads[1][1])):
            pair = torch.sqrt(sep[..., :D // 2] ** 2 + sep[..., D // 2:] ** 2).repeat(1, 1, 1, 2) + 1e-30
            worst = float(((fused - sep).abs() / pair).max())
            print(f"  {name} after {calls} call(s): max err / pair length {worst:.2e}", flush=True)
            assert worst <= 1e-6, name
