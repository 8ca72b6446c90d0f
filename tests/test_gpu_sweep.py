"""GPU parity over a seeded sweep of random shapes and position layouts, against the fp64 oracle.

Hand-picked cases (test_gpu_parity.py) cover the edges one by one; this sweep draws, from one fixed seed, head
dimension, batch, ragged query and key counts (some a row either side of a tile boundary), mask, one or two
position segments per side in either order (so that the causal rule skips whole tiles between the two runs a
workgroup visits, on either side), positions near the top of the range, and the output dtype.  Each case runs
the forward and the backward through the C ABI (and, for the rotary cases, the fused-rotation entry points) and
meets the bars of every other parity test, with one reading: where the bf16 rounding of P and dS that the path
prescribes can itself move an element by more than 1e-2 (a few keys seen by hundreds of queries give gradients of
several units), that element is held to its rounding bound instead (tests/parity.py derives it, and
test_parity_bound.py checks it against an explicit emulation of those roundings); rel-L2 <= 5e-3 holds
throughout.  The case list is fixed by the seed: the same cases run every time.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea
import synth
from oracle.rope import rope, round_bf16
from tests.parity import assert_close, assert_lse, assert_within, banner, rounding_bounds, scale_of, seg_positions
from tests.test_gpu_parity import _run_dense

DEV = "cuda"
TOP = 2 ** 31


def _size(rng):
    if rng.random() < 0.3:  # a row either side of a tile boundary, or on it
        base = int(rng.choice([32, 64, 128, 256, 512, 1024]))
        return base + int(rng.integers(-1, 2))
    return int(rng.integers(1, 1300))


def _segments(rng, n, hi):
    """(start0, len0[, start1, len1]) for n rows, starts below hi, the second run anywhere (also before the first)."""
    if n >= 2 and rng.random() < 0.5:
        a = int(rng.integers(1, n))
        s0, s1 = (int(x) for x in rng.integers(0, hi, 2))
        return [s0, a, s1, n - a]
    return [int(rng.integers(0, hi)), n]


def _draw_cases(seed, count, rope):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(count):
        D = int(rng.choice([64, 128]))
        B = int(rng.choice([1, 1, 2]))
        sq, sk = _size(rng), _size(rng)
        causal = bool(rng.random() < 0.75)
        span = 2 * max(sq, sk)
        k_seg = _segments(rng, sk, span)
        q_seg = _segments(rng, sq, span + span // 2)
        if rng.random() < 0.15:  # the same layout moved to the top of the position range
            off = TOP - 4 * span
            k_seg = [x + off if i % 2 == 0 else x for i, x in enumerate(k_seg)]
            q_seg = [x + off if i % 2 == 0 else x for i, x in enumerate(q_seg)]
        o_dtype = torch.bfloat16 if (not rope and rng.random() < 0.2) else torch.float32
        theta = float(rng.choice([1e4, 1e6, 1e9])) if rope else None
        cases.append((D, B, sq, sk, causal, q_seg, k_seg, o_dtype, theta))
    return cases


DENSE = _draw_cases(20261203, 40, rope=False)
ROPE = _draw_cases(20261204, 12, rope=True)


def test_drawn_cases_are_valid():
    """Every drawn layout is one the interface accepts: lengths add up, every position below 2^31."""
    for D, B, sq, sk, causal, q_seg, k_seg, o_dtype, theta in DENSE + ROPE:
        for seg, n in ((q_seg, sq), (k_seg, sk)):
            assert sum(seg[1::2]) == n and len(seg) in (2, 4)
            assert all(s >= 0 and s + ln <= TOP for s, ln in zip(seg[0::2], seg[1::2]))


def test_drawn_cases_cover_the_features():
    """The fixed draws include what the module docstring promises: both head dimensions and masks, batches of
    two, two-run layouts with the second run first (on the query and on the key side), positions near 2^31,
    counts a row either side of a tile boundary, bf16 outputs, and each rotary base."""
    def two_runs_reversed(seg):
        return len(seg) == 4 and seg[2] < seg[0]
    for cases in (DENSE, ROPE):
        assert {c[0] for c in cases} == {64, 128} and {c[4] for c in cases} == {True, False}
        assert any(c[1] == 2 for c in cases)
    assert any(two_runs_reversed(c[5]) for c in DENSE) and any(two_runs_reversed(c[6]) for c in DENSE)
    assert any(c[5][0] > TOP // 2 for c in DENSE) and any(c[5][0] > TOP // 2 for c in ROPE)
    assert any(n % 32 in (1, 31) for c in DENSE for n in (c[2], c[3]))
    assert any(c[7] == torch.bfloat16 for c in DENSE)
    assert {c[8] for c in ROPE} == {1e4, 1e6, 1e9}
    assert any(len(b) == 4 for *_, b, _ in SPLIT) and any(b[i] == b[i + 1] for *_, b, _ in SPLIT for i in range(len(b) - 1))


@pytest.mark.gpu
@pytest.mark.parametrize("case", DENSE, ids=[f"dense{i}" for i in range(len(DENSE))])
def test_dense_sweep(case):
    D, B, sq, sk, causal, q_seg, k_seg, o_dtype, _ = case
    banner(f"D={D} B={B} Sq={sq} Sk={sk} causal={causal} q_seg={q_seg} k_seg={k_seg} o={o_dtype}")
    H = 2
    seed = 7000 + 10 * (sq + 3 * sk)
    q, k, v, do = (synth.normal_draw((B, s, H, D), seed + i, 1.0, DEV).to(torch.bfloat16)
                   for i, s in enumerate((sq, sk, sk, sq)))
    res = _run_dense(q, k, v, do, q_seg, k_seg, causal, o_dtype)
    pq, pk, scale = seg_positions(q_seg), seg_positions(k_seg), scale_of(D)
    ref = oracle.attn_bwd_heads(q, k, v, do, pq, pk, causal, scale)
    bound = rounding_bounds(q, k, v, do, pq, pk, causal, scale, ref)
    if o_dtype == torch.bfloat16:  # a bf16 output carries its own rounding: its rel-L2 only
        assert_close("O(bf16)", res["o"], ref["o"], max_abs=float("inf"))
    else:
        assert_within("O", res["o"], ref["o"], bound["o"])
    assert_lse("LSE", res["lse"], ref["lse"])
    for name in ("dq", "dk", "dv"):
        assert_within(name, res[name], ref[name], bound[name])


@pytest.mark.gpu
@pytest.mark.parametrize("case", ROPE, ids=[f"rope{i}" for i in range(len(ROPE))])
def test_rope_sweep(case):
    """Keys turned by ea_rope, queries turned inside the forward (which also writes them out for the backward),
    dQ and dK turned back inside the backward: against the oracle's attention on the unrotated rows."""
    D, B, sq, sk, causal, q_seg, k_seg, _, theta = case
    banner(f"rope D={D} B={B} Sq={sq} Sk={sk} causal={causal} q_seg={q_seg} k_seg={k_seg} theta={theta:g}")
    H = 2
    seed = 8000 + 10 * (sq + 3 * sk)
    q, k, v, do = (synth.normal_draw((B, s, H, D), seed + i, 1.0, DEV).to(torch.bfloat16)
                   for i, s in enumerate((sq, sk, sk, sq)))
    kr = torch.empty_like(k)
    ea.ea_rope(k, kr, k_seg, theta)
    f32 = lambda *s: torch.zeros(*s, device=DEV)
    o, lse, delta = f32(B, sq, H, D), f32(B, sq, H), f32(B, sq, H)
    dq, dk, dv = f32(B, sq, H, D), f32(B, sk, H, D), f32(B, sk, H, D)
    q_rot = torch.empty_like(q)
    ea.ea_attn_fwd_rope(q, kr, v, o, lse, q_seg, k_seg, theta, q_rot=q_rot, causal=causal)
    ea.ea_attn_bwd_rope(q_rot, kr, v, o, do, lse, delta, dq, dk, dv, q_seg, k_seg, theta, causal)
    torch.cuda.synchronize()
    pq, pk, scale = seg_positions(q_seg), seg_positions(k_seg), scale_of(D)
    ref = oracle.attn_bwd_rope_heads(q, k, v, do, pq, pk, causal, scale, theta)
    # the bound on the turned bf16 rows; turning dQ and dK back mixes dims d and d + D/2 of a row
    qr, kr_ref = (round_bf16(rope(x.cpu().double().numpy(), p, theta)) for x, p in ((q, pq), (k, pk)))
    bound = rounding_bounds(qr, kr_ref, v, do, pq, pk, causal, scale,
                            oracle.attn_bwd_heads(qr, kr_ref, v, do, pq, pk, causal, scale))
    for name in ("dq", "dk"):
        pair = bound[name][..., :D // 2] + bound[name][..., D // 2:]
        bound[name] = np.concatenate([pair, pair], axis=-1)
    assert_within("O", o, ref["o"], bound["o"])
    assert_lse("LSE", lse, ref["lse"])
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_within(name, got, ref[name], bound[name])


# ---- the keys split into parts, as a ring visits them -------------------------------------------------------
def _slice_segments(seg, a, b):
    """The (start, len) runs of rows [a, b) of the layout `seg`."""
    out, row = [], 0
    for s, n in zip(seg[0::2], seg[1::2]):
        lo, hi = max(a, row), min(b, row + n)
        if hi > lo:
            out += [s + (lo - row), hi - lo]
        row += n
    return out or [0, 0]


def _draw_split_cases(seed, count):
    rng = np.random.default_rng(seed)
    cases = []
    for D, B, sq, sk, causal, q_seg, k_seg, _, _ in _draw_cases(seed, count, rope=False):
        cuts = sorted(int(x) for x in rng.integers(0, sk + 1, int(rng.choice([1, 2]))))  # parts may be empty
        bounds = [0] + cuts + [sk]
        order = [int(i) for i in rng.permutation(len(bounds) - 1)]
        cases.append((D, B, sq, sk, causal, q_seg, k_seg, bounds, order))
    return cases


SPLIT = _draw_split_cases(20261205, 16) + [
    # an empty part visited first (the forward writes -inf / 0, the first backward call still writes Delta),
    # and an empty part visited between two others
    (128, 1, 300, 200, True, [100, 300], [0, 200], [0, 0, 120, 200], [0, 1, 2]),
    (64, 2, 257, 190, True, [0, 257], [0, 90, 300, 100], [0, 90, 90, 190], [2, 1, 0]),
]


@pytest.mark.gpu
@pytest.mark.parametrize("case", SPLIT, ids=[f"split{i}" for i in range(len(SPLIT))])
def test_split_keys_sweep(case):
    """The keys cut into parts visited in a random order: the first part's forward, the others merged into the
    accumulator (ea_attn_fwd_merge); Delta written by the first backward call and reused; dQ accumulated over
    the parts, each part's dK and dV written through row views of the whole tensors.  Against the oracle's
    attention over all keys at once."""
    D, B, sq, sk, causal, q_seg, k_seg, bounds, order = case
    banner(f"split D={D} B={B} Sq={sq} Sk={sk} causal={causal} q_seg={q_seg} k_seg={k_seg} parts={bounds} "
           f"order={order}")
    H = 2
    seed = 9000 + 10 * (sq + 3 * sk)
    q, k, v, do = (synth.normal_draw((B, s, H, D), seed + i, 1.0, DEV).to(torch.bfloat16)
                   for i, s in enumerate((sq, sk, sk, sq)))
    f32 = lambda *s: torch.zeros(*s, device=DEV)
    o, lse, delta = f32(B, sq, H, D), f32(B, sq, H), f32(B, sq, H)
    dq, dk, dv = f32(B, sq, H, D), f32(B, sk, H, D), f32(B, sk, H, D)
    parts = [(bounds[i], bounds[i + 1], _slice_segments(k_seg, bounds[i], bounds[i + 1])) for i in order]
    for n, (a, b, seg) in enumerate(parts):
        call = ea.ea_attn_fwd if n == 0 else ea.ea_attn_fwd_merge
        call(q, k[:, a:b], v[:, a:b], o, lse, q_seg, seg, causal)
    for n, (a, b, seg) in enumerate(parts):
        ea.ea_attn_bwd(q, k[:, a:b], v[:, a:b], o, do, lse, delta, dq, dk[:, a:b], dv[:, a:b], q_seg, seg, causal,
                       delta_ready=n > 0)
    torch.cuda.synchronize()
    pq, pk, scale = seg_positions(q_seg), seg_positions(k_seg), scale_of(D)
    ref = oracle.attn_bwd_heads(q, k, v, do, pq, pk, causal, scale)
    bound = rounding_bounds(q, k, v, do, pq, pk, causal, scale, ref)
    assert_within("O", o, ref["o"], bound["o"])
    assert_lse("LSE", lse, ref["lse"])
    for name, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert_within(name, got, ref[name], bound[name])
