"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small and mid sizes that span several tiles with ragged tails, both masks, two
position segments, batch strides, bf16 and fp32 outputs, edge cases, and the
zigzag ring of one rank; full-size workloads live in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea
import synth
from tests.parity import assert_close, assert_lse, banner, scale_of, seg_positions, to_np

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _rand(shape, seed, std=1.0):
    return synth.normal_draw(shape, seed, std, DEV).to(torch.bfloat16)


def _sentinel(shape, dtype, pad=4096):
    """Tensor view with NaN guard bands before and after (to catch stray writes)."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device=DEV)
    return buf, buf[pad:pad + n].view(shape), pad


def _guards_intact(buf, pad):
    return bool(torch.isnan(buf[:pad].float()).all()) and bool(torch.isnan(buf[-pad:].float()).all())


def _run_dense(q, k, v, do, q_seg, k_seg, causal, o_dtype=torch.float32, scale=None):
    B, sq, H, D = q.shape
    sk = k.shape[1]
    scale = scale_of(D) if scale is None else scale
    ob, o, po = _sentinel((B, sq, H, D), o_dtype)
    lb, lse, pl = _sentinel((B, sq, H), torch.float32)
    ea.ea_attn_fwd(q, k, v, o, lse, q_seg, k_seg, causal, scale)
    dqb, dq, p1 = _sentinel((B, sq, H, D), torch.float32)
    dkb, dk, p2 = _sentinel((B, sk, H, D), torch.float32)
    dvb, dv, p3 = _sentinel((B, sk, H, D), torch.float32)
    dlb, delta, p4 = _sentinel((B, sq, H), torch.float32)
    dq.zero_(), dk.zero_(), dv.zero_()
    ea.ea_attn_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, q_seg, k_seg, causal, scale)
    torch.cuda.synchronize()
    for buf, pad in ((ob, po), (lb, pl), (dqb, p1), (dkb, p2), (dvb, p3), (dlb, p4)):
        assert _guards_intact(buf, pad), "write outside an output buffer"
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)


def _check_dense(res, q, k, v, do, q_seg, k_seg, causal, scale=None, o_tol=None):
    B, sq, H, D = q.shape
    scale = scale_of(D) if scale is None else scale
    pq, pk = seg_positions(q_seg), seg_positions(k_seg)
    ref = oracle.attn_bwd_heads(q, k, v, do, pq, pk, causal, scale)
    if res["o"].dtype == torch.bfloat16:
        # a bf16 output carries its own rounding (2^-9 relative): gate its rel-L2 only
        assert_close("O(bf16)", res["o"], ref["o"], max_abs=float("inf"))
    else:
        assert_close("O", res["o"], ref["o"])
    assert_lse("LSE", res["lse"], ref["lse"])
    assert_close("dQ", res["dq"], ref["dq"])
    assert_close("dK", res["dk"], ref["dk"])
    assert_close("dV", res["dv"], ref["dv"])
    return ref


def test_c1_all_heads():
    cfg = synth.get("c1")
    banner(f"{cfg.name}")
    t = synth.make_dense_case(cfg, DEV)
    res = _run_dense(t["q"], t["k"], t["v"], t["do"], [0, cfg.S], [0, cfg.S], True)
    _check_dense(res, t["q"], t["k"], t["v"], t["do"], [0, cfg.S], [0, cfg.S], True)


CASES = [
    # D, B, Sq, Sk, causal, q_seg, k_seg, o_dtype
    (128, 1, 200, 333, True, [133, 200], [0, 333], torch.float32),
    (128, 1, 333, 200, False, [0, 333], [0, 200], torch.float32),
    (64, 2, 257, 257, True, [0, 257], [0, 257], torch.float32),
    (128, 1, 300, 700, True, [50, 150, 550, 150], [0, 350, 350, 350], torch.float32),  # two segments each
    (128, 1, 128, 512, True, [0, 64, 448, 64], [0, 256, 256, 256], torch.bfloat16),
    (64, 1, 1, 1, True, [7, 1], [3, 1], torch.float32),
    (128, 1, 1, 450, True, [449, 1], [0, 450], torch.float32),
    (128, 1, 450, 1, True, [0, 450], [0, 1], torch.float32),
    (128, 1, 190, 190, True, [0, 190], [100, 190], torch.float32),  # rows 0..99 see no key
    (64, 3, 70, 130, False, [0, 70], [0, 130], torch.bfloat16),
    # positions at the top of the range (every position < 2^31)
    (128, 1, 300, 400, True, [2 ** 31 - 300, 300], [2 ** 31 - 500, 400], torch.float32),
    (64, 1, 200, 200, True, [2 ** 31 - 200, 100, 1000, 100], [2 ** 31 - 150, 150, 0, 50], torch.float32),
    # second segment before the first, so that the causal rule skips whole tiles between the two runs a
    # workgroup visits, far enough into its run for the loads to step over them: query tiles in dK/dV
    # (ragged Sq), key tiles in the forward and dQ (ragged Sk)
    (128, 1, 700, 600, True, [1000, 300, 0, 400], [0, 600], torch.float32),
    (128, 1, 1200, 700, True, [0, 1200], [1000, 400, 0, 300], torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_dense_cases(case):
    D, B, sq, sk, causal, q_seg, k_seg, o_dtype = case
    banner(f"D={D} B={B} Sq={sq} Sk={sk} causal={causal} q_seg={q_seg} k_seg={k_seg} o={o_dtype}")
    H = 3
    q, k, v, do = (_rand((B, s, H, D), 50 + i) for i, s in enumerate((sq, sk, sk, sq)))
    res = _run_dense(q, k, v, do, q_seg, k_seg, causal, o_dtype)
    _check_dense(res, q, k, v, do, q_seg, k_seg, causal)


def test_batch_row_stride_views():
    """Row sub-ranges of larger buffers (pointer offsets, parent batch stride)."""
    banner("views with batch_rows > S")
    B, S, H, D = 2, 300, 2, 128
    Q, K, V, DO = (_rand((B, S, H, D), 70 + i) for i in range(4))
    q, do = Q[:, 100:260], DO[:, 100:260]
    k, v = K[:, 40:290], V[:, 40:290]
    q_seg, k_seg = [100, 160], [40, 250]
    O = torch.zeros((B, S, H, D), device=DEV)
    LSE = torch.zeros((B, S, H), device=DEV)
    DQ = torch.zeros((B, S, H, D), device=DEV)
    DK = torch.zeros_like(DQ)
    DV = torch.zeros_like(DQ)
    DL = torch.zeros_like(LSE)
    ea.ea_attn_fwd(q, k, v, O[:, 100:260], LSE[:, 100:260], q_seg, k_seg, True)
    ea.ea_attn_bwd(q, k, v, O[:, 100:260], do, LSE[:, 100:260], DL[:, 100:260], DQ[:, 100:260], DK[:, 40:290],
                   DV[:, 40:290], q_seg, k_seg, True)
    torch.cuda.synchronize()
    assert float(O[:, :100].abs().max()) == 0 and float(O[:, 260:].abs().max()) == 0
    assert float(DK[:, :40].abs().max()) == 0 and float(DK[:, 290:].abs().max()) == 0
    ref = oracle.attn_bwd_heads(q, k, v, do, seg_positions(q_seg), seg_positions(k_seg), True, scale_of(D))
    assert_close("O", O[:, 100:260], ref["o"])
    assert_lse("LSE", LSE[:, 100:260], ref["lse"])
    assert_close("dQ", DQ[:, 100:260], ref["dq"])
    assert_close("dK", DK[:, 40:290], ref["dk"])
    assert_close("dV", DV[:, 40:290], ref["dv"])


def test_empty_keys():
    banner("Sk = 0")
    q = _rand((1, 130, 2, 64), 1)
    k = torch.zeros((1, 0, 2, 64), dtype=torch.bfloat16, device=DEV)
    o = torch.full((1, 130, 2, 64), 5.0, device=DEV)
    lse = torch.zeros((1, 130, 2), device=DEV)
    ea.ea_attn_fwd(q, k, k, o, lse, [0, 130], [0, 0], True)
    dq = torch.full((1, 130, 2, 64), 2.0, device=DEV)
    dl = torch.zeros((1, 130, 2), device=DEV)
    ea.ea_attn_bwd(q, k, k, o, q, lse, dl, dq, k.float(), k.float(), [0, 130], [0, 0], True)
    torch.cuda.synchronize()
    assert float(o.abs().max()) == 0
    assert bool(torch.isneginf(lse).all())
    assert float((dq - 2.0).abs().max()) == 0


def test_accumulation_adds():
    """bwd adds into dq/dk/dv: two identical calls give twice one call."""
    banner("accumulation")
    B, S, H, D = 1, 200, 2, 128
    q, k, v, do = (_rand((B, S, H, D), 90 + i) for i in range(4))
    r1 = _run_dense(q, k, v, do, [0, S], [0, S], True)
    dq, dk, dv = r1["dq"].clone(), r1["dk"].clone(), r1["dv"].clone()
    ea.ea_attn_bwd(q, k, v, r1["o"], do, r1["lse"], r1["delta"], dq, dk, dv, [0, S], [0, S], True,
                   delta_ready=True)
    torch.cuda.synchronize()
    for a, b in ((dq, r1["dq"]), (dk, r1["dk"]), (dv, r1["dv"])):
        assert float((a - 2 * b).abs().max()) <= 1e-5 * max(1.0, float(b.abs().max()))


def test_merge_against_oracle():
    banner("lse merge")
    B, S, H, D = 2, 300, 3, 128
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    oa = torch.randn((B, S, H, D), generator=g, device=DEV)
    op = torch.randn((B, S, H, D), generator=g, device=DEV)
    la = torch.randn((B, S, H), generator=g, device=DEV) * 3
    lp = torch.randn((B, S, H), generator=g, device=DEV) * 3
    la[0, :50] = float("-inf")
    oa[0, :50] = 0
    lp[0, 25:75] = float("-inf")
    op[0, 25:75] = 0
    ref_o, ref_l = oracle.lse_merge(oa.cpu(), la.cpu(), op.cpu(), lp.cpu())
    ea.ea_lse_merge(oa, la, op, lp)
    torch.cuda.synchronize()
    assert_close("O", oa, ref_o, max_abs=1e-5, rel_l2=1e-6)
    assert_lse("LSE", la, ref_l, tol=1e-5)
    # bf16 partial
    oa2 = torch.randn((1, 64, 2, 64), generator=g, device=DEV)
    la2 = torch.randn((1, 64, 2), generator=g, device=DEV)
    op2 = torch.randn((1, 64, 2, 64), generator=g, device=DEV).to(torch.bfloat16)
    lp2 = torch.randn((1, 64, 2), generator=g, device=DEV)
    ref_o2, ref_l2 = oracle.lse_merge(oa2.cpu(), la2.cpu(), op2.cpu(), lp2.cpu())
    ea.ea_lse_merge(oa2, la2, op2, lp2)
    torch.cuda.synchronize()
    assert_close("O(bf16 part)", oa2, ref_o2, max_abs=1e-5, rel_l2=1e-6)
    assert_lse("LSE(bf16 part)", la2, ref_l2, tol=1e-5)


MERGE_CASES = [
    # D, B, q_seg, first key segment, merged key segment, causal
    (128, 1, [0, 300], [0, 150], [150, 150], True),     # rows < 150 see nothing in the merged call
    (128, 1, [0, 300], [150, 150], [0, 150], True),     # rows < 150 start from an empty accumulator
    (64, 2, [0, 200], [0, 90, 500, 40], [90, 110], False),
    (128, 1, [0, 130], [200, 77], [300, 64], True),      # no key for any row in either call
    (128, 1, [40, 257], [0, 100], [100, 0], True),       # empty merged call
    (128, 1, [2 ** 31 - 300, 300], [2 ** 31 - 700, 400], [2 ** 31 - 300, 300], True),
]


@pytest.mark.parametrize("case", MERGE_CASES, ids=[f"case{i}" for i in range(len(MERGE_CASES))])
def test_fwd_merge(case):
    """ea_attn_fwd_merge against ea_attn_fwd into a partial followed by ea_lse_merge (the same arithmetic, so
    to within a few fp32 roundings), and both key sets together against the oracle's attention over their union."""
    D, B, q_seg, ka_seg, kb_seg, causal = case
    H = 2
    sq, ska, skb = sum(q_seg[1::2]), sum(ka_seg[1::2]), sum(kb_seg[1::2])
    banner(f"fwd_merge D={D} B={B} q_seg={q_seg} first={ka_seg} merged={kb_seg} causal={causal}")
    q = _rand((B, sq, H, D), 810)
    ka, va = _rand((B, ska, H, D), 811), _rand((B, ska, H, D), 812)
    kb, vb = _rand((B, skb, H, D), 813), _rand((B, skb, H, D), 814)
    of, lf = torch.empty((B, sq, H, D), device=DEV), torch.empty((B, sq, H), device=DEV)
    ea.ea_attn_fwd(q, ka, va, of, lf, q_seg, ka_seg, causal)
    first_o, first_l = of.clone(), lf.clone()
    ea.ea_attn_fwd_merge(q, kb, vb, of, lf, q_seg, kb_seg, causal)
    osep, lsep = first_o.clone(), first_l.clone()
    op, lp = torch.empty_like(osep), torch.empty_like(lsep)
    ea.ea_attn_fwd(q, kb, vb, op, lp, q_seg, kb_seg, causal)
    ea.ea_lse_merge(osep, lsep, op, lp)
    torch.cuda.synchronize()
    assert torch.equal(torch.isneginf(lf), torch.isneginf(lsep))
    fin = ~torch.isneginf(lsep)
    if bool(fin.any()):
        assert float((lf[fin] - lsep[fin]).abs().max()) <= 1e-6
    assert float((of - osep).abs().max()) <= 1e-6
    if skb == 0:  # an empty merged call leaves the accumulator as it was
        assert torch.equal(of, first_o) and torch.equal(lf, first_l)
    k_all, v_all = torch.cat([ka, kb], dim=1), torch.cat([va, vb], dim=1)
    pk = np.concatenate([seg_positions(ka_seg), seg_positions(kb_seg)])
    ref_o, ref_l = oracle.attn_fwd_heads(q, k_all, v_all, seg_positions(q_seg), pk, causal, scale_of(D))
    assert_close("O", of, ref_o)
    assert_lse("LSE", lf, ref_l)


def test_ring_fused_and_separate_merge_agree():
    W, C, H, D, rank = 4, 70, 2, 128, 1
    banner(f"zigzag ring fused vs separate merge W={W} C={C} rank={rank}")
    t = {n: _rand((1, s, H, D), 830 + i) for i, (n, s) in
         enumerate((("q", 2 * C), ("k", 2 * W * C), ("v", 2 * W * C), ("do", 2 * C)))}
    fused = ea.ZigzagRingRank(t["q"], t["k"], t["v"], W, rank)
    sep = ea.ZigzagRingRank(t["q"], t["k"], t["v"], W, rank, fused_merge=False)
    fused.step(t["do"])
    sep.step(t["do"])
    torch.cuda.synchronize()
    for n in ("o", "lse", "dq", "dk", "dv"):
        a, b = getattr(fused, n), getattr(sep, n)
        assert float((a - b).abs().max()) <= 1e-5 * max(1.0, float(b.abs().max())), n


@pytest.mark.parametrize("rank", [0, 3, 7])
@pytest.mark.parametrize("C,D", [(100, 128), (64, 64), (37, 128)])
def test_zigzag_ring_small(rank, C, D):
    W, H = 8, 2
    banner(f"zigzag ring W={W} C={C} rank={rank} D={D}")
    cfg = synth.get("c3")
    t = synth.make_ring_case(cfg, DEV, C=C, H=H, rank=rank) if D == 128 else None
    if t is None:
        t = {n: _rand((1, s, H, D), 300 + i) for i, (n, s) in
             enumerate((("q", 2 * C), ("k", 2 * W * C), ("v", 2 * W * C), ("do", 2 * C)))}
    drv = ea.ZigzagRingRank(t["q"], t["k"], t["v"], W, rank)
    drv.step(t["do"])
    torch.cuda.synchronize()
    S = 2 * W * C
    pq = oracle.zigzag_positions(S, W, rank)
    # K/V rows are the W ranks' shares side by side
    pk = np.concatenate([oracle.zigzag_positions(S, W, s) for s in range(W)])
    ref = oracle.attn_bwd_heads(t["q"], t["k"], t["v"], t["do"], pq, pk, True, scale_of(D))
    assert_close("O", drv.o, ref["o"])
    assert_lse("LSE", drv.lse, ref["lse"])
    assert_close("dQ", drv.dq, ref["dq"])
    assert_close("dK", drv.dk, ref["dk"])
    assert_close("dV", drv.dv, ref["dv"])


def test_bitwise_reproducible():
    """No atomics anywhere: two runs of the same call give identical bits (O, LSE, dQ, dK, dV)."""
    banner("bitwise reproducibility, D=128 S=700 causal")
    q, k, v, do = (_rand((1, 700, 4, 128), 90 + i) for i in range(4))
    a = _run_dense(q, k, v, do, [0, 700], [0, 700], True)
    b = _run_dense(q, k, v, do, [0, 700], [0, 700], True)
    for name in ("o", "lse", "dq", "dk", "dv", "delta"):
        assert torch.equal(a[name], b[name]), name


@pytest.mark.parametrize("W,C,theta", [(4, 48, None), (3, 37, 1e6)])
def test_zigzag_ring_all_ranks_reassemble(W, C, theta):
    """Every rank of a W-rank zigzag ring, run one after another on this GPU, reassembled into the whole
    sequence: O, LSE, dQ (scattered back) and dK, dV (summed over the ranks) against the dense causal driver
    on the whole sequence and against the oracle."""
    H, D = 2, 128
    S = 2 * W * C
    banner(f"zigzag ring all ranks W={W} C={C} theta={theta}")
    q, k, v, do = (_rand((1, S, H, D), 400 + i) for i in range(4))
    kk = torch.cat([ea.zigzag_shard(k, W, s) for s in range(W)], dim=1)
    vv = torch.cat([ea.zigzag_shard(v, W, s) for s in range(W)], dim=1)
    outs = {"o": [], "lse": [], "dq": []}
    dk_sum = torch.zeros((1, S, H, D), device=DEV)
    dv_sum = torch.zeros_like(dk_sum)
    for r in range(W):
        drv = ea.ZigzagRingRank(ea.zigzag_shard(q, W, r), kk, vv, W, r, rope_theta=theta)
        drv.step(ea.zigzag_shard(do, W, r))
        outs["o"].append(drv.o.clone())
        outs["lse"].append(drv.lse.clone())
        outs["dq"].append(drv.dq.clone())
        dk_sum += drv.dk
        dv_sum += drv.dv
    torch.cuda.synchronize()
    got = {n: ea.zigzag_unshard(x, W) for n, x in outs.items()}
    shares = lambda t: [t[:, 2 * C * s: 2 * C * (s + 1)] for s in range(W)]  # noqa: E731
    got["dk"] = ea.zigzag_unshard(shares(dk_sum), W)
    got["dv"] = ea.zigzag_unshard(shares(dv_sum), W)
    dense = ea.DenseCausal(q, k, v, causal=True, rope_theta=theta)
    dense.step(do)
    torch.cuda.synchronize()
    pos = np.arange(S)
    if theta is None:
        ref = oracle.attn_bwd_heads(q, k, v, do, pos, pos, True, scale_of(D))
    else:
        ref = oracle.attn_bwd_rope_heads(q, k, v, do, pos, pos, True, scale_of(D), theta)
    for n in ("o", "dq", "dk", "dv"):
        assert_close(f"{n} (ring) vs oracle", got[n], ref[n])
        # and the two paths of the library agree with each other within the same bars
        assert_close(f"{n} (ring) vs dense", got[n], getattr(dense, n))
    assert_lse("LSE (ring)", got["lse"], ref["lse"])


def test_work_mapping_covers_every_item():
    """Five heads of 16484 tokens: the work lists (65 query blocks, 129 key blocks per head) do not split into
    whole heads per XCD, so the launches deal them out in rounds with a ragged last round.  Each head's results
    must be bit-identical to a launch over that head alone, whose list is dealt in contiguous slices: every work
    item is computed exactly once under both mappings."""
    B, S, H, D = 1, 16484, 5, 128
    banner(f"work mapping S={S} H={H}")
    q, k, v, do = (_rand((B, S, H, D), 700 + i) for i in range(4))
    whole = ea.DenseCausal(q, k, v, causal=True)
    whole.step(do)
    torch.cuda.synchronize()
    for h in range(H):
        one = ea.DenseCausal(*(x[:, :, h:h + 1].contiguous() for x in (q, k, v)), causal=True)
        one.step(do[:, :, h:h + 1].contiguous())
        torch.cuda.synchronize()
        for n in ("o", "lse", "dq", "dk", "dv"):
            a, b = getattr(whole, n), getattr(one, n)
            assert torch.equal(a[:, :, h:h + 1], b), (h, n)


def test_ulysses_ranks_match_the_whole_layer():
    """Every rank of a 4-way Ulysses split (H / 4 heads over all tokens each), run on this GPU and gathered
    over heads: bit-identical to the dense driver over all heads (each head's arithmetic does not depend on the
    others), and within the bars of the oracle."""
    W, S, H, D = 4, 300, 8, 128
    banner(f"ulysses W={W} S={S} H={H}")
    q, k, v, do = (_rand((1, S, H, D), 500 + i) for i in range(4))
    outs = {n: [] for n in ("o", "lse", "dq", "dk", "dv")}
    for r in range(W):
        drv = ea.DenseCausal(*(ea.ulysses_shard(x, W, r) for x in (q, k, v)), causal=True)
        drv.step(ea.ulysses_shard(do, W, r))
        for n in outs:
            outs[n].append(getattr(drv, n).clone())
    whole = ea.DenseCausal(q, k, v, causal=True)
    whole.step(do)
    torch.cuda.synchronize()
    for n, parts in outs.items():
        assert torch.equal(ea.ulysses_unshard(parts), getattr(whole, n)), n
    pos = np.arange(S)
    ref = oracle.attn_bwd_heads(q, k, v, do, pos, pos, True, scale_of(D))
    for n in ("o", "dq", "dk", "dv"):
        assert_close(n, ea.ulysses_unshard(outs[n]), ref[n])
