"""GPU parity of the backward that keeps dS in a workspace panel (ea_attn_bwd_ws).

The same cases as the recompute path: both masks, two position segments, ragged
tails, batch strides, rows without keys, positions at the top of the range;
plus sizes spanning several 256-query panel blocks, head groups forced by a
small workspace, guard bands around the workspace, the zigzag ring of one rank,
and agreement with the recompute path (dK and dV are formed by the same
key-major pass and must be identical bit for bit).
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea
import synth
from tests.parity import assert_close, assert_lse, banner, scale_of, seg_positions
from tests.test_gpu_parity import CASES, _check_dense, _guards_intact, _rand, _sentinel

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _workspace(nbytes, pad=4096):
    """Workspace of nbytes (at least 16) with NaN guard bands (fp32 words) before and after."""
    n = max(16, nbytes) // 4 + 1
    buf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.float32, device=DEV)
    return buf, buf[pad:pad + n], pad


def _run(q, k, v, do, q_seg, k_seg, causal, o_dtype=torch.float32, heads_per_group=None, scale=None):
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
    per_head = ea.ea_attn_bwd_ws_bytes(sq, sk, q_seg, k_seg, causal)
    n = B * H if heads_per_group is None else heads_per_group
    wb, ws, pw = _workspace(per_head * n)
    ea.ea_attn_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, q_seg, k_seg, causal, scale, workspace=ws)
    torch.cuda.synchronize()
    for buf, pad in ((ob, po), (lb, pl), (dqb, p1), (dkb, p2), (dvb, p3), (dlb, p4), (wb, pw)):
        assert _guards_intact(buf, pad), "write outside an output buffer or the workspace"
    return dict(o=o, lse=lse, dq=dq, dk=dk, dv=dv, delta=delta)


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_panel_dense_cases(case):
    D, B, sq, sk, causal, q_seg, k_seg, o_dtype = case
    banner(f"panel D={D} B={B} Sq={sq} Sk={sk} causal={causal} q_seg={q_seg} k_seg={k_seg} o={o_dtype}")
    H = 3
    q, k, v, do = (_rand((B, s, H, D), 50 + i) for i, s in enumerate((sq, sk, sk, sq)))
    res = _run(q, k, v, do, q_seg, k_seg, causal, o_dtype)
    _check_dense(res, q, k, v, do, q_seg, k_seg, causal)


BLOCK_CASES = [
    # D, B, Sq, Sk, causal, q_seg, k_seg: several 256-query blocks, ragged tails, segment boundaries inside
    # blocks and key groups
    (128, 1, 1000, 1000, True, [0, 1000], [0, 1000]),
    (128, 1, 777, 1301, True, [300, 400, 2000, 377], [0, 650, 1800, 651]),
    (64, 2, 600, 900, True, [250, 600], [0, 900]),
    (128, 1, 530, 610, False, [0, 530], [0, 610]),
    (128, 1, 700, 700, True, [0, 350, 1050, 350], [350, 350, 700, 350]),  # zigzag-like halves
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[f"blocks{i}" for i in range(len(BLOCK_CASES))])
def test_panel_several_blocks(case):
    D, B, sq, sk, causal, q_seg, k_seg = case
    banner(f"panel blocks D={D} B={B} Sq={sq} Sk={sk} causal={causal} q_seg={q_seg} k_seg={k_seg}")
    H = 2
    q, k, v, do = (_rand((B, s, H, D), 150 + i) for i, s in enumerate((sq, sk, sk, sq)))
    res = _run(q, k, v, do, q_seg, k_seg, causal)
    _check_dense(res, q, k, v, do, q_seg, k_seg, causal)


@pytest.mark.parametrize("per_group", [1, 2, 5])
def test_panel_head_groups(per_group):
    """A workspace for fewer (batch, head) slices than B*H: heads run in groups, batch by batch."""
    D, B, H, sq, sk = 128, 2, 3, 520, 700
    q_seg, k_seg = [180, sq], [0, sk]
    banner(f"panel head groups of {per_group}, B={B} H={H}")
    q, k, v, do = (_rand((B, s, H, D), 250 + i) for i, s in enumerate((sq, sk, sk, sq)))
    res = _run(q, k, v, do, q_seg, k_seg, True, heads_per_group=per_group)
    _check_dense(res, q, k, v, do, q_seg, k_seg, True)


def test_panel_matches_recompute_path():
    """dK and dV come from the same key-major pass in both paths (identical bits); dQ agrees closely."""
    D, H, S = 128, 4, 1100
    banner(f"panel vs recompute S={S} H={H}")
    q, k, v, do = (_rand((1, S, H, D), 350 + i) for i in range(4))
    seg = [0, S]
    a = _run(q, k, v, do, seg, seg, True)
    b = {n: torch.zeros_like(a[n]) for n in ("dq", "dk", "dv", "delta")}
    ea.ea_attn_bwd(q, k, v, a["o"], do, a["lse"], b["delta"], b["dq"], b["dk"], b["dv"], seg, seg, True)
    torch.cuda.synchronize()
    assert torch.equal(a["dk"], b["dk"]) and torch.equal(a["dv"], b["dv"])
    assert torch.equal(a["delta"], b["delta"])
    assert_close("dQ panel vs recompute", a["dq"], b["dq"], max_abs=2e-3, rel_l2=1e-3)


def test_panel_too_small_workspace_is_rejected():
    D, H, S = 128, 1, 300
    q, k, v, do = (_rand((1, S, H, D), 370 + i) for i in range(4))
    o = torch.zeros((1, S, H, D), device=DEV)
    lse = torch.zeros((1, S, H), device=DEV)
    dq, dk, dv = (torch.zeros((1, S, H, D), device=DEV) for _ in range(3))
    delta = torch.zeros_like(lse)
    per_head = ea.ea_attn_bwd_ws_bytes(S, S, [0, S], [0, S], True)
    ws = torch.empty(per_head - 16, dtype=torch.uint8, device=DEV)
    with pytest.raises(ea.EaError) as ei:
        ea.ea_attn_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, [0, S], [0, S], True, workspace=ws)
    assert ei.value.status == 8


@pytest.mark.parametrize("rank", [0, 3, 7])
def test_panel_zigzag_ring_small(rank):
    W, H, C, D = 8, 2, 100, 128
    banner(f"panel zigzag ring W={W} C={C} rank={rank}")
    t = synth.make_ring_case(synth.get("c3"), DEV, C=C, H=H, rank=rank)
    drv = ea.ZigzagRingRank(t["q"], t["k"], t["v"], W, rank, panel_bytes=1 << 40)
    assert drv.panel is not None
    drv.step(t["do"])
    torch.cuda.synchronize()
    S = 2 * W * C
    pq = oracle.zigzag_positions(S, W, rank)
    pk = np.concatenate([oracle.zigzag_positions(S, W, s) for s in range(W)])
    ref = oracle.attn_bwd_heads(t["q"], t["k"], t["v"], t["do"], pq, pk, True, scale_of(D))
    assert_close("O", drv.o, ref["o"])
    assert_lse("LSE", drv.lse, ref["lse"])
    assert_close("dQ", drv.dq, ref["dq"])
    assert_close("dK", drv.dk, ref["dk"])
    assert_close("dV", drv.dv, ref["dv"])


def test_panel_dense_driver_with_rope():
    cfg = synth.get("c1")
    banner("panel dense driver, rotary base 1e6")
    S, H = 700, 2
    t = synth.make_dense_case(cfg, DEV, S=S, H=H)
    drv = ea.DenseCausal(t["q"], t["k"], t["v"], causal=True, rope_theta=1e6, panel_bytes=1 << 40)
    drv.step(t["do"])
    torch.cuda.synchronize()
    pos = np.arange(S)
    ref = oracle.attn_bwd_rope_heads(t["q"], t["k"], t["v"], t["do"], pos, pos, True, scale_of(cfg.D), 1e6)
    assert_close("O", drv.o, ref["o"])
    assert_close("dQ", drv.dq, ref["dq"])
    assert_close("dK", drv.dk, ref["dk"])
    assert_close("dV", drv.dv, ref["dv"])


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_panel_fullsize_t():
    """The 64K-token workload on the panel path (the whole panel in one workspace): sampled rows and tail keys
    against the oracle, and the any-size properties."""
    from tests.test_gpu_fullsize import _check_properties, _check_rows, _check_tail_keys, _sampled_rows
    cfg = synth.get("t")
    banner(f"panel {cfg.name}")
    t = synth.make_dense_case(cfg, DEV)
    drv = ea.DenseCausal(t["q"], t["k"], t["v"], causal=True, scale=cfg.scale, rope_theta=cfg.rope_theta,
                         panel_bytes=160 << 30)
    assert drv.panel is not None
    drv.step(t["do"])
    torch.cuda.synchronize()
    pos = np.arange(cfg.S)
    rng = np.random.default_rng(cfg.seed + 1)
    for h in (0, cfg.H - 1):
        _check_rows(cfg.name, t, drv, h, _sampled_rows(cfg.S, rng), pos, pos, cfg.scale, cfg.rope_theta)
        _check_tail_keys(cfg.name, t, drv, h, pos, pos, cfg.scale, cfg.rope_theta)
    _check_properties(cfg.name, t, drv, pos, pos, cfg.rope_theta)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", ["c3", "c4"])
def test_panel_fullsize_ring_head_groups(key):
    """One rank's share of the 512K-token ring, or of the 700K-token ring (43750-token chunks: ragged tiles and
    panel blocks), with a workspace for 5 of the 32 heads (7 head groups per ring step): sampled rows and tail
    keys against the oracle, and the any-size properties."""
    from tests.test_gpu_fullsize import _check_properties, _check_rows, _check_tail_keys
    cfg = synth.get(key)
    banner(f"panel {cfg.name}, head groups of 5")
    t = synth.make_ring_case(cfg, DEV)
    C = cfg.C
    qs = ea.ea_zigzag_segments(cfg.s_total, cfg.W, cfg.rank)
    per_head = max(ea.ea_attn_bwd_ws_bytes(2 * C, 2 * C, qs, ea.ea_zigzag_segments(cfg.s_total, cfg.W, s), True)
                   for s in range(cfg.W))
    drv = ea.ZigzagRingRank(t["q"], t["k"], t["v"], cfg.W, cfg.rank, scale=cfg.scale, panel_bytes=5 * per_head)
    assert drv.panel.numel() == 5 * per_head
    drv.step(t["do"])
    torch.cuda.synchronize()
    pos_q = oracle.zigzag_positions(cfg.s_total, cfg.W, cfg.rank)
    pos_k = np.concatenate([oracle.zigzag_positions(cfg.s_total, cfg.W, s) for s in range(cfg.W)])
    rng = np.random.default_rng(cfg.seed + 1)
    rows = np.array(sorted({0, 1, C - 1, C, C + 1, 2 * C - 1} | set(rng.integers(0, 2 * C, size=24).tolist())))
    for h in (0, 4, 5, cfg.H - 1):  # first and last head of a group, first head of the next, last head
        _check_rows(cfg.name, t, drv, h, rows, pos_q, pos_k, cfg.scale)
        _check_tail_keys(cfg.name, t, drv, h, pos_q, pos_k, cfg.scale)
    _check_properties(cfg.name, t, drv, pos_q, pos_k)
