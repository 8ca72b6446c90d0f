"""GPU parity at the full workload sizes, in the launch configuration the bench times.

The whole workload (all heads, full sequence) runs on the GPU exactly as in
bench.py, with the rotary embedding fused into the attention calls for the
workloads with a rotary base.  The fp64 oracle then checks, per workload:
  * every output element of whole heads (O, LSE, dQ of every query row; dK, dV
    of every key, including keys whose gradients sum over tens of thousands of
    queries): the 32K-token layer (heads 0, 31 and a seeded head), the
    64K-token layer (heads 0 and 31), the 128K-token layer (head 0) and the
    512K-token ring rank (head 0, over all 524288 keys);
  * where a whole head would take the host too long (the 700K-token ring rank,
    the 4-head 512K-token layer: 6 and 12 minutes of fp64 per head), sampled
    query rows (O, LSE, dQ; each row's oracle cost is one pass over its keys)
    and the visible keys with the largest positions (dK, dV from every query
    that sees them);
  * properties that hold at any size: keys nobody may see get dK = dV = 0
    exactly; sum_j dK_j = 0; sum_j dV_j = sum of dO over rows with keys.
Bars: max-abs <= 1e-2 and relative L2 <= 5e-3 on O, dQ, dK, dV (fp32 outputs);
LSE within 1e-3.  The oracle runs with 2^26-score row blocks here (the
result does not depend on the block size; larger blocks keep its BLAS calls
efficient on 524288 keys).
"""
import time

import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea
import synth
from tests.parity import assert_close, assert_lse, banner, to_np

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda"


@pytest.fixture(autouse=True)
def _big_oracle_blocks(monkeypatch):
    monkeypatch.setattr(oracle.attention, "ROW_BLOCK_ELEMS", 1 << 26)


def _head_np(x, h):
    return x[0, :, h].double().cpu().numpy()


def _run_dense(cfg):
    t = synth.make_dense_case(cfg, DEV)
    drv = ea.DenseCausal(t["q"], t["k"], t["v"], causal=True, scale=cfg.scale, rope_theta=cfg.rope_theta)
    drv.step(t["do"])
    torch.cuda.synchronize()
    return t, drv


def _sampled_rows(S, rng, n=24):
    """Tile-boundary rows, the first and last rows, and random rows."""
    picks = {0, 1, 31, 32, 63, 64, 127, 128, S // 2, S - 129, S - 128, S - 2, S - 1}
    picks |= set(rng.integers(0, S, size=n).tolist())
    return np.array(sorted(p for p in picks if 0 <= p < S))


def _ref(q, k, v, do, pos_q, pos_k, scale, theta):
    if theta is None:
        return oracle.attn_bwd(q, k, v, do, pos_q, pos_k, True, scale)
    return oracle.attn_bwd_rope(q, k, v, do, pos_q, pos_k, True, scale, theta)


def _check_rows(name, t, drv, h, rows, pos_q, pos_k, scale, theta=None):
    q, k, v, do = (_head_np(t[n], h) for n in ("q", "k", "v", "do"))
    ref = _ref(q[rows], k, v, do[rows], pos_q[rows], pos_k, scale, theta)
    assert_close(f"{name} h{h} O(rows)", _head_np(drv.o, h)[rows], ref["o"])
    assert_lse(f"{name} h{h} LSE(rows)", _head_np(drv.lse, h)[rows], ref["lse"])
    assert_close(f"{name} h{h} dQ(rows)", _head_np(drv.dq, h)[rows], ref["dq"])


def _check_keys(name, t, drv, h, keys, pos_q, pos_k, scale, theta=None):
    """dK, dV of the given keys, from every query that may see any of them (one oracle call)."""
    kmin = pos_k[keys].min()
    qrows = np.nonzero(pos_q >= kmin)[0]
    q, k, v, do = (_head_np(t[n], h) for n in ("q", "k", "v", "do"))
    ref = _ref(q[qrows], k, v, do[qrows], pos_q[qrows], pos_k, scale, theta)
    assert_close(f"{name} h{h} dK({len(keys)} keys from {kmin}, {len(qrows)} queries)", _head_np(drv.dk, h)[keys],
                 ref["dk"][keys])
    assert_close(f"{name} h{h} dV({len(keys)} keys from {kmin})", _head_np(drv.dv, h)[keys], ref["dv"][keys])


def _check_tail_keys(name, t, drv, h, pos_q, pos_k, scale, theta=None, n_keys=256):
    """The visible keys with the largest positions: few queries see them."""
    visible = np.nonzero(pos_k <= pos_q.max())[0]
    keys = np.sort(visible[np.argsort(pos_k[visible])[-n_keys:]])
    _check_keys(name, t, drv, h, keys, pos_q, pos_k, scale, theta)


def _ref_chunked(name, q, k, v, do, pos_q, pos_k, scale, theta, rows=8192):
    """The oracle over query-row chunks (rows are independent; key gradients add up over the chunks), printing
    its progress so that a long host computation is visibly alive."""
    out = None
    t0 = time.perf_counter()
    for i0 in range(0, q.shape[0], rows):
        sel = slice(i0, min(q.shape[0], i0 + rows))
        r = _ref(q[sel], k, v, do[sel], pos_q[sel], pos_k, scale, theta)
        if out is None:
            out = {n: np.zeros((q.shape[0],) + r[n].shape[1:]) for n in ("o", "lse", "dq")}
            out["dk"], out["dv"] = r["dk"], r["dv"]
        else:
            out["dk"] += r["dk"]
            out["dv"] += r["dv"]
        for n in ("o", "lse", "dq"):
            out[n][sel] = r[n]
        print(f"  {name}: oracle rows {sel.stop}/{q.shape[0]} ({time.perf_counter() - t0:.0f} s)", flush=True)
    return out


def _check_whole_heads(name, t, drv, heads, pos_q, pos_k, scale, theta=None):
    """Every row and every key of the given heads against the oracle."""
    for h in heads:
        q, k, v, do = (_head_np(t[n], h) for n in ("q", "k", "v", "do"))
        ref = _ref_chunked(f"{name} h{h}", q, k, v, do, pos_q, pos_k, scale, theta)
        assert_close(f"{name} h{h} O", _head_np(drv.o, h), ref["o"])
        assert_lse(f"{name} h{h} LSE", _head_np(drv.lse, h), ref["lse"])
        assert_close(f"{name} h{h} dQ", _head_np(drv.dq, h), ref["dq"])
        assert_close(f"{name} h{h} dK", _head_np(drv.dk, h), ref["dk"])
        assert_close(f"{name} h{h} dV", _head_np(drv.dv, h), ref["dv"])


def _rotated_key_sums(dk, pos_k, theta, chunk=8192):
    """sum_j R(pos_j) dK_j and sum_j |R(pos_j) dK_j| in fp64 (the gradient w.r.t. the rotated keys)."""
    S, H, D = dk.shape
    half = D // 2
    f = torch.pow(torch.tensor(float(theta), dtype=torch.float64), -2.0 * torch.arange(half, dtype=torch.float64) / D)
    f = f.to(DEV)
    pk = torch.from_numpy(np.asarray(pos_k, dtype=np.int64)).to(DEV)
    s = torch.zeros((H, D), dtype=torch.float64, device=DEV)
    a = torch.zeros((H, D), dtype=torch.float64, device=DEV)
    for j0 in range(0, S, chunk):
        x = dk[j0:j0 + chunk].double()
        ang = pk[j0:j0 + chunk, None].double() * f[None, :]
        c, sn = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
        r = torch.cat([x[..., :half] * c - x[..., half:] * sn, x[..., half:] * c + x[..., :half] * sn], dim=-1)
        s += r.sum(dim=0)
        a += r.abs().sum(dim=0)
    return s, a


def _check_properties(name, t, drv, pos_q, pos_k, theta=None):
    # keys that no query may see
    dead = pos_k > pos_q.max()
    if dead.any():
        idx = torch.from_numpy(np.nonzero(dead)[0]).to(DEV)
        assert float(drv.dk[0, idx].abs().max()) == 0.0 and float(drv.dv[0, idx].abs().max()) == 0.0
    # sum over keys of dK vanishes (of the gradient w.r.t. the rotated keys, with a rotary base); sum over keys
    # of dV equals the sum of dO (every row has keys here)
    f64 = torch.float64
    if theta is None:
        sk = drv.dk[0].sum(dim=0, dtype=f64)                      # [H, D]
        ak = drv.dk[0].abs().sum(dim=0, dtype=f64).clamp_min(1e-30)
    else:
        sk, ak = _rotated_key_sums(drv.dk[0], pos_k, theta)
        ak = ak.clamp_min(1e-30)
    sv = drv.dv[0].sum(dim=0, dtype=f64)
    sd = t["do"][0].sum(dim=0, dtype=f64)
    ratio = float((sk.abs() / ak).max())
    print(f"  {name}: max |sum_j dK_j| / sum_j |dK_j| = {ratio:.2e}", flush=True)
    assert ratio < 1e-2, f"{name}: sum_j dK_j far from 0"
    rel = float((sv - sd).norm() / sd.norm())
    print(f"  {name}: |sum dV - sum dO| / |sum dO| = {rel:.2e}", flush=True)
    assert rel < 5e-3


@pytest.mark.timeout(900)
def test_c2_full_heads():
    cfg = synth.get("c2")
    banner(cfg.name)
    t, drv = _run_dense(cfg)
    pos = np.arange(cfg.S)
    heads = [0, cfg.H - 1, int(np.random.default_rng(cfg.seed).integers(1, cfg.H - 1))]
    if cfg.rope_theta is None:
        ref = oracle.attn_bwd_heads(t["q"], t["k"], t["v"], t["do"], pos, pos, True, cfg.scale, heads=heads)
    else:
        ref = oracle.attn_bwd_rope_heads(t["q"], t["k"], t["v"], t["do"], pos, pos, True, cfg.scale,
                                         cfg.rope_theta, heads=heads)
    got = {n: getattr(drv, n)[:, :, heads] for n in ("o", "lse", "dq", "dk", "dv")}
    assert_close("O", got["o"], ref["o"])
    assert_lse("LSE", got["lse"], ref["lse"])
    assert_close("dQ", got["dq"], ref["dq"])
    assert_close("dK", got["dk"], ref["dk"])
    assert_close("dV", got["dv"], ref["dv"])
    _check_properties(cfg.name, t, drv, pos, pos, cfg.rope_theta)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("key,heads", [("t", (0, 31)), ("c5", (0,))])
def test_dense_whole_heads(key, heads):
    cfg = synth.get(key)
    banner(f"{cfg.name} whole heads {heads}")
    t, drv = _run_dense(cfg)
    pos = np.arange(cfg.S)
    _check_whole_heads(cfg.name, t, drv, heads, pos, pos, cfg.scale, cfg.rope_theta)
    _check_properties(cfg.name, t, drv, pos, pos, cfg.rope_theta)


@pytest.mark.timeout(900)
def test_dense_sampled_u3():
    cfg = synth.get("u3")
    banner(cfg.name)
    t, drv = _run_dense(cfg)
    pos = np.arange(cfg.S)
    rng = np.random.default_rng(cfg.seed)
    for h in (0, cfg.H - 1):
        _check_rows(cfg.name, t, drv, h, _sampled_rows(cfg.S, rng), pos, pos, cfg.scale, cfg.rope_theta)
        _check_tail_keys(cfg.name, t, drv, h, pos, pos, cfg.scale, cfg.rope_theta)
    _check_properties(cfg.name, t, drv, pos, pos, cfg.rope_theta)


def _run_ring(cfg):
    t = synth.make_ring_case(cfg, DEV)
    drv = ea.ZigzagRingRank(t["q"], t["k"], t["v"], cfg.W, cfg.rank, scale=cfg.scale)
    drv.step(t["do"])
    torch.cuda.synchronize()
    S = cfg.s_total
    pos_q = oracle.zigzag_positions(S, cfg.W, cfg.rank)
    pos_k = np.concatenate([oracle.zigzag_positions(S, cfg.W, s) for s in range(cfg.W)])
    return t, drv, pos_q, pos_k


def _ring_rows(cfg, rng):
    C = cfg.C
    return np.array(sorted({0, 1, C - 1, C, C + 1, 2 * C - 1} | set(rng.integers(0, 2 * C, size=24).tolist())))


@pytest.mark.timeout(900)
def test_ring_whole_head_c3():
    """The 512K-token ring rank: head 0 whole (every local query, all 524288 keys), the last head sampled."""
    cfg = synth.get("c3")
    banner(f"{cfg.name} whole head 0")
    t, drv, pos_q, pos_k = _run_ring(cfg)
    _check_whole_heads(cfg.name, t, drv, (0,), pos_q, pos_k, cfg.scale)
    h = cfg.H - 1
    _check_rows(cfg.name, t, drv, h, _ring_rows(cfg, np.random.default_rng(cfg.seed)), pos_q, pos_k, cfg.scale)
    _check_tail_keys(cfg.name, t, drv, h, pos_q, pos_k, cfg.scale)
    _check_properties(cfg.name, t, drv, pos_q, pos_k)


@pytest.mark.timeout(900)
def test_ring_sampled_c4():
    """The 700K-token ring rank (ragged tiles): sampled rows and the tail keys of the first and last head."""
    cfg = synth.get("c4")
    banner(cfg.name)
    t, drv, pos_q, pos_k = _run_ring(cfg)
    rng = np.random.default_rng(cfg.seed)
    for h in (0, cfg.H - 1):
        _check_rows(cfg.name, t, drv, h, _ring_rows(cfg, rng), pos_q, pos_k, cfg.scale)
        _check_tail_keys(cfg.name, t, drv, h, pos_q, pos_k, cfg.scale)
    _check_properties(cfg.name, t, drv, pos_q, pos_k)
