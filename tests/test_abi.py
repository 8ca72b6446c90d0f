"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects bad arguments on the host before any HIP call.

Only invalid argument sets are passed here (with fake, never-dereferenced
pointers), so no kernel is ever launched.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import long_context_causal_ea_amd as ea
from long_context_causal_ea_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ea_attn.h")

OK, NULL, SHAPE, UNSUP, POS, ALIGN, ALIAS, HIP = range(8)
P = 0x10000          # fake 16-byte aligned device addresses, far apart
STEP = 1 << 40


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ea_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ea.lib()
    names = _declared()
    assert set(names) >= {"ea_attn_fwd", "ea_attn_bwd", "ea_lse_merge"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.EXPORTS)
    assert ea.ea_version() >= 100
    assert ea.strerror(OK) == "ok"


def _seg(*xs):
    arr = (ctypes.c_int64 * len(xs))(*xs)
    return arr, len(xs) // 2


def _fwd(**kw):
    a = dict(q=P, k=P + STEP, v=P + 2 * STEP, o=P + 3 * STEP, o_dtype=0, lse=P + 4 * STEP, B=1, H=2, Sq=128,
             Sk=128, D=128, qbr=128, kbr=128, qseg=(0, 128), kseg=(0, 128), mask=1, scale=0.088)
    a.update(kw)
    qs, nq = _seg(*a["qseg"])
    ks, nk = _seg(*a["kseg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_attn_fwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["o_dtype"], vp(a["lse"]),
                                a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["qbr"], a["kbr"], qs, nq, ks, nk,
                                a["mask"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL),
    (dict(B=0), SHAPE), (dict(H=0), SHAPE), (dict(Sq=-1), SHAPE), (dict(Sk=-5), SHAPE),
    (dict(B=2, qbr=100), SHAPE), (dict(kbr=64), SHAPE), (dict(Sq=1 << 31, qbr=1 << 31), SHAPE),
    (dict(D=96), UNSUP), (dict(D=256), UNSUP), (dict(mask=2), UNSUP), (dict(o_dtype=5), UNSUP),
    (dict(scale=0.0), UNSUP), (dict(scale=-1.0), UNSUP), (dict(scale=float("inf")), UNSUP),
    (dict(scale=float("nan")), UNSUP),
    (dict(qseg=(0, 100)), POS), (dict(kseg=(0, 64, 64, 60)), POS), (dict(qseg=(-1, 128)), POS),
    (dict(qseg=(0, 64, 10, 64, 20, 0)), POS), (dict(kseg=((1 << 31) - 10, 128)), POS),
    (dict(kseg=(5, -1, 0, 129)), POS),
    (dict(q=P + 8), ALIGN), (dict(o=P + 3 * STEP + 4), ALIGN), (dict(lse=P + 4 * STEP + 2), ALIGN),
    (dict(k=P + STEP + 8), ALIGN),
    (dict(o=P), ALIAS), (dict(lse=P + STEP + 64), ALIAS), (dict(lse=P + 3 * STEP + 16), ALIAS),
])
def test_fwd_rejects_bad_arguments(kw, code):
    assert _fwd(**kw) == code


def test_fwd_empty_query_is_a_noop_without_pointers():
    assert _fwd(Sq=0, qseg=(0, 0), q=0, o=0, lse=0) == OK


def _fwd_merge(**kw):
    a = dict(q=P, k=P + STEP, v=P + 2 * STEP, o=P + 3 * STEP, lse=P + 4 * STEP, B=1, H=2, Sq=128, Sk=128, D=128,
             qbr=128, kbr=128, qseg=(0, 128), kseg=(0, 128), mask=1, scale=0.088)
    a.update(kw)
    qs, nq = _seg(*a["qseg"])
    ks, nk = _seg(*a["kseg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_attn_fwd_merge(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), vp(a["lse"]), a["B"],
                                      a["H"], a["Sq"], a["Sk"], a["D"], a["qbr"], a["kbr"], qs, nq, ks, nk,
                                      a["mask"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL), (dict(k=0), NULL),
    (dict(B=0), SHAPE), (dict(B=2, qbr=100), SHAPE), (dict(D=96), UNSUP), (dict(mask=3), UNSUP),
    (dict(scale=0.0), UNSUP), (dict(qseg=(0, 100)), POS), (dict(kseg=((1 << 31) - 10, 128)), POS),
    (dict(o=P + 3 * STEP + 4), ALIGN), (dict(lse=P + 4 * STEP + 2), ALIGN),
    (dict(o=P), ALIAS), (dict(lse=P + 2 * STEP + 64), ALIAS), (dict(lse=P + 3 * STEP + 16), ALIAS),
])
def test_fwd_merge_rejects_bad_arguments(kw, code):
    assert _fwd_merge(**kw) == code


def test_fwd_merge_empty_query_is_a_noop_without_pointers():
    assert _fwd_merge(Sq=0, qseg=(0, 0), q=0, o=0, lse=0) == OK


def _bwd(**kw):
    a = dict(q=P, k=P + STEP, v=P + 2 * STEP, o=P + 3 * STEP, o_dtype=0, do=P + 4 * STEP, lse=P + 5 * STEP,
             delta=P + 6 * STEP, ready=0, dq=P + 7 * STEP, dk=P + 8 * STEP, dv=P + 9 * STEP, B=1, H=2, Sq=128,
             Sk=256, D=64, qbr=128, kbr=256, qseg=(0, 128), kseg=(0, 256), mask=1, scale=0.125)
    a.update(kw)
    qs, nq = _seg(*a["qseg"])
    ks, nk = _seg(*a["kseg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_attn_bwd(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["o_dtype"], vp(a["do"]),
                                vp(a["lse"]), vp(a["delta"]), a["ready"], vp(a["dq"]), vp(a["dk"]), vp(a["dv"]),
                                a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["qbr"], a["kbr"], qs, nq, ks, nk,
                                a["mask"], a["scale"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(do=0), NULL), (dict(lse=0), NULL), (dict(delta=0), NULL), (dict(dq=0), NULL),
    (dict(dk=0), NULL), (dict(dv=0), NULL), (dict(o=0), NULL),
    (dict(D=32), UNSUP), (dict(o_dtype=2), UNSUP), (dict(mask=-1), UNSUP),
    (dict(H=-2), SHAPE), (dict(kseg=(0, 255)), POS), (dict(qseg=(0, 100, 50, 29)), POS),
    (dict(dq=P + 7 * STEP + 4), ALIGN), (dict(do=P + 4 * STEP + 2), ALIGN),
    (dict(dq=P), ALIAS), (dict(dk=P + STEP), ALIAS), (dict(dv=P + 8 * STEP), ALIAS),
    (dict(delta=P + 7 * STEP), ALIAS), (dict(dk=P + 5 * STEP), ALIAS),
])
def test_bwd_rejects_bad_arguments(kw, code):
    assert _bwd(**kw) == code


def test_bwd_o_optional_when_delta_ready_but_other_checks_still_apply():
    # o may be NULL when Delta is supplied; the call still fails on the bad scale first
    assert _bwd(o=0, ready=1, scale=0.0) == UNSUP


def _merge(**kw):
    a = dict(oa=P, la=P + STEP, op=P + 2 * STEP, dt=0, lp=P + 3 * STEP, B=1, H=4, Sq=100, D=128, qbr=100)
    a.update(kw)
    vp = ctypes.c_void_p
    return ea.lib().ea_lse_merge(vp(a["oa"]), vp(a["la"]), vp(a["op"]), a["dt"], vp(a["lp"]), a["B"], a["H"],
                                 a["Sq"], a["D"], a["qbr"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(oa=0), NULL), (dict(lp=0), NULL), (dict(D=100), UNSUP), (dict(dt=3), UNSUP), (dict(B=0), SHAPE),
    (dict(qbr=50, B=2), SHAPE), (dict(oa=P + 4), ALIGN), (dict(op=P), ALIAS), (dict(lp=P + STEP), ALIAS),
])
def test_merge_rejects_bad_arguments(kw, code):
    assert _merge(**kw) == code


def test_merge_empty_is_noop():
    assert _merge(Sq=0, qbr=0, oa=0, la=0, op=0, lp=0) == OK


def _xent(**kw):
    a = dict(x=P, dt=1, y=P + STEP, loss=P + 2 * STEP, lse=P + 3 * STEP, rows=4, V=32000, rs=32000, ign=-100,
             g=0.25)
    a.update(kw)
    vp = ctypes.c_void_p
    return ea.lib().ea_xent_fwd_bwd(vp(a["x"]), a["dt"], vp(a["y"]), vp(a["loss"]), vp(a["lse"]), a["rows"], a["V"],
                                    a["rs"], a["ign"], a["g"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), NULL), (dict(y=0), NULL), (dict(loss=0), NULL), (dict(lse=0), NULL),
    (dict(rows=-1), SHAPE), (dict(V=0), SHAPE), (dict(rs=31999), SHAPE), (dict(rows=1 << 31), SHAPE),
    (dict(dt=2), UNSUP), (dict(g=float("inf")), UNSUP), (dict(g=float("nan")), UNSUP),
    (dict(x=P + 1), ALIGN), (dict(dt=0, x=P + 2), ALIGN), (dict(y=P + STEP + 4), ALIGN),
    (dict(loss=P + 2 * STEP + 2), ALIGN),
    (dict(y=P + 64), ALIAS), (dict(loss=P), ALIAS), (dict(lse=P + 2 * STEP + 8), ALIAS),
    (dict(lse=P + STEP + 16), ALIAS),
])
def test_xent_rejects_bad_arguments(kw, code):
    assert _xent(**kw) == code


def test_xent_empty_is_noop():
    assert _xent(rows=0, x=0, y=0, loss=0, lse=0) == OK


@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("C", [1, 5, 37, 32768, 43750])
def test_zigzag_segments_match_oracle_positions(W, C):
    S = 2 * W * C
    for r in range(W):
        s0, l0, s1, l1 = ea.ea_zigzag_segments(S, W, r)
        pos = np.concatenate([s0 + np.arange(l0), s1 + np.arange(l1)])
        assert np.array_equal(pos, oracle.zigzag_positions(S, W, r))
        assert [ea.ea_ring_source(r, t, W) for t in range(W)] == [oracle.ring_source(r, t, W) for t in range(W)]


def test_zigzag_segments_errors():
    out = (ctypes.c_int64 * 4)()
    f = ea.lib().ea_zigzag_segments
    assert f(10, 3, 0, out) == POS
    assert f(16, 4, 4, out) == POS
    assert f(16, 0, 0, out) == POS
    assert f(0, 1, 0, out) == POS
    assert f(1 << 32, 1, 0, out) == POS
    assert f(16, 4, 1, None) == NULL
    assert ea.lib().ea_ring_source(0, 0, 0) == -1
    assert ea.lib().ea_ring_source(3, 1, 2) == -1


def test_python_binding_rejects_bad_views():
    import torch
    q = torch.zeros(1, 8, 2, 64, dtype=torch.bfloat16)
    o = torch.zeros(1, 8, 2, 64)
    lse = torch.zeros(1, 8, 2)
    with pytest.raises(ValueError):
        ea.ea_attn_fwd(q, q, q, o, lse, [0, 8, 0, 0, 0, 0], [0, 8])
    with pytest.raises(ValueError):
        ea.ea_attn_fwd(q.float(), q, q, o, lse, [0, 8], [0, 8])
    with pytest.raises(ValueError):
        ea.ea_attn_fwd(q.transpose(1, 2), q, q, o, lse, [0, 8], [0, 8])


def _rope(**kw):
    a = dict(x=P, y=P + STEP, dt=1, B=1, H=32, S=1024, D=128, br=1024, seg=(0, 1024), theta=1e6, inv=0)
    a.update(kw)
    seg = (ctypes.c_int64 * len(a["seg"]))(*a["seg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_rope(vp(a["x"]), vp(a["y"]), a["dt"], a["B"], a["H"], a["S"], a["D"], a["br"], seg,
                            len(a["seg"]) // 2, a["theta"], a["inv"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=0), NULL), (dict(y=0), NULL),
    (dict(B=0), SHAPE), (dict(H=0), SHAPE), (dict(S=-1), SHAPE), (dict(br=1000), SHAPE), (dict(S=1 << 31), SHAPE),
    (dict(B=3, S=1 << 30, br=1 << 30, seg=(0, 1 << 30)), SHAPE),
    (dict(D=96), UNSUP), (dict(dt=2), UNSUP), (dict(theta=0.0), UNSUP), (dict(theta=-1.0), UNSUP),
    (dict(theta=float("inf")), UNSUP), (dict(theta=float("nan")), UNSUP), (dict(inv=2), UNSUP),
    (dict(seg=(0, 1000)), POS), (dict(seg=(-1, 1024)), POS), (dict(seg=(0, 512, 0, 256, 0, 256)), POS),
    (dict(seg=((1 << 31) - 10, 1024)), POS),
    (dict(x=P + 8), ALIGN), (dict(y=P + STEP + 4), ALIGN),
    (dict(y=P + 4096), ALIAS), (dict(x=P + STEP + 16 * 1024), ALIAS),
])
def test_rope_rejects_bad_arguments(kw, code):
    assert _rope(**kw) == code


def test_rope_empty_is_noop():
    assert _rope(S=0, br=0, seg=(5, 0), x=0, y=0) == OK


# ---- backward with the dS panel in a caller workspace (ea_attn_bwd_ws, ea_attn_bwd_ws_bytes)
WORKSPACE = 8


def _panel_blocks_brute(pos_q, pos_k, causal):
    """(256-query block, 32-key group) pairs holding at least one allowed pair, counted over positions."""
    n = 0
    for i0 in range(0, len(pos_q), 256):
        qmax = pos_q[i0:i0 + 256].max()
        for j0 in range(0, len(pos_k), 32):
            if not causal or pos_k[j0:j0 + 32].min() <= qmax:
                n += 1
    return n


@pytest.mark.parametrize("sq,sk,q_seg,k_seg,causal", [
    (512, 512, [0, 512], [0, 512], True),
    (1000, 1000, [0, 1000], [0, 1000], True),
    (333, 200, [0, 333], [0, 200], False),
    (777, 1301, [300, 400, 2000, 377], [0, 650, 1800, 651], True),
    (190, 190, [0, 190], [100, 190], True),
    (300, 400, [2 ** 31 - 300, 300], [2 ** 31 - 500, 400], True),
    (200, 200, [2 ** 31 - 200, 100, 1000, 100], [2 ** 31 - 150, 150, 0, 50], True),
    (1, 450, [449, 1], [0, 450], True),
    (450, 1, [0, 450], [5000, 1], True),  # no allowed pair at all
])
def test_panel_bytes_match_brute_force(sq, sk, q_seg, k_seg, causal):
    from tests.parity import seg_positions
    got = ea.ea_attn_bwd_ws_bytes(sq, sk, q_seg, k_seg, causal)
    assert got == _panel_blocks_brute(seg_positions(q_seg), seg_positions(k_seg), causal) * 256 * 32 * 2


@pytest.mark.parametrize("W,C", [(8, 37), (4, 100), (8, 43750 // 16)])
def test_panel_bytes_zigzag_steps(W, C):
    for r in (0, W // 2, W - 1):
        pq = oracle.zigzag_positions(2 * W * C, W, r)
        for t in range(W):
            s = oracle.ring_source(r, t, W)
            pk = oracle.zigzag_positions(2 * W * C, W, s)
            got = ea.ea_attn_bwd_ws_bytes(2 * C, 2 * C, ea.ea_zigzag_segments(2 * W * C, W, r),
                                          ea.ea_zigzag_segments(2 * W * C, W, s), True)
            assert got == _panel_blocks_brute(pq, pk, True) * 16384, (r, t)


def test_panel_bytes_errors():
    out = ctypes.c_int64(-1)
    qs, nq = _seg(0, 100)
    ks, nk = _seg(0, 50)
    lib = ea.lib()
    assert lib.ea_attn_bwd_ws_bytes(100, 50, qs, nq, ks, nk, 1, None) == NULL
    assert lib.ea_attn_bwd_ws_bytes(100, 60, qs, nq, ks, nk, 1, ctypes.byref(out)) == POS
    assert lib.ea_attn_bwd_ws_bytes(100, 50, qs, nq, ks, nk, 3, ctypes.byref(out)) == UNSUP
    assert lib.ea_attn_bwd_ws_bytes(-1, 50, qs, nq, ks, nk, 1, ctypes.byref(out)) == SHAPE
    z, nz = _seg(0, 0)
    assert lib.ea_attn_bwd_ws_bytes(0, 50, z, nz, ks, nk, 1, ctypes.byref(out)) == OK and out.value == 0


WS = P + 10 * STEP


def _bwd_ws(ws=WS, ws_bytes=1 << 30, **kw):
    a = dict(q=P, k=P + STEP, v=P + 2 * STEP, o=P + 3 * STEP, o_dtype=0, do=P + 4 * STEP, lse=P + 5 * STEP,
             delta=P + 6 * STEP, ready=0, dq=P + 7 * STEP, dk=P + 8 * STEP, dv=P + 9 * STEP, B=1, H=2, Sq=128,
             Sk=256, D=64, qbr=128, kbr=256, qseg=(0, 128), kseg=(0, 256), mask=1, scale=0.125)
    a.update(kw)
    qs, nq = _seg(*a["qseg"])
    ks, nk = _seg(*a["kseg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_attn_bwd_ws(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["o_dtype"], vp(a["do"]),
                                   vp(a["lse"]), vp(a["delta"]), a["ready"], vp(a["dq"]), vp(a["dk"]),
                                   vp(a["dv"]), a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["qbr"], a["kbr"], qs,
                                   nq, ks, nk, a["mask"], a["scale"], vp(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ws_bytes=16384 * 4 - 16), WORKSPACE),   # one (batch, head) needs 4 blocks here (keys 0..127)
    (dict(ws_bytes=0), WORKSPACE),
    (dict(ws=0), NULL),
    (dict(ws=WS + 8), ALIGN),
    (dict(ws=P + 7 * STEP - 4096), ALIAS),          # runs into dq
    (dict(ws=P + 2 * STEP), ALIAS),                 # over v
    (dict(q=0), NULL), (dict(D=32), UNSUP), (dict(kseg=(0, 255)), POS), (dict(dq=P), ALIAS),
])
def test_bwd_ws_rejects_bad_arguments(kw, code):
    assert _bwd_ws(**kw) == code


def test_bwd_ws_empty_query_is_a_noop():
    assert _bwd_ws(Sq=0, qseg=(0, 0), q=0, ws=0, ws_bytes=0) == OK
