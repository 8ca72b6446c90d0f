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
    assert ea.ea_version() >= 200
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


def _bf(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.bfloat16)


def _f32(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.float32)


def _expect(match, fn, *args, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*args, **kw)


def test_python_binding_checks_before_the_library():
    """Every wrapper checks dtypes, the B/Sq/Sk extents, strides and the device of every tensor first: a wrong
    tensor would otherwise reach the kernels (a host pointer, a batch past the end, fp32 writes into bf16)."""
    B, S, Sk, H, D = 2, 8, 6, 2, 64
    q, do, k, v = _bf(B, S, H, D), _bf(B, S, H, D), _bf(B, Sk, H, D), _bf(B, Sk, H, D)
    o, dq, dk, dv = _f32(B, S, H, D), _f32(B, S, H, D), _f32(B, Sk, H, D), _f32(B, Sk, H, D)
    lse, delta = _f32(B, S, H), _f32(B, S, H)
    seg_q, seg_k = [0, S], [0, Sk]
    fwd = lambda **c: ea.ea_attn_fwd(**{**dict(q=q, k=k, v=v, o=o, lse=lse, q_seg=seg_q, k_seg=seg_k), **c})
    bwd = lambda **c: ea.ea_attn_bwd(**{**dict(q=q, k=k, v=v, o=o, dout=do, lse=lse, delta=delta, dq=dq, dk=dk,
                                               dv=dv, q_seg=seg_q, k_seg=seg_k), **c})
    # batch count: k with one batch against q's two would read past the end of k
    _expect("k must be", fwd, k=_bf(1, Sk, H, D), v=_bf(1, Sk, H, D))
    _expect("v must have shape", fwd, v=_bf(B, Sk + 1, H, D))
    _expect("o must have shape", fwd, o=_f32(B, S + 1, H, D))
    _expect("lse must have shape", fwd, lse=_f32(1, S, H))
    _expect("lse must be", fwd, lse=_bf(B, S, H))
    # fp32 outputs: a bf16 buffer would take writes up to twice its size
    for name, bad in (("dq", _bf(B, S, H, D)), ("dk", _bf(B, Sk, H, D)), ("dv", _bf(B, Sk, H, D)),
                      ("delta", _bf(B, S, H)), ("lse", _bf(B, S, H))):
        _expect(f"{name} must be torch.float32", bwd, **{name: bad})
    _expect("dout must have shape", bwd, dout=_bf(B, Sk, H, D))
    _expect("dk must have shape", bwd, dk=_f32(B, S, H, D))
    _expect("delta must have shape", bwd, delta=_f32(B, S + 2, H))
    _expect("q must be", bwd, q=_f32(B, S, H, D))
    _expect("o is needed", bwd, o=None)
    # the merge: fp32 accumulators, matching shapes
    _expect("o_acc must be", ea.ea_lse_merge, _bf(B, S, H, D), lse, o, lse)
    _expect("lse_part must be", ea.ea_lse_merge, o, lse, o, _bf(B, S, H))
    _expect("o_part must have shape", ea.ea_lse_merge, o, lse, _f32(B, S - 1, H, D), lse)
    _expect("lse_acc must have shape", ea.ea_lse_merge, o, _f32(B, S - 1, H), o, lse)
    # the fused-merge forward needs an fp32 accumulator; the rotary forward a bf16 q_rot of q's shape
    _expect("o must be torch.float32", ea.ea_attn_fwd_merge, q, k, v, _bf(B, S, H, D), lse, seg_q, seg_k)
    _expect("q_rot must be", ea.ea_attn_fwd_rope, q, k, v, o, lse, seg_q, seg_k, 1e6, q_rot=o)
    _expect("q_rot must have shape", ea.ea_attn_fwd_rope, q, k, v, o, lse, seg_q, seg_k, 1e6, q_rot=_bf(B, S, H + 1, D))
    _expect("o must be torch.float32", ea.ea_attn_fwd_rope, q, k, v, _bf(B, S, H, D), lse, seg_q, seg_k, 1e6,
            merge=True)
    _expect("x must be", ea.ea_rope, torch_int(B, S, H, D), torch_int(B, S, H, D), seg_q, 1e6)
    # every check above passes for these host tensors, so the device check is what stops them
    _expect("on cpu", fwd)
    _expect("on cpu", bwd)
    _expect("on cpu", ea.ea_attn_fwd_rope, q, k, v, o, lse, seg_q, seg_k, 1e6, q_rot=_bf(B, S, H, D))
    _expect("on cpu", ea.ea_attn_bwd_rope, q, k, v, o, do, lse, delta, dq, dk, dv, seg_q, seg_k, 1e6)
    _expect("on cpu", ea.ea_lse_merge, o, lse, _bf(B, S, H, D), lse)
    _expect("on cpu", ea.ea_rope, q, q, seg_q, 1e6)
    import torch
    x, y = _bf(4, 16), torch.zeros(4, dtype=torch.int64)
    _expect("on cpu", ea.ea_xent_fwd_bwd, x, y, _f32(4), _f32(4))


def torch_int(*shape):
    import torch
    return torch.zeros(*shape, dtype=torch.int32)


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


# ---- forward and backward with the rotary embedding fused in (ea_attn_fwd_rope, ea_attn_bwd_rope)

def _fwd_rope(**kw):
    a = dict(q=P, k=P + STEP, v=P + 2 * STEP, o=P + 3 * STEP, o_dtype=0, lse=P + 4 * STEP, qr=P + 5 * STEP, merge=0,
             B=1, H=2, Sq=128, Sk=128, D=128, qbr=128, kbr=128, qseg=(0, 128), kseg=(0, 128), mask=1, scale=0.088,
             theta=1e6)
    a.update(kw)
    qs, nq = _seg(*a["qseg"])
    ks, nk = _seg(*a["kseg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_attn_fwd_rope(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["o_dtype"], vp(a["lse"]),
                                     vp(a["qr"]), a["merge"], a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["qbr"],
                                     a["kbr"], qs, nq, ks, nk, a["mask"], a["scale"], a["theta"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(o=0), NULL), (dict(lse=0), NULL), (dict(k=0), NULL),
    (dict(B=0), SHAPE), (dict(D=96), UNSUP), (dict(mask=2), UNSUP), (dict(scale=0.0), UNSUP),
    (dict(theta=0.0), UNSUP), (dict(theta=-1e4), UNSUP), (dict(theta=float("inf")), UNSUP),
    (dict(theta=float("nan")), UNSUP), (dict(merge=2), UNSUP), (dict(merge=-1), UNSUP),
    (dict(merge=1, o_dtype=1), UNSUP), (dict(qseg=(0, 100)), POS),
    (dict(qr=P + 5 * STEP + 8), ALIGN), (dict(q=P + 8), ALIGN),
    (dict(qr=P), ALIAS), (dict(qr=P + 3 * STEP + 64), ALIAS), (dict(qr=P + STEP), ALIAS), (dict(o=P), ALIAS),
])
def test_fwd_rope_rejects_bad_arguments(kw, code):
    assert _fwd_rope(**kw) == code


def test_fwd_rope_empty_query_is_a_noop_without_pointers():
    assert _fwd_rope(Sq=0, qseg=(0, 0), q=0, o=0, lse=0, qr=0) == OK


def _bwd_rope(**kw):
    a = dict(q=P, k=P + STEP, v=P + 2 * STEP, o=P + 3 * STEP, o_dtype=0, do=P + 4 * STEP, lse=P + 5 * STEP,
             delta=P + 6 * STEP, ready=0, dq=P + 7 * STEP, dk=P + 8 * STEP, dv=P + 9 * STEP, B=1, H=2, Sq=128,
             Sk=256, D=64, qbr=128, kbr=256, qseg=(0, 128), kseg=(0, 256), mask=1, scale=0.125, theta=1e9)
    a.update(kw)
    qs, nq = _seg(*a["qseg"])
    ks, nk = _seg(*a["kseg"])
    vp = ctypes.c_void_p
    return ea.lib().ea_attn_bwd_rope(vp(a["q"]), vp(a["k"]), vp(a["v"]), vp(a["o"]), a["o_dtype"], vp(a["do"]),
                                     vp(a["lse"]), vp(a["delta"]), a["ready"], vp(a["dq"]), vp(a["dk"]),
                                     vp(a["dv"]), a["B"], a["H"], a["Sq"], a["Sk"], a["D"], a["qbr"], a["kbr"], qs,
                                     nq, ks, nk, a["mask"], a["scale"], a["theta"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(dq=0), NULL), (dict(dk=0), NULL), (dict(o=0), NULL),
    (dict(theta=0.0), UNSUP), (dict(theta=float("inf")), UNSUP), (dict(theta=float("nan")), UNSUP),
    (dict(D=32), UNSUP), (dict(H=0), SHAPE), (dict(kseg=(0, 255)), POS),
    (dict(dq=P + 7 * STEP + 4), ALIGN), (dict(dq=P), ALIAS), (dict(dk=P + 5 * STEP), ALIAS),
])
def test_bwd_rope_rejects_bad_arguments(kw, code):
    assert _bwd_rope(**kw) == code


def test_bwd_rope_empty_query_is_a_noop():
    assert _bwd_rope(Sq=0, qseg=(0, 0), q=0, do=0, lse=0, delta=0, dq=0, o=0) == OK


# ---- launch sizes: a grid needing 2^32 threads or more is a shape error found on the host.  The cases just
# below each bound carry a misaligned pointer, an error checked after the sizes, so no call ever launches.

def test_attention_launch_size_bounds():
    # Delta: B*H*Sq*D/8 threads in 256-thread workgroups
    assert _fwd(H=1024, Sq=1 << 18, qbr=1 << 18, qseg=(0, 1 << 18), q=P + 8) == SHAPE
    assert _fwd(H=1024, Sq=(1 << 18) - 16, qbr=(1 << 18) - 16, qseg=(0, (1 << 18) - 16), q=P + 8) == ALIGN
    assert _bwd(H=2048, D=64, Sq=1 << 18, qbr=1 << 18, qseg=(0, 1 << 18), dq=P + 7 * STEP + 4) == SHAPE
    # dK/dV: B*H*ceil(Sk/128) workgroups of 512 threads
    big = 1 << 20
    assert _bwd(H=1024, Sk=big, kbr=big, kseg=(0, big), dq=P + 7 * STEP + 4) == SHAPE
    assert _bwd(H=1024, Sk=big - 128, kbr=big - 128, kseg=(0, big - 128), dq=P + 7 * STEP + 4) == ALIGN
    assert _fwd_rope(H=1024, Sq=1 << 18, qbr=1 << 18, qseg=(0, 1 << 18), q=P + 8) == SHAPE


def test_elementwise_launch_size_bounds():
    assert _merge(H=1024, D=128, Sq=1 << 18, qbr=1 << 18) == SHAPE
    assert _merge(H=1024, D=128, Sq=(1 << 18) - 16, qbr=(1 << 18) - 16, oa=P + 4) == ALIGN
    assert _xent(rows=1 << 23) == SHAPE
    assert _xent(rows=(1 << 23) - 1, y=P + STEP + 4) == ALIGN
    assert _rope(B=1, S=1 << 26, br=1 << 26, seg=(0, 1 << 26)) == SHAPE
    assert _rope(B=1, S=(1 << 26) - 4, br=(1 << 26) - 4, seg=(0, (1 << 26) - 4), x=P + 8) == ALIGN
