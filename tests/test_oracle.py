"""Pins for the CPU oracle (no GPU).

Each pin ties the oracle to something other than itself: hand-derived fixtures,
a pure-Python brute force on tiny inputs, torch fp64 autograd of the textbook
formula, central finite differences, closed forms and exact invariants.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ev(expr: str) -> float:
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log, "inf": math.inf}))


def _arr(x):
    if isinstance(x, str):
        return _ev(x)
    return np.array([_arr(e) for e in x], dtype=np.float64)


# ---------------------------------------------------------------- fixtures

@pytest.mark.parametrize("name", ["causal_two_tokens.json", "full_one_query.json"])
def test_golden_attention(name):
    g = json.load(open(os.path.join(GOLDEN, name)))
    ins = {k: _arr(v) for k, v in g["inputs"].items()}
    scale = _ev(g["scale"])
    r = A.attn_bwd(ins["q"], ins["k"], ins["v"], ins["do"], g["pos_q"], g["pos_k"], g["causal"], scale)
    o, lse = A.attn_fwd(ins["q"], ins["k"], ins["v"], g["pos_q"], g["pos_k"], g["causal"], scale)
    for key, val in g["expected"].items():
        np.testing.assert_allclose(r[key], _arr(val), rtol=0, atol=1e-14, err_msg=key)
    np.testing.assert_allclose(o, _arr(g["expected"]["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _arr(g["expected"]["lse"]), rtol=0, atol=1e-14)


def test_golden_merge():
    g = json.load(open(os.path.join(GOLDEN, "merge_cases.json")))
    for c in g["cases"]:
        o, lse = A.lse_merge(_arr(c["o1"])[None], np.array([_ev(c["lse1"])]),
                             _arr(c["o2"])[None], np.array([_ev(c["lse2"])]))
        exp_lse = _ev(c["lse"])
        if math.isinf(exp_lse):
            assert lse[0] == exp_lse, c["note"]
        else:
            assert abs(lse[0] - exp_lse) < 1e-14, c["note"]
        np.testing.assert_allclose(o[0], _arr(c["o"]), atol=1e-14, err_msg=c["note"])
        assert not np.isnan(o).any()


def test_golden_zigzag():
    g = json.load(open(os.path.join(GOLDEN, "zigzag_w2_c2.json")))
    for r, pos in g["positions"].items():
        got = oracle.zigzag_positions(g["s_total"], g["world"], int(r))
        assert got.tolist() == pos
        n = A.allowed_mask(got, np.arange(g["s_total"]), True).sum()
        assert n == g["causal_pairs"][r]
        assert [oracle.ring_source(int(r), t, g["world"]) for t in range(g["world"])] == g["ring_sources"][r]


# ---------------------------------------------------------------- brute force

def _brute(q, k, v, do, pos_q, pos_k, causal, scale):
    """Scalar pure-Python evaluation of the definition (tiny sizes only)."""
    sq, d = len(q), len(q[0])
    sk = len(k)
    O = [[0.0] * d for _ in range(sq)]
    L = [-math.inf] * sq
    P = [[0.0] * sk for _ in range(sq)]
    for i in range(sq):
        ok = [j for j in range(sk) if (not causal) or pos_k[j] <= pos_q[i]]
        if not ok:
            continue
        s = {j: scale * sum(q[i][c] * k[j][c] for c in range(d)) for j in ok}
        L[i] = math.log(sum(math.exp(x) for x in s.values()))
        for j in ok:
            P[i][j] = math.exp(s[j] - L[i])
        for c in range(d):
            O[i][c] = sum(P[i][j] * v[j][c] for j in ok)
    dQ = [[0.0] * d for _ in range(sq)]
    dK = [[0.0] * d for _ in range(sk)]
    dV = [[0.0] * d for _ in range(sk)]
    for i in range(sq):
        delta = sum(do[i][c] * O[i][c] for c in range(d))
        for j in range(sk):
            if P[i][j] == 0.0:
                continue
            dp = sum(do[i][c] * v[j][c] for c in range(d))
            ds = P[i][j] * (dp - delta)
            for c in range(d):
                dQ[i][c] += scale * ds * k[j][c]
                dK[j][c] += scale * ds * q[i][c]
                dV[j][c] += P[i][j] * do[i][c]
    return np.array(O), np.array(L), np.array(dQ), np.array(dK), np.array(dV)


def _rand_case(rng, sq, sk, d, pos_mode):
    q = rng.standard_normal((sq, d))
    k = rng.standard_normal((sk, d))
    v = rng.standard_normal((sk, d))
    do = rng.standard_normal((sq, d))
    if pos_mode == "contig":
        pos_q = np.arange(sk - sq, sk) if sk >= sq else np.arange(sq)
        pos_k = np.arange(sk)
    else:  # arbitrary positions, duplicates allowed, unordered
        pos_q = rng.integers(0, 20, size=sq)
        pos_k = rng.integers(0, 20, size=sk)
    return q, k, v, do, pos_q, pos_k


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("pos_mode", ["contig", "random"])
def test_bruteforce_tiny(seed, causal, pos_mode):
    rng = np.random.default_rng(100 + seed)
    sq, sk, d = int(rng.integers(1, 9)), int(rng.integers(1, 11)), int(rng.choice([1, 3, 4]))
    q, k, v, do, pq, pk = _rand_case(rng, sq, sk, d, pos_mode)
    scale = 1.0 / math.sqrt(d) if seed % 2 else 0.7
    bo, bl, bdq, bdk, bdv = _brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), pq.tolist(), pk.tolist(),
                                   causal, scale)
    r = A.attn_bwd(q, k, v, do, pq, pk, causal, scale)
    o, lse = A.attn_fwd(q, k, v, pq, pk, causal, scale)
    np.testing.assert_allclose(o, bo, atol=1e-12)
    np.testing.assert_allclose(r["o"], bo, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(bl))
    fin = np.isfinite(bl)
    np.testing.assert_allclose(lse[fin], bl[fin], atol=1e-12)
    np.testing.assert_allclose(r["dq"], bdq, atol=1e-12)
    np.testing.assert_allclose(r["dk"], bdk, atol=1e-12)
    np.testing.assert_allclose(r["dv"], bdv, atol=1e-12)


# ---------------------------------------------------------------- torch autograd (library routine)

def _torch_ref(q, k, v, do, pq, pk, causal, scale):
    q, k, v, do = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, do))
    mask = torch.ones(len(pq), len(pk), dtype=torch.bool)
    if causal:
        mask = torch.tensor(pk)[None, :] <= torch.tensor(pq)[:, None]
    s = scale * q @ k.T
    s = s.masked_fill(~mask, float("-inf"))
    has = mask.any(dim=1)
    lse = torch.logsumexp(s, dim=1)
    p = torch.softmax(s.masked_fill(~has[:, None], 0.0), dim=1) * has[:, None]
    o = p @ v
    (o * do).sum().backward()
    return o.detach().numpy(), lse.detach().numpy(), q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("d", [4, 64])
def test_torch_autograd(seed, causal, d):
    rng = np.random.default_rng(200 + seed)
    sq, sk = int(rng.integers(1, 65)), int(rng.integers(1, 65))
    q, k, v, do, pq, pk = _rand_case(rng, sq, sk, d, "contig" if seed % 2 else "random")
    scale = 1.0 / math.sqrt(d)
    to, tl, tdq, tdk, tdv = _torch_ref(q, k, v, do, pq, pk, causal, scale)
    r = A.attn_bwd(q, k, v, do, pq, pk, causal, scale)
    np.testing.assert_allclose(r["o"], to, atol=1e-12)
    fin = np.isfinite(tl)
    assert np.array_equal(np.isfinite(r["lse"]), fin)
    np.testing.assert_allclose(r["lse"][fin], tl[fin], atol=1e-12)
    for a, b in ((r["dq"], tdq), (r["dk"], tdk), (r["dv"], tdv)):
        np.testing.assert_allclose(a, b, atol=1e-10)


# ---------------------------------------------------------------- finite differences

def test_finite_differences():
    rng = np.random.default_rng(7)
    sq, sk, d = 5, 7, 3
    q, k, v, do, pq, pk = _rand_case(rng, sq, sk, d, "random")
    pq = np.array([3, 9, 0, 12, 5])           # includes a row that sees few keys
    pk = np.array([0, 2, 4, 6, 8, 10, 12])
    scale = 0.6

    def loss(qq, kk, vv):
        o, _ = A.attn_fwd(qq, kk, vv, pq, pk, True, scale)
        return float(np.sum(o * do))

    r = A.attn_bwd(q, k, v, do, pq, pk, True, scale)
    eps = 1e-6
    for name, x, g in (("q", q, r["dq"]), ("k", k, r["dk"]), ("v", v, r["dv"])):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = loss(args["q"], args["k"], args["v"])
            args[name] = xm
            lm = loss(args["q"], args["k"], args["v"])
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, err_msg=name)


# ---------------------------------------------------------------- closed forms

def test_zero_query_counts_and_means():
    rng = np.random.default_rng(11)
    sq, sk, d = 9, 13, 5
    pq = rng.integers(0, 15, size=sq)
    pk = rng.integers(0, 15, size=sk)
    q = np.zeros((sq, d))
    k = rng.standard_normal((sk, d))
    v = rng.standard_normal((sk, d))
    o, lse = A.attn_fwd(q, k, v, pq, pk, True, 0.3)
    for i in range(sq):
        ok = pk <= pq[i]
        n = int(ok.sum())
        if n == 0:
            assert lse[i] == -np.inf and np.all(o[i] == 0)
        else:
            assert abs(lse[i] - math.log(n)) < 1e-13
            np.testing.assert_allclose(o[i], v[ok].mean(axis=0), atol=1e-13)


def test_single_key_and_constant_v():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((4, 6))
    k = rng.standard_normal((1, 6))
    v = rng.standard_normal((1, 6))
    o, lse = A.attn_fwd(q, k, v, np.zeros(4, int), np.zeros(1, int), True, 0.5)
    np.testing.assert_allclose(o, np.repeat(v, 4, axis=0), atol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]), atol=1e-13)
    # constant V rows: O equals that row whatever the weights
    k2 = rng.standard_normal((10, 6))
    v2 = np.tile(rng.standard_normal((1, 6)), (10, 1))
    o2, _ = A.attn_fwd(q, k2, v2, np.arange(4) + 6, np.arange(10), True, 0.5)
    np.testing.assert_allclose(o2, v2[:4], atol=1e-13)


def test_first_causal_row_is_first_value():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((8, 4)) for _ in range(3))
    o, lse = A.attn_fwd(q, k, v, np.arange(8), np.arange(8), True, 0.5)
    np.testing.assert_allclose(o[0], v[0], atol=1e-15)
    assert abs(lse[0] - 0.5 * q[0] @ k[0]) < 1e-14


# ---------------------------------------------------------------- exact invariants of the gradient

@pytest.mark.parametrize("causal", [True, False])
def test_gradient_invariants(causal):
    rng = np.random.default_rng(21)
    sq, sk, d = 40, 57, 16
    q, k, v, do, pq, pk = _rand_case(rng, sq, sk, d, "random")
    r = A.attn_bwd(q, k, v, do, pq, pk, causal, 0.25)
    has = A.allowed_mask(pq, pk, causal).any(axis=1)
    # sum_j dS_ij = 0 for every row, so sum_j dK_j = 0
    np.testing.assert_allclose(r["dk"].sum(axis=0), 0.0, atol=1e-12)
    # sum_j P_ij = 1 on rows with keys, so sum_j dV_j = sum of those rows' dO
    np.testing.assert_allclose(r["dv"].sum(axis=0), do[has].sum(axis=0), atol=1e-12)
    # empty rows: no gradient, LSE -inf
    assert np.all(r["dq"][~has] == 0) and np.all(r["lse"][~has] == -np.inf)
    # shifting every key by one vector changes no output and no gradient
    c = rng.standard_normal(d)
    r2 = A.attn_bwd(q, k + c, v, do, pq, pk, causal, 0.25)
    for key in ("o", "dq", "dk", "dv"):
        np.testing.assert_allclose(r2[key], r[key], atol=1e-11, err_msg=key)
    # identical keys: uniform weights, dQ = 0
    r3 = A.attn_bwd(q, np.tile(k[:1], (sk, 1)), v, do, pq, pk, causal, 0.25)
    np.testing.assert_allclose(r3["dq"], 0.0, atol=1e-12)


# ---------------------------------------------------------------- key-split merge invariant

def _split_merge(q, k, v, pq, pk, causal, scale, parts):
    o_acc = np.zeros((q.shape[0], v.shape[1]))
    l_acc = np.full(q.shape[0], -np.inf)
    for idx in parts:
        o_p, l_p = A.attn_fwd(q, k[idx], v[idx], pq, pk[idx], causal, scale)
        o_acc, l_acc = A.lse_merge(o_acc, l_acc, o_p, l_p)
    return o_acc, l_acc


@pytest.mark.parametrize("kind", ["contiguous", "interleaved", "random", "with_empty"])
@pytest.mark.parametrize("causal", [True, False])
def test_split_merge_equals_unsplit(kind, causal):
    rng = np.random.default_rng(31)
    sq, sk, d = 33, 70, 8
    q, k, v, _, pq, pk = _rand_case(rng, sq, sk, d, "random")
    scale = 0.35
    o, lse = A.attn_fwd(q, k, v, pq, pk, causal, scale)
    idx = np.arange(sk)
    if kind == "contiguous":
        parts = np.split(idx, [11, 30, 31, 55])
    elif kind == "interleaved":
        parts = [idx[i::4] for i in range(4)]
    elif kind == "random":
        lab = rng.integers(0, 5, size=sk)
        parts = [idx[lab == i] for i in range(5)]
    else:
        parts = [idx[:0], idx[:20], idx[20:20], idx[20:], idx[:0]]
    for order in (parts, parts[::-1], [parts[i] for i in rng.permutation(len(parts))]):
        om, lm = _split_merge(q, k, v, pq, pk, causal, scale, order)
        assert np.array_equal(np.isinf(lm), np.isinf(lse))
        fin = np.isfinite(lse)
        np.testing.assert_allclose(lm[fin], lse[fin], atol=1e-12)
        np.testing.assert_allclose(om, o, atol=1e-12)
        assert not np.isnan(om).any()


# ---------------------------------------------------------------- zigzag reassembly

@pytest.mark.parametrize("W", [1, 2, 3, 4, 8])
@pytest.mark.parametrize("C", [1, 5, 37])
def test_zigzag_reassembles_causal_attention(W, C):
    S = 2 * W * C
    rng = np.random.default_rng(1000 * W + C)
    d = 4
    q, k, v, do = (rng.standard_normal((S, d)) for _ in range(4))
    full = A.attn_bwd(q, k, v, do, np.arange(S), np.arange(S), True, 0.5)
    seen = np.zeros(S, dtype=int)
    o = np.zeros_like(q)
    lse = np.zeros(S)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(W):
        pos = oracle.zigzag_positions(S, W, r)
        seen[pos] += 1
        # the balanced load: 2W C^2 + C allowed pairs on every rank
        assert A.allowed_mask(pos, np.arange(S), True).sum() == 2 * W * C * C + C
        loc = A.attn_bwd(q[pos], k, v, do[pos], pos, np.arange(S), True, 0.5)
        o[pos], lse[pos], dq[pos] = loc["o"], loc["lse"], loc["dq"]
        dk += loc["dk"]
        dv += loc["dv"]
        # ring form of the forward: visit each source rank's keys, merge partials
        o_acc = np.zeros((2 * C, d))
        l_acc = np.full(2 * C, -np.inf)
        srcs = []
        for t in range(W):
            src = oracle.ring_source(r, t, W)
            srcs.append(src)
            kp = oracle.zigzag_positions(S, W, src)
            o_p, l_p = A.attn_fwd(q[pos], k[kp], v[kp], pos, kp, True, 0.5)
            o_acc, l_acc = A.lse_merge(o_acc, l_acc, o_p, l_p)
        assert sorted(srcs) == list(range(W))
        np.testing.assert_allclose(o_acc, loc["o"], atol=1e-12)
        np.testing.assert_allclose(l_acc, loc["lse"], atol=1e-12)
    assert np.all(seen == 1)                       # positions form a bijection
    for a, b in ((o, full["o"]), (lse, full["lse"]), (dq, full["dq"]), (dk, full["dk"]), (dv, full["dv"])):
        np.testing.assert_allclose(a, b, atol=1e-12)


def test_zigzag_rejects_bad_layout():
    with pytest.raises(ValueError):
        oracle.zigzag_positions(10, 3, 0)
    with pytest.raises(ValueError):
        oracle.zigzag_positions(8, 2, 2)


# ---------------------------------------------------------------- allowed-pair sums (probe expectations)

@pytest.mark.parametrize("causal", [True, False])
def test_allowed_sums_match_mask(causal):
    rng = np.random.default_rng(41)
    for _ in range(5):
        sq, sk = int(rng.integers(1, 60)), int(rng.integers(1, 80))
        pq = rng.integers(0, 50, size=sq)
        pk = rng.integers(0, 50, size=sk)
        w = rng.integers(0, 3, size=(sk, 4))
        ref = A.allowed_mask(pq, pk, causal).astype(np.int64) @ w
        assert np.array_equal(A.allowed_sums(pq, pk, causal, w), ref)


def test_allowed_sums_zigzag_count():
    # every rank of an 8-rank zigzag layout sees 16 C^2 + C causal pairs
    C, W = 11, 8
    S = 2 * W * C
    pk = np.arange(S)
    for r in range(W):
        pq = oracle.zigzag_positions(S, W, r)
        assert A.allowed_sums(pq, pk, True, np.ones((S, 1))).sum() == 16 * C * C + C
