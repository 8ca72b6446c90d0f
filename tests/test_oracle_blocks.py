"""Pins for the oracle paths that every full-size comparison goes through.

At the full workload sizes the oracle splits a head's query rows into blocks
(at most ROW_BLOCK_ELEMS scores each), drops the keys no row of a block may
see, and adds each block's key gradients into dK and dV.  The ``[B, S, H, D]``
wrappers pick heads and batches out of the token-major tensors.  Both are
checked here on sizes where other evaluations exist: the pure-Python brute
force of the definition, and torch fp64 autograd of masked softmax attention
over the whole ``[B, S, H, D]`` tensors (a library routine, batched over heads
by torch, so it shares no indexing with the wrappers).
"""
import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import rope as R
from tests.test_oracle import _brute


def _positions(rng, mode, sq, sk):
    if mode == "contig":      # queries are the last rows of the keys' range
        return np.arange(sk - sq, sk) if sk >= sq else np.arange(sq), np.arange(sk)
    if mode == "zigzag":      # two segments per side, like a ring rank's share
        c = max(1, sq // 2)
        pq = np.concatenate([np.arange(c), np.arange(3 * c, 3 * c + sq - c)])
        ck = max(1, sk // 2)
        pk = np.concatenate([np.arange(ck, 2 * ck), np.arange(2 * ck + 5, 2 * ck + 5 + sk - ck)])
        return pq, pk
    return rng.integers(0, 30, size=sq), rng.integers(0, 30, size=sk)  # unordered, duplicates


def test_row_blocks_partition_the_rows():
    for sq in (1, 2, 7, 33):
        for sk in (1, 5, 40):
            for budget in (1, sk - 1, sk, 2 * sk + 1, 5 * sk, 10 ** 9):
                blocks = list(A._row_blocks(sq, sk, max(1, budget)))
                assert blocks[0][0] == 0 and blocks[-1][1] == sq
                for (a0, a1), (b0, b1) in zip(blocks, blocks[1:]):
                    assert a1 == b0
                assert all(i1 > i0 for i0, i1 in blocks)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("mode", ["contig", "zigzag", "random"])
@pytest.mark.parametrize("rows_per_block", [1, 2, 3, 7])
def test_row_blocks_match_bruteforce(causal, mode, rows_per_block):
    """Several row blocks per head (each key seen by many blocks) against the scalar definition."""
    rng = np.random.default_rng(100 * rows_per_block + (7 if causal else 0) + len(mode))
    sq, sk, d = 19, 23, 4
    q, k, v, do = (rng.standard_normal(s) for s in ((sq, d), (sk, d), (sk, d), (sq, d)))
    pq, pk = _positions(rng, mode, sq, sk)
    scale = 0.7
    budget = rows_per_block * sk + (sk - 1 if rows_per_block > 1 else 0)  # ragged: a partial row's worth extra
    O, L, dQ, dK, dV = _brute(q.tolist(), k.tolist(), v.tolist(), do.tolist(), pq.tolist(), pk.tolist(), causal,
                              scale)
    r = A.attn_bwd(q, k, v, do, pq, pk, causal, scale, block_elems=budget)
    o, lse = A.attn_fwd(q, k, v, pq, pk, causal, scale, block_elems=budget)
    assert len(list(A._row_blocks(sq, sk, budget))) >= sq // rows_per_block
    fin = np.isfinite(L)
    for got in (r["lse"], lse):
        assert np.array_equal(np.isfinite(got), fin)
        np.testing.assert_allclose(got[fin], L[fin], rtol=0, atol=1e-12)
    for got in (r["o"], o):
        np.testing.assert_allclose(got, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dq"], dQ, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dk"], dK, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["dv"], dV, rtol=0, atol=1e-12)


def _torch_heads(q, k, v, do, pos_q, pos_k, causal, scale):
    """Masked softmax attention over whole [B, S, H, D] fp64 tensors, gradients by torch autograd."""
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = torch.einsum("bihd,bjhd->bhij", qt, kt) * scale
    if causal:
        allowed = torch.tensor(pos_k)[None, :] <= torch.tensor(pos_q)[:, None]
        s = s.masked_fill(~allowed, float("-inf"))
    p = torch.softmax(s, dim=-1)
    o = torch.einsum("bhij,bjhd->bihd", p, vt)
    lse = torch.logsumexp(s, dim=-1).permute(0, 2, 1)
    (o * torch.tensor(do)).sum().backward()
    return {"o": o.detach().numpy(), "lse": lse.detach().numpy(), "dq": qt.grad.numpy(), "dk": kt.grad.numpy(),
            "dv": vt.grad.numpy()}


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("small_blocks", [False, True])
def test_head_wrappers_match_batched_torch(causal, small_blocks, monkeypatch):
    """attn_fwd_heads / attn_bwd_heads on B = 2 and distinct heads, all heads and a reordered subset."""
    rng = np.random.default_rng(31 + causal)
    B, sq, sk, H, D = 2, 9, 11, 3, 4
    q, do = rng.standard_normal((B, sq, H, D)), rng.standard_normal((B, sq, H, D))
    k, v = rng.standard_normal((B, sk, H, D)), rng.standard_normal((B, sk, H, D))
    pq = rng.integers(3, 20, size=sq)
    pk = np.concatenate([[0], rng.integers(0, 20, size=sk - 1)])  # every query row sees key 0
    scale = 0.45
    if small_blocks:  # the default budget, shrunk so every head runs several row blocks
        monkeypatch.setattr(A, "ROW_BLOCK_ELEMS", 2 * sk + 3)
    ref = _torch_heads(q, k, v, do, pq, pk, causal, scale)
    for heads in (None, [2, 0]):
        sel = list(range(H)) if heads is None else heads
        o, lse = A.attn_fwd_heads(q, k, v, pq, pk, causal, scale, heads=heads)
        r = A.attn_bwd_heads(q, k, v, do, pq, pk, causal, scale, heads=heads)
        np.testing.assert_allclose(o, ref["o"][:, :, sel], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, ref["lse"][:, :, sel], rtol=0, atol=1e-12)
        for key in ("o", "lse", "dq", "dk", "dv"):
            np.testing.assert_allclose(r[key], ref[key][:, :, sel], rtol=0, atol=1e-12, err_msg=key)
        np.testing.assert_allclose(r["delta"], np.sum(ref["o"] * do, axis=-1)[:, :, sel], rtol=0, atol=1e-12)


def test_rope_head_wrapper_matches_single_heads():
    """attn_bwd_rope_heads on B = 2, distinct heads, a reordered subset: each output slice equals the single-head
    oracle (itself pinned by the rotary and attention pins) on that batch's and head's rows."""
    rng = np.random.default_rng(5)
    B, sq, H, D = 2, 8, 3, 4
    q, k, v, do = (rng.standard_normal((B, sq, H, D)) for _ in range(4))
    pos = np.arange(100, 100 + sq)
    heads = [1, 2, 0]
    r = R.attn_bwd_rope_heads(q, k, v, do, pos, pos, True, 0.5, 1e4, heads=heads)
    for b in range(B):
        for n, h in enumerate(heads):
            one = R.attn_bwd_rope(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], pos, pos, True, 0.5, 1e4)
            for key in ("o", "lse", "delta", "dq", "dk", "dv"):
                np.testing.assert_array_equal(r[key][b, :, n], one[key], err_msg=f"{key} b={b} h={h}")
