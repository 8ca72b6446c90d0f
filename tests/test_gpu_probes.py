"""Bit-exact probes of the mask and position indexing at full workload shapes.

The inputs are chosen so that every probability is exactly 1 on allowed pairs
and 0 elsewhere, and the value / key / query rows carry the binary digits of
their global positions and row indices.  Every output is then an exact integer
(a count of allowed pairs, or a sum of 0/1 digits over them, all < 2^24), so the
GPU result must equal the host expectation exactly:

  forward  (Q = 0, scale any):   O_i * n_i = sum over allowed keys of V_j
  backward (lse = 0, O = 0, scale = 1, V = e_0, dO[:,0] = 1):
      run 1, Q = 0:  dQ_i = sum over allowed keys of K_j;  dV_j = sum over allowed queries of dO_i
      run 2, K = 0:  dK_j = sum over allowed queries of Q_i

Expectations come from the oracle's allowed_sums (keys sorted by position,
prefix sums), itself pinned against the explicit mask in test_oracle.py.
"""
import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea
from tests.parity import banner, seg_positions

pytestmark = pytest.mark.gpu
DEV = "cuda"
NBITS = 20  # positions and row indices of every workload are < 2^20


def _bits(x, nbits=NBITS):
    x = np.asarray(x, dtype=np.int64)
    return ((x[:, None] >> np.arange(nbits)[None, :]) & 1).astype(np.int64)


def _payload(pos, nrows, D):
    """[nrows, D] int: column 0 = 1, 1..20 = bits of the position, 21..40 = bits of the row index."""
    w = np.zeros((nrows, D), dtype=np.int64)
    w[:, 0] = 1
    w[:, 1:1 + NBITS] = _bits(pos)
    w[:, 1 + NBITS:1 + 2 * NBITS] = _bits(np.arange(nrows))
    return w


def _dev(a, H, dtype=torch.bfloat16):
    """[S, D] int array -> [1, S, H, D] device tensor (same values in every head)."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dtype)
    return t[None, :, None, :].expand(1, a.shape[0], H, a.shape[1]).contiguous().to(DEV)


def probe_fwd(q_seg, k_seg, causal, D=128, H=2):
    pq, pk = seg_positions(q_seg), seg_positions(k_seg)
    sq, sk = len(pq), len(pk)
    wv = _payload(pk, sk, D)
    q = torch.zeros((1, sq, H, D), dtype=torch.bfloat16, device=DEV)
    k = _dev(np.random.default_rng(0).integers(-3, 4, size=(sk, D)), H)
    v = _dev(wv, H)
    o = torch.empty((1, sq, H, D), device=DEV)
    lse = torch.empty((1, sq, H), device=DEV)
    ea.ea_attn_fwd(q, k, v, o, lse, q_seg, k_seg, causal, D ** -0.5)
    torch.cuda.synchronize()
    exp_sum = oracle.allowed_sums(pq, pk, causal, wv)        # [sq, D]
    n = exp_sum[:, 0]
    o_np = o[0].double().cpu().numpy()
    lse_np = lse[0].double().cpu().numpy()
    empty = n == 0
    for h in range(H):
        assert np.all(np.isneginf(lse_np[empty, h])), "rows without keys must have LSE = -inf"
        assert np.all(o_np[empty, h] == 0), "rows without keys must have O = 0"
        got = np.rint(o_np[~empty, h] * n[~empty, None]).astype(np.int64)
        assert np.array_equal(got, exp_sum[~empty]), f"head {h}: allowed-key sums differ"
        np.testing.assert_allclose(np.exp(lse_np[~empty, h]), n[~empty], rtol=4e-6)
    return int(n.sum())


def probe_bwd(q_seg, k_seg, causal, D=128, H=2):
    pq, pk = seg_positions(q_seg), seg_positions(k_seg)
    sq, sk = len(pq), len(pk)
    wk = _payload(pk, sk, D)
    wq = _payload(pq, sq, D)
    e0 = np.zeros((sk, D), dtype=np.int64)
    e0[:, 0] = 1
    zq = torch.zeros((1, sq, H, D), dtype=torch.bfloat16, device=DEV)
    zk = torch.zeros((1, sk, H, D), dtype=torch.bfloat16, device=DEV)
    v = _dev(e0, H)
    do = _dev(wq, H)                                           # column 0 = 1
    o = torch.zeros((1, sq, H, D), device=DEV)
    lse = torch.zeros((1, sq, H), device=DEV)
    delta = torch.empty((1, sq, H), device=DEV)
    exp_dq = oracle.allowed_sums(pq, pk, causal, wk)          # per query: sum over allowed keys
    # per key: sum over the queries that may see it (pos_k <= pos_q  <=>  -pos_q <= -pos_k)
    exp_kv = oracle.allowed_sums(-pk, -pq, causal, wq)
    for run in (1, 2):
        q = zq if run == 1 else _dev(wq, H)
        k = _dev(wk, H) if run == 1 else zk
        dq = torch.zeros((1, sq, H, D), device=DEV)
        dk = torch.zeros((1, sk, H, D), device=DEV)
        dv = torch.zeros((1, sk, H, D), device=DEV)
        ea.ea_attn_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, q_seg, k_seg, causal, 1.0)
        torch.cuda.synchronize()
        for h in range(H):
            if run == 1:
                assert np.array_equal(dq[0, :, h].double().cpu().numpy(), exp_dq), f"dQ sums differ (head {h})"
                assert np.array_equal(dv[0, :, h].double().cpu().numpy(), exp_kv), f"dV sums differ (head {h})"
                assert float(dk.abs().max()) == 0.0
            else:
                assert np.array_equal(dk[0, :, h].double().cpu().numpy(), exp_kv), f"dK sums differ (head {h})"
                assert float(dq.abs().max()) == 0.0


DENSE = [("c1", 512, 64), ("c2", 32768, 128), ("t", 65536, 128), ("c5", 131072, 128)]


@pytest.mark.parametrize("name,S,D", DENSE, ids=[d[0] for d in DENSE])
def test_probe_dense_causal(name, S, D):
    banner(f"probe {name}: causal S={S} D={D}")
    n = probe_fwd([0, S], [0, S], True, D)
    assert n == S * (S + 1) // 2
    probe_bwd([0, S], [0, S], True, D)


def test_probe_full_mask_ragged():
    banner("probe full mask, ragged")
    probe_fwd([5, 1000], [0, 777], False)
    probe_bwd([5, 1000], [0, 777], False)


RING = [("c3", 8, 32768), ("c4", 8, 43750)]


@pytest.mark.parametrize("name,W,C", RING, ids=[r[0] for r in RING])
def test_probe_zigzag_ring_all_ranks(name, W, C):
    """Every rank, every ring step, forward; the per-rank total equals 2W C^2 + C."""
    S = 2 * W * C
    for r in range(W):
        q_seg = ea.ea_zigzag_segments(S, W, r)
        total = 0
        for t in range(W):
            src = ea.ea_ring_source(r, t, W)
            k_seg = ea.ea_zigzag_segments(S, W, src)
            banner(f"probe {name} rank {r} step {t} (source {src}) fwd")
            total += probe_fwd(q_seg, k_seg, True, H=1)
        assert total == 2 * W * C * C + C


@pytest.mark.parametrize("name,W,C", RING, ids=[r[0] for r in RING])
@pytest.mark.parametrize("rank", [0, 3, 7])
def test_probe_zigzag_ring_bwd(name, W, C, rank):
    S = 2 * W * C
    q_seg = ea.ea_zigzag_segments(S, W, rank)
    for t in range(W):
        src = ea.ea_ring_source(rank, t, W)
        banner(f"probe {name} rank {rank} step {t} (source {src}) bwd")
        probe_bwd(q_seg, ea.ea_zigzag_segments(S, W, src), True, H=1)
