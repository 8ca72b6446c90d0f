"""Oracle: masked softmax attention, its vector-Jacobian product and the LSE merge.

Plain fp64 NumPy on the exact (upcast) input values.  Per head, with query rows
q_i, keys k_j, values v_j, global integer positions pos_q(i), pos_k(j) and
softmax scale s:

  allowed(i, j)  = True                     (full mask)
                 = pos_k(j) <= pos_q(i)     (causal mask; the diagonal is kept)
  S_ij   = s <q_i, k_j>           where allowed, else -inf
  LSE_i  = ln sum_j exp(S_ij)     (-inf for a row with no allowed key)
  P_ij   = exp(S_ij - LSE_i)
  O_i    = sum_j P_ij v_j         (0 for a row with no allowed key)

Backward with cotangent dO (the recompute-from-LSE gradient that the
core-technology page's Flash Attention section refers to; hotelren.com, section
2):

  Delta_i = <dO_i, O_i>
  dP_ij   = <dO_i, v_j>
  dS_ij   = P_ij (dP_ij - Delta_i)
  dV_j    = sum_i P_ij dO_i
  dQ_i    = s sum_j dS_ij k_j
  dK_j    = s sum_i dS_ij q_i

Merge of two partial results over disjoint key sets (ring attention visits the
keys one rank's share at a time; hotelren.com page, section 1):

  LSE = ln(exp LSE_1 + exp LSE_2)
  O   = exp(LSE_1 - LSE) O_1 + exp(LSE_2 - LSE) O_2

with a side whose LSE is -inf contributing nothing, and (-inf, 0) when both are.

Readings (the pages print no formula): natural-log LSE; the causal rule keeps
the diagonal (causal-LM training of Llama models); empty rows give LSE = -inf,
O = 0 and zero gradients.

The forward is computed two-pass per row: the row maximum first, then the sum
of exponentials and P V using that maximum.  Rows are processed in blocks only
to bound memory (rows are independent; a block holds at most ROW_BLOCK_ELEMS
scores, or the ``block_elems`` a caller passes); inside a block the keys that
no row of the block may see are dropped before the products, which removes
exact zeros from the sums and nothing else.  Key gradients add up over the
blocks.
"""
import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):          # torch tensor (any dtype, incl. bf16)
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def allowed_mask(pos_q, pos_k, causal: bool) -> np.ndarray:
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    if not causal:
        return np.ones((pos_q.shape[0], pos_k.shape[0]), dtype=bool)
    return pos_k[None, :] <= pos_q[:, None]


def allowed_sums(pos_q, pos_k, causal: bool, weights) -> np.ndarray:
    """Per query row i: sum over the keys j allowed for i of weights[j] (weights [Sk, C]).

    Same rule as allowed_mask, evaluated for long sequences without forming the
    mask: keys sorted by position, prefix sums, and for each query the number of
    keys with pos_k <= pos_q(i).  Exact for integer weights.
    """
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    w = np.asarray(weights, dtype=np.int64).reshape(pos_k.shape[0], -1)
    total = w.sum(axis=0)
    if not causal:
        return np.broadcast_to(total, (pos_q.shape[0], w.shape[1])).copy()
    order = np.argsort(pos_k, kind="stable")
    csum = np.concatenate([np.zeros((1, w.shape[1]), dtype=np.int64), np.cumsum(w[order], axis=0)])
    n = np.searchsorted(pos_k[order], pos_q, side="right")
    return csum[n]


ROW_BLOCK_ELEMS = 1 << 24   # scores held at once (128 MiB of fp64)


def _row_blocks(sq: int, sk: int, budget_elems: int):
    rows = max(1, min(sq, budget_elems // max(1, sk)))
    for i0 in range(0, sq, rows):
        yield i0, min(sq, i0 + rows)


def _block_fwd(qb, kc, vc, mask, scale):
    """Two-pass softmax over one row block; kc/vc already restricted to useful keys."""
    s = scale * (qb @ kc.T)
    s = np.where(mask, s, NEG_INF)
    has = mask.any(axis=1)
    m = np.where(has, np.max(s, axis=1, initial=NEG_INF), 0.0)
    e = np.exp(s - m[:, None])                      # exp(-inf) = 0 on masked entries
    l = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(has, m + np.log(np.where(has, l, 1.0)), NEG_INF)
    p = np.where(has[:, None], np.exp(s - np.where(has, lse, 0.0)[:, None]), 0.0)
    o = p @ vc
    return o, lse, p


def _useful_keys(pos_q_blk, pos_k, causal):
    if not causal:
        return np.arange(pos_k.shape[0])
    return np.nonzero(pos_k <= pos_q_blk.max())[0] if pos_q_blk.size else np.arange(0)


def attn_fwd(q, k, v, pos_q, pos_k, causal: bool, scale: float, block_elems=None):
    """One head.  q [Sq, D], k/v [Sk, D] -> O [Sq, D] fp64, LSE [Sq] fp64.

    block_elems: scores per row block (default ROW_BLOCK_ELEMS); any value gives the same result."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    sq, d = q.shape
    sk = k.shape[0]
    o = np.zeros((sq, v.shape[1]), dtype=np.float64)
    lse = np.full(sq, NEG_INF)
    for i0, i1 in _row_blocks(sq, sk, ROW_BLOCK_ELEMS if block_elems is None else block_elems):
        cols = _useful_keys(pos_q[i0:i1], pos_k, causal)
        if cols.size == 0:
            continue
        mask = allowed_mask(pos_q[i0:i1], pos_k[cols], causal)
        ob, lb, _ = _block_fwd(q[i0:i1], k[cols], v[cols], mask, scale)
        o[i0:i1] = ob
        lse[i0:i1] = lb
    return o, lse


def attn_bwd(q, k, v, do, pos_q, pos_k, causal: bool, scale: float, block_elems=None):
    """One head.  Returns dict with o, lse, delta, dq, dk, dv (all fp64).

    block_elems: scores per row block (default ROW_BLOCK_ELEMS); any value gives the same result."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    pos_q = np.asarray(pos_q, dtype=np.int64)
    pos_k = np.asarray(pos_k, dtype=np.int64)
    sq, d = q.shape
    sk = k.shape[0]
    o = np.zeros((sq, v.shape[1]))
    lse = np.full(sq, NEG_INF)
    delta = np.zeros(sq)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i0, i1 in _row_blocks(sq, sk, ROW_BLOCK_ELEMS if block_elems is None else block_elems):
        cols = _useful_keys(pos_q[i0:i1], pos_k, causal)
        if cols.size == 0:
            continue
        kc, vc = k[cols], v[cols]
        mask = allowed_mask(pos_q[i0:i1], pos_k[cols], causal)
        ob, lb, p = _block_fwd(q[i0:i1], kc, vc, mask, scale)
        o[i0:i1] = ob
        lse[i0:i1] = lb
        dob = do[i0:i1]
        dl = np.sum(dob * ob, axis=1)
        delta[i0:i1] = dl
        dp = dob @ vc.T
        ds = p * (dp - dl[:, None])
        dq[i0:i1] = scale * (ds @ kc)
        dk[cols] += scale * (ds.T @ q[i0:i1])
        dv[cols] += p.T @ dob
    return {"o": o, "lse": lse, "delta": delta, "dq": dq, "dk": dk, "dv": dv}


def lse_merge(o1, lse1, o2, lse2):
    """Combine partial (O, LSE) over two disjoint key sets.

    lse* have shape R (any), o* have shape R + (D,).
    """
    o1, o2 = _f64(o1), _f64(o2)
    lse1, lse2 = _f64(lse1), _f64(lse2)
    lse = np.logaddexp(lse1, lse2)                  # -inf with -inf gives -inf
    fin = np.isfinite(lse)
    safe = np.where(fin, lse, 0.0)
    w1 = np.where(fin, np.exp(lse1 - safe), 0.0)[..., None]
    w2 = np.where(fin, np.exp(lse2 - safe), 0.0)[..., None]
    return w1 * o1 + w2 * o2, lse


# ---- [B, S, H, D] helpers: heads and batches are independent problems ----
# Inputs may be torch tensors or arrays of any dtype; each head is upcast to fp64
# on its own so that large workloads never hold a whole fp64 copy.

def _dims(q, k):
    B, sq, H, D = q.shape
    return B, sq, H, D, k.shape[1]


def attn_fwd_heads(q, k, v, pos_q, pos_k, causal, scale, heads=None):
    """q [B,Sq,H,D], k/v [B,Sk,H,D] -> O [B,Sq,H',D], LSE [B,Sq,H'] over the selected heads."""
    B, sq, H, D, sk = _dims(q, k)
    heads = list(range(H)) if heads is None else list(heads)
    o = np.zeros((B, sq, len(heads), D))
    lse = np.zeros((B, sq, len(heads)))
    for b in range(B):
        for n, h in enumerate(heads):
            o[b, :, n], lse[b, :, n] = attn_fwd(q[b, :, h], k[b, :, h], v[b, :, h], pos_q, pos_k, causal, scale)
    return o, lse


def attn_bwd_heads(q, k, v, do, pos_q, pos_k, causal, scale, heads=None):
    """Same layout; returns o, lse, delta, dq (query side) and dk, dv (key side) per selected head."""
    B, sq, H, D, sk = _dims(q, k)
    heads = list(range(H)) if heads is None else list(heads)
    nh = len(heads)
    res = {"o": np.zeros((B, sq, nh, D)), "lse": np.zeros((B, sq, nh)), "delta": np.zeros((B, sq, nh)),
           "dq": np.zeros((B, sq, nh, D)), "dk": np.zeros((B, sk, nh, D)), "dv": np.zeros((B, sk, nh, D))}
    for b in range(B):
        for n, h in enumerate(heads):
            r = attn_bwd(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], pos_q, pos_k, causal, scale)
            for key, val in r.items():
                res[key][b, :, n] = val
    return res
