"""Oracle: rotary position embedding (RoPE) of query and key rows by their global positions.

TEST INFRASTRUCTURE ONLY (see the package header).

The pages extend the context by raising the base frequency of the rotary
position encoding: EasyContext core-technology page (hotelren.com), the list of
further optimisations; the 200-line training-script walkthrough (mlqm.cn), key
optimisation tips (the rope-theta option); the ZeRO-3 offload page (kwkr.cn),
the training script's rope-theta of 1e6 and the section on advanced
optimisation, item 2; the "1M tokens" page (cn486.com), training strategy (the
base raised step by step to 1e9).  They print no formula.  Reading: the Llama
convention ("rotate-half") that the models they train use.  For one head row x
of even dimension D at integer position p, and k = 0 .. D/2-1:

  phi_k        = p * theta^(-2k/D)
  x'_k         = x_k cos(phi_k) - x_{k+D/2} sin(phi_k)
  x'_{k+D/2}   = x_{k+D/2} cos(phi_k) + x_k sin(phi_k)

The rotation is orthogonal; its inverse (the transpose, rotation by -phi_k)
carries a gradient with respect to the rotated rows back to the unrotated ones.

`attn_bwd_rope` is the attention step on unrotated inputs: rotate Q and K by
their positions, round the rotated rows once to bf16 (reading: the rotated
tensors are stored in the input precision, as the attention inputs are), run
the attention oracle, and rotate dQ and dK back.
"""
import numpy as np

from .attention import _f64, attn_bwd


def inv_freq(D: int, theta: float) -> np.ndarray:
    """theta^(-2k/D) for k = 0 .. D/2-1, fp64."""
    if D % 2:
        raise ValueError("D must be even")
    k = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * k / D)


def rope(x, pos, theta: float, inverse: bool = False) -> np.ndarray:
    """Rotate x [..., S, H, D] (positions pos [S]) in fp64; inverse=True applies the transpose."""
    x = _f64(x)
    pos = np.asarray(pos, dtype=np.int64)
    D = x.shape[-1]
    half = D // 2
    if x.shape[-3] != pos.shape[0]:
        raise ValueError("one position per row")
    phi = pos.astype(np.float64)[:, None] * inv_freq(D, theta)[None, :]  # [S, D/2]
    c = np.cos(phi)[:, None, :]   # broadcast over heads
    s = np.sin(phi)[:, None, :]
    if inverse:
        s = -s
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bfloat16 (ties to even), returned as fp64.

    bfloat16 keeps the sign, the 8-bit exponent and the top 7 fraction bits of
    an IEEE single; for normal values in single range this is rounding the fp64
    significand to 8 bits.  The fp64 pattern is rounded directly (no detour
    through fp32, so no double rounding).
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    bits = x.view(np.uint64)
    drop = np.uint64(52 - 7)                      # fraction bits removed
    one = np.uint64(1)
    half_ulp = (one << (drop - one)) - one        # just under half of the kept last place
    lsb = (bits >> drop) & one                    # ties go to the even neighbour
    r = (bits + half_ulp + lsb) & ~((one << drop) - one)
    out = r.view(np.float64)
    return np.where(np.isfinite(x), out, x)


def attn_bwd_rope(q, k, v, do, pos_q, pos_k, causal: bool, scale: float, theta: float):
    """One head on unrotated q [Sq, D], k [Sk, D]: O, LSE and the gradients w.r.t. the unrotated q, k.

    Returns the dict of `attn_bwd` with dq and dk rotated back, plus the rotated
    bf16 inputs used ("q_rot", "k_rot").
    """
    qr = round_bf16(rope(_f64(q)[:, None, :], pos_q, theta)[:, 0, :])
    kr = round_bf16(rope(_f64(k)[:, None, :], pos_k, theta)[:, 0, :])
    out = attn_bwd(qr, kr, v, do, pos_q, pos_k, causal, scale)
    out["dq"] = rope(out["dq"][:, None, :], pos_q, theta, inverse=True)[:, 0, :]
    out["dk"] = rope(out["dk"][:, None, :], pos_k, theta, inverse=True)[:, 0, :]
    out["q_rot"], out["k_rot"] = qr, kr
    return out


def attn_bwd_rope_heads(q, k, v, do, pos_q, pos_k, causal, scale, theta, heads=None):
    """[B, S, H, D] layout over the selected heads, like `attn_bwd_heads`, for unrotated q and k."""
    B, sq, H, D = q.shape
    sk = k.shape[1]
    heads = list(range(H)) if heads is None else list(heads)
    nh = len(heads)
    res = {"o": np.zeros((B, sq, nh, D)), "lse": np.zeros((B, sq, nh)), "delta": np.zeros((B, sq, nh)),
           "dq": np.zeros((B, sq, nh, D)), "dk": np.zeros((B, sk, nh, D)), "dv": np.zeros((B, sk, nh, D))}
    for b in range(B):
        for n, h in enumerate(heads):
            r = attn_bwd_rope(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], pos_q, pos_k, causal, scale, theta)
            for key in res:
                res[key][b, :, n] = r[key]
    return res
