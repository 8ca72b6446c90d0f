"""Oracle: cross-entropy over vocabulary logits and its gradient with respect to the logits.

TEST INFRASTRUCTURE ONLY (see the package header).

The training script the pages walk through computes its language-model loss
with FlashAttention's fused cross-entropy kernel, backward done in place over
the logits (EasyContext memory-optimisation page on DeepSpeed ZeRO-3 offload,
kwkr.cn, section on advanced optimisation combined with other techniques, item
1; EasyContext "1M tokens with minimal resources" page, cn486.com, the summary
of the training script's technology stack).  No
formula is printed; this is the textbook definition, per row i of a [N, V]
logit matrix x with integer label y_i:

  LSE_i  = ln sum_j exp(x_ij)
  loss_i = LSE_i - x_{i, y_i}
  dx_ij  = g * (exp(x_ij - LSE_i) - [j == y_i])

for a scalar upstream gradient g per row (for a mean over the rows that are not
ignored, g = 1 / that count).  Reading: a row whose label equals ignore_index
contributes loss 0 and gradient 0; its LSE is still reported.
"""
import numpy as np


def xent_fwd_bwd(logits, labels, grad_scale=1.0, ignore_index=-100):
    """fp64 per-row loss, LSE and gradient of the loss with respect to the logits."""
    x = np.asarray(logits, dtype=np.float64)
    y = np.asarray(labels, dtype=np.int64)
    n, v = x.shape
    m = x.max(axis=1)
    lse = m + np.log(np.exp(x - m[:, None]).sum(axis=1))
    keep = y != ignore_index
    if np.any(keep & ((y < 0) | (y >= v))):
        raise ValueError("label out of range")
    rows = np.arange(n)
    picked = np.where(keep, x[rows, np.where(keep, y, 0)], 0.0)
    loss = np.where(keep, lse - picked, 0.0)
    p = np.exp(x - lse[:, None])
    grad = p.copy()
    grad[rows[keep], y[keep]] -= 1.0
    grad *= grad_scale
    grad[~keep] = 0.0
    return {"loss": loss, "lse": lse, "grad": grad}
