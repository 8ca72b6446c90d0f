"""GPU parity of the fused cross-entropy (forward + in-place backward) against the fp64 oracle.

Bars, from the arithmetic: loss and LSE within 2e-4 absolute (fp32 sums of up to
10^5 exponentials); gradient per element within 2^-8 |ref| (bf16 output: round to
nearest even, 2^-9 relative, doubled for the fp32 error before rounding) or
1e-5 |ref| (fp32 output), plus g p (|x| + |lse|) 2^-21 for the fp32 exponent
argument (x log2e and lse log2e are rounded products, so p = exp(x - lse) carries
a relative error proportional to the magnitudes involved; where p is 1 and the
gradient 0, as with one class, that term is all that remains).  Ignored rows must
be exactly 0; a label outside [0, V) must give NaN loss and gradient.
"""
import numpy as np
import pytest
import torch

import long_context_causal_ea_amd as ea
from oracle.xent import xent_fwd_bwd
from tests.parity import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(rows, V, dtype, seed, row_stride=None, ignore_frac=0.1, outliers=True):
    g = torch.Generator().manual_seed(seed)
    rs = V if row_stride is None else row_stride
    x = torch.randn((rows, rs), generator=g) * 2.0
    if outliers:
        x[::5, 3 % V] += 30.0       # a dominant logit in some rows
        x[1::7, (V - 1)] -= 40.0    # a very negative one in others
    x = x.to(dtype)
    y = torch.randint(0, V, (rows,), generator=g)
    y[torch.rand(rows, generator=g) < ignore_frac] = -100
    y[0] = V - 1                    # a label in the last (possibly partial) chunk
    if rows > 1:
        y[1] = 0
    return x, y


def _check(name, x, y, V, grad_scale, ignore_index=-100, col0=0):
    rows = x.shape[0]
    cols = slice(col0, col0 + V)
    ref_in = x[:, cols].double().numpy()
    ref = xent_fwd_bwd(ref_in, y.numpy(), grad_scale, ignore_index)
    xd = x.to(DEV)
    yd = y.to(DEV)
    loss = torch.empty(rows, device=DEV)
    lse = torch.empty(rows, device=DEV)
    ea.ea_xent_fwd_bwd(xd[:, cols], yd, loss, lse, grad_scale, ignore_index)
    torch.cuda.synchronize()
    got = xd[:, cols].double().cpu().numpy()
    np.testing.assert_allclose(lse.double().cpu().numpy(), ref["lse"], rtol=0, atol=2e-4, err_msg=f"{name} lse")
    np.testing.assert_allclose(loss.double().cpu().numpy(), ref["loss"], rtol=0, atol=2e-4, err_msg=f"{name} loss")
    # fp32 forms exp(x - lse) as exp2(x log2e - lse log2e): each product carries a rounding of its own size,
    # so p = exp(x - lse) is off by up to p (|x| + |lse|) 2^-22 (relative to p, not to the gradient, which may be 0)
    p = np.exp(ref_in - ref["lse"][:, None])
    arg = np.abs(ref_in) + np.abs(ref["lse"])[:, None]
    fp32_term = abs(grad_scale) * p * arg * 2.0 ** -21 + 1e-30
    if x.dtype == torch.bfloat16:
        tol = 2.0 ** -8 * np.abs(ref["grad"]) + fp32_term
    else:
        tol = 1e-5 * np.abs(ref["grad"]) + fp32_term
    err = np.abs(got - ref["grad"])
    worst = float((err / tol).max())
    rel = float(np.linalg.norm(got - ref["grad"]) / max(np.linalg.norm(ref["grad"]), 1e-30))
    print(f"  {name}: grad max err/tol {worst:.3f}, rel-L2 {rel:.2e}", flush=True)
    assert worst <= 1.0, f"{name}: gradient outside tolerance ({worst:.3f})"
    ign = (y == ignore_index).numpy()
    assert np.all(got[ign] == 0) and np.all(loss.cpu().numpy()[ign] == 0)
    if x.shape[1] > V:  # columns outside a strided view are untouched
        assert torch.equal(xd[:, :col0].cpu(), x[:, :col0])
        assert torch.equal(xd[:, col0 + V:].cpu(), x[:, col0 + V:])


CASES = [
    # rows, V, dtype, stride
    (7, 5, torch.bfloat16, None),          # tail only (no full 16-byte chunk)
    (33, 1000, torch.bfloat16, None),
    (3, 129, torch.float32, None),         # one tail element after 32 full chunks
    (16, 32000, torch.bfloat16, 32008),    # Llama-2 vocabulary, padded rows
    (9, 32000, torch.float32, None),
    (4, 32768, torch.bfloat16, None),
    (3, 65536, torch.bfloat16, None),      # largest register-resident row
    (2, 65536, torch.float32, None),
    (2, 65537, torch.bfloat16, None),      # smallest streamed row
    (4, 100003, torch.bfloat16, None),     # streamed twice
    (3, 70001, torch.float32, None),       # streamed twice, fp32
    (300, 4099, torch.bfloat16, None),
    (6, 50257, torch.bfloat16, None),      # GPT-2 vocabulary: rows start on every 2-byte offset
    (5, 50257, torch.float32, None),
    (8, 3, torch.bfloat16, 11),            # short rows, head elements only
    (5, 1, torch.bfloat16, None),          # one class: loss 0, gradient 0
    (6, 2, torch.float32, None),           # two classes, rows on 8-byte steps
]


@pytest.mark.parametrize("rows,V,dtype,stride", CASES, ids=[f"{c[0]}x{c[1]}-{str(c[2])[6:]}" for c in CASES])
def test_xent_matches_oracle(rows, V, dtype, stride):
    name = f"xent {rows}x{V} {dtype}"
    banner(name)
    x, y = _case(rows, V, dtype, seed=rows * 1000 + V, row_stride=stride)
    n_valid = int((y != -100).sum())
    _check(name, x, y, V, 1.0 / max(1, n_valid))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("col0", [1, 3])
def test_xent_unaligned_view(dtype, col0):
    """A view starting col0 elements into padded rows: head, aligned body and tail in every row."""
    banner(f"xent view at column {col0} {dtype}")
    x, y = _case(12, 2053, dtype, seed=col0 + 7, row_stride=2064)
    x = x[:, :2064]
    y = torch.where(y == -100, y, y.clamp(max=2052))
    y[2], y[3], y[4] = 0, 2052, 5   # labels in the head, the tail and the first aligned chunk
    _check(f"view@{col0}", x, y, 2053, 0.5, col0=col0)


def test_xent_custom_ignore_index_and_scale():
    banner("xent ignore_index=7, g=-2")
    x, y = _case(20, 513, torch.bfloat16, seed=3, ignore_frac=0.0)
    y[::4] = 7
    _check("custom ignore", x, y, 513, -2.0, ignore_index=7)


def test_xent_bad_label_gives_nan():
    banner("xent bad label")
    x, y = _case(4, 300, torch.float32, seed=4, ignore_frac=0.0)
    y[2] = 300
    xd, yd = x.to(DEV), y.to(DEV)
    loss = torch.empty(4, device=DEV)
    lse = torch.empty(4, device=DEV)
    ea.ea_xent_fwd_bwd(xd, yd, loss, lse, 1.0)
    torch.cuda.synchronize()
    assert torch.isnan(loss[2]) and torch.isnan(xd[2]).all()
    assert torch.isfinite(loss[[0, 1, 3]]).all() and torch.isfinite(xd[[0, 1, 3]]).all()


@pytest.mark.slow
def test_xent_full_size_sampled_rows():
    """The bench workload (65536 rows x 32000, bf16): every row computed, 64 sampled rows checked."""
    rows, V = 65536, 32000
    banner(f"xent full size {rows}x{V}")
    g = torch.Generator(device=DEV).manual_seed(11)
    x = (torch.randn((rows, V), generator=g, device=DEV) * 2.0).to(torch.bfloat16)
    y = torch.randint(0, V, (rows,), generator=g, device=DEV)
    y[::10] = -100
    pick = np.sort(np.random.default_rng(11).choice(rows, 64, replace=False))
    pick[0], pick[-1] = 0, rows - 1
    pick = np.unique(pick)
    xin = x[pick].double().cpu().numpy()
    ycpu = y[pick].cpu().numpy()
    n_valid = int((y != -100).sum())
    ref = xent_fwd_bwd(xin, ycpu, 1.0 / n_valid)
    loss = torch.empty(rows, device=DEV)
    lse = torch.empty(rows, device=DEV)
    ea.ea_xent_fwd_bwd(x, y, loss, lse, 1.0 / n_valid)
    torch.cuda.synchronize()
    idx = torch.from_numpy(pick).to(DEV)
    got = x[idx].double().cpu().numpy()
    np.testing.assert_allclose(lse[idx].double().cpu().numpy(), ref["lse"], atol=2e-4)
    np.testing.assert_allclose(loss[idx].double().cpu().numpy(), ref["loss"], atol=2e-4)
    p = np.exp(xin - ref["lse"][:, None])
    tol = 2.0 ** -8 * np.abs(ref["grad"]) + p * (np.abs(xin) + np.abs(ref["lse"])[:, None]) * 2.0 ** -21 / n_valid
    assert float((np.abs(got - ref["grad"]) / tol).max()) <= 1.0
