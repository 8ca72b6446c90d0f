"""A whole step recorded as a HIP graph (``capture_step``) against the same step run eagerly, with and without
the rotary embedding fused into the attention calls, dense and ring.

Each replay follows eager work of the program's own (an eager step of a second driver on the same inputs, and
new inputs copied in place) with synchronisations in between, and every replay must reproduce the eager results
bit for bit: the kernels use no atomics, so the same launches on the same inputs give the same bits.
"""
import pytest
import torch

import long_context_causal_ea_amd as ea
import synth
from tests.parity import banner

pytestmark = pytest.mark.gpu
DEV = "cuda"
OUTS = ("o", "lse", "dq", "dk", "dv")


def _draw(shape, seed):
    return synth.normal_draw(shape, seed, 1.0, DEV).to(torch.bfloat16)


def _replays_match(make, inputs, reseed, n=3):
    drv, ref = make(), make()
    graph = ea.capture_step(drv, inputs["do"])
    torch.cuda.synchronize()
    for i in range(n):
        for j, (name, x) in enumerate(inputs.items()):
            x.copy_(_draw(x.shape, reseed + 10 * i + j))
        ref.step(inputs["do"])
        torch.cuda.synchronize()
        for name in OUTS:  # stale values a skipped launch would leave behind
            getattr(drv, name).fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name in OUTS:
            assert torch.equal(getattr(drv, name), getattr(ref, name)), (i, name)


@pytest.mark.parametrize("rope", [None, 1e6])
def test_dense_step_graph(rope):
    B, S, H, D = 1, 700, 4, 128
    banner(f"graph DenseCausal S={S} H={H} rope={rope}")
    inputs = {n: _draw((B, S, H, D), 300 + i) for i, n in enumerate(("q", "k", "v", "do"))}
    _replays_match(lambda: ea.DenseCausal(inputs["q"], inputs["k"], inputs["v"], rope_theta=rope), inputs, 400)


@pytest.mark.parametrize("rope", [None, 1e6])
def test_ring_step_graph(rope):
    W, C, H, D, rank = 4, 40, 2, 64, 2
    banner(f"graph ZigzagRingRank W={W} C={C} rank={rank} rope={rope}")
    inputs = {"q": _draw((1, 2 * C, H, D), 500), "k": _draw((1, 2 * W * C, H, D), 501),
              "v": _draw((1, 2 * W * C, H, D), 502), "do": _draw((1, 2 * C, H, D), 503)}
    _replays_match(lambda: ea.ZigzagRingRank(inputs["q"], inputs["k"], inputs["v"], W, rank, rope_theta=rope),
                   inputs, 600)
