"""Host helpers that move a whole sequence to and from the zigzag ranks' local orders (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
import long_context_causal_ea_amd as ea


@pytest.mark.parametrize("W,C", [(1, 5), (2, 3), (3, 7), (4, 4), (8, 3)])
def test_shard_takes_the_rank_positions(W, C):
    S = 2 * W * C
    x = torch.arange(S).view(1, S, 1, 1)
    for r in range(W):
        got = ea.zigzag_shard(x, W, r).flatten().numpy()
        np.testing.assert_array_equal(got, oracle.zigzag_positions(S, W, r))


@pytest.mark.parametrize("W,C", [(1, 5), (2, 3), (3, 7), (8, 3)])
def test_unshard_inverts_shard(W, C):
    S = 2 * W * C
    x = torch.randn(2, S, 3, 4)
    parts = [ea.zigzag_shard(x, W, r) for r in range(W)]
    assert all(p.shape == (2, 2 * C, 3, 4) for p in parts)
    assert torch.equal(ea.zigzag_unshard(parts, W), x)
    # the ring driver's key/value buffer is the ranks' shares side by side
    kv = torch.cat(parts, dim=1)
    pos = np.concatenate([oracle.zigzag_positions(S, W, s) for s in range(W)])
    np.testing.assert_array_equal(kv[0, :, 0, 0].numpy(), x[0, pos, 0, 0].numpy())


def test_unshard_needs_every_rank():
    with pytest.raises(ValueError):
        ea.zigzag_unshard([torch.zeros(1, 4, 1, 1)], 2)


def test_ulysses_shard_round_trip():
    x = torch.randn(2, 10, 8, 4)
    parts = [ea.ulysses_shard(x, 4, r) for r in range(4)]
    assert all(p.shape == (2, 10, 2, 4) and p.is_contiguous() for p in parts)
    assert torch.equal(parts[3], x[:, :, 6:8])
    assert torch.equal(ea.ulysses_unshard(parts), x)
    with pytest.raises(ValueError):
        ea.ulysses_shard(x, 3, 0)
