"""Oracle: global token positions of one rank's share in a zigzag ring.

Reading (the pages only name the zigzag ring mode and say it interleaves tokens
across ranks -- EasyContext training-script walkthrough, mlqm.cn, section on
parallel strategies; each rank then runs its model on local ids carrying the
rank's position ids -- cn486.com page, usage code): a sequence of S_total tokens
is cut into 2*W equal chunks of C tokens; rank r holds chunk r followed by chunk
2W-1-r.  Pairing an early chunk with a late one gives every rank the same number
of causal (query, key) pairs.  Parity unpinned as to the layout itself (no page
prints it); the tests pin the properties any such layout must have: a bijection
onto 0..S_total-1 and the balanced pair count.

Ring order reading: at step t rank r holds the key/value share of rank
(r - t) mod W.
"""
import numpy as np


def chunk_positions(chunk: int, C: int) -> np.ndarray:
    return chunk * C + np.arange(C, dtype=np.int64)


def zigzag_positions(s_total: int, world: int, rank: int) -> np.ndarray:
    if world < 1 or not (0 <= rank < world):
        raise ValueError("bad world/rank")
    if s_total % (2 * world) != 0:
        raise ValueError("s_total must be a multiple of 2*world")
    C = s_total // (2 * world)
    return np.concatenate([chunk_positions(rank, C), chunk_positions(2 * world - 1 - rank, C)])


def ring_source(rank: int, step: int, world: int) -> int:
    return (rank - step) % world
