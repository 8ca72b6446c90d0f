"""Workload table: shapes, seeds and value distributions of the synthetic inputs.

The shapes follow the attention shapes of the models the EasyContext pages train
(Llama-2-7B: 32 heads of 128; Llama-2-13B: 40 heads of 128) and the sequence
lengths they report (32K training script, 512K and 700K ring training).  The
pages measure on a text dataset; seeded Gaussian tensors of the same shapes
stand in for it.

Nothing here computes positions or masks: a ring workload is described by
(ranks, chunk length, rank) and each side derives positions with its own code.
"""
from dataclasses import dataclass
from typing import Optional


@dataclass(frozen=True)
class Config:
    name: str
    kind: str                 # "dense" (one causal call over positions 0..S-1) or "ring"
    B: int
    H: int
    D: int
    S: int = 0                # dense: sequence length
    W: int = 0                # ring: number of ranks
    C: int = 0                # ring: chunk length (the sequence is 2*W chunks)
    rank: int = 0             # ring: which rank's share is computed
    std: float = 1.0          # standard deviation of the Gaussian draws
    rope_theta: Optional[float] = None   # rotary base the attention step applies to Q and K (None: no rotation)
    seed: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / (self.D ** 0.5)

    @property
    def s_total(self) -> int:
        return self.S if self.kind == "dense" else 2 * self.W * self.C

    @property
    def sq(self) -> int:
        """Local query rows."""
        return self.S if self.kind == "dense" else 2 * self.C

    @property
    def sk(self) -> int:
        """All keys the local queries are checked against."""
        return self.s_total

    def causal_pairs_per_head(self) -> int:
        """Allowed (query, key) pairs per head; closed forms, used for FLOP counts."""
        if self.kind == "dense":
            return self.S * (self.S + 1) // 2
        return 2 * self.W * self.C * self.C + self.C

    def flops(self) -> dict:
        """Algorithmic FLOPs: 4*D per allowed pair forward, 10*D backward."""
        n = self.causal_pairs_per_head() * self.B * self.H
        return {"fwd": 4 * self.D * n, "bwd": 10 * self.D * n, "total": 14 * self.D * n}


CONFIGS = {
    "c1": Config("causal-b1-h2-d64-s512", "dense", B=1, H=2, D=64, S=512, seed=1001),
    "c2": Config("causal-b1-h32-d128-s32768-rope1e6", "dense", B=1, H=32, D=128, S=32768,
                 rope_theta=1e6, seed=1002),
    "c3": Config("zigzag-ring-512k-w8-rank3-h32-d128", "ring", B=1, H=32, D=128, W=8, C=32768,
                 rank=3, seed=1003),
    "c4": Config("zigzag-ring-700k-w8-rank3-h32-d128", "ring", B=1, H=32, D=128, W=8, C=43750,
                 rank=3, seed=1004),
    "c5": Config("causal-b1-h40-d128-s131072-std0.5-rope1e9", "dense", B=1, H=40, D=128,
                 S=131072, std=0.5, rope_theta=1e9, seed=1005),
    "t": Config("causal-b1-h32-d128-s65536-rope1e6", "dense", B=1, H=32, D=128, S=65536,
                rope_theta=1e6, seed=1006),
    # one GPU's share of an 8-way Ulysses split of the 512K-token Llama-2-7B attention: after the
    # sequence-to-head all-to-all a GPU holds every token of 32 / 8 = 4 heads
    "u3": Config("ulysses-512k-w8-h4-d128", "dense", B=1, H=4, D=128, S=524288, seed=1007),
}


def get(key: str) -> Config:
    return CONFIGS[key.lower()]
