"""Host-side drivers of the attention path on one GPU (no collectives).

``ZigzagRingRank`` runs one rank's share of a zigzag ring attention layer:
the ring visits every rank's key/value share in turn (EasyContext
core-technology page, hotelren.com, section 1 "sequence parallelism"), with
tokens interleaved across ranks (mlqm.cn training-script walkthrough, zigzag
mode).  Here the W key/value shares sit side by side in one buffer, so the
ring's send/receive is a pointer offset; every step is an ``ea_attn_fwd`` /
``ea_attn_bwd`` call and the per-step partial results are combined with
``ea_lse_merge``.  Positions come from ``ea_zigzag_segments``, and the causal
rule on global positions selects, per step, the full, causal or half blocks.

``DenseCausal`` is the whole-sequence case: one forward and one backward
call over positions 0..S-1.

With ``rope_theta`` set, both drivers take unrotated Q and K.  The forward
rotates K by its global positions (``ea_rope`` into a buffer the driver owns)
and hands Q unrotated to ``ea_attn_fwd_rope``, which turns each query row in
registers and writes the turned rows once for the backward; the backward
(``ea_attn_bwd_rope``) turns each dQ and dK contribution back before adding it,
so the gradients are with respect to the unrotated inputs and no separate
rotation pass over Q, dQ or dK is needed.

All buffers are allocated when the driver is built; ``forward`` and
``backward`` enqueue work on the given stream (default: the current one) and
allocate nothing, so a whole step can be recorded as a HIP graph
(``capture_step``), alone or inside a caller's larger captured training step.

``ulysses_shard`` / ``ulysses_unshard`` do the same for the head split of the
Ulysses mode (mlqm.cn walkthrough, parallel modes): after its all-to-all a rank
holds every token of H / world heads, and its attention is one ``DenseCausal``
over them.

``zigzag_shard`` / ``zigzag_unshard`` move a whole sequence to and from the
ranks' local orders (the input preparation that hands each rank its share with
its positions, cn486.com page, usage code); they are plain tensor copies along
the sequence axis, laid out by ``ea_zigzag_segments``.
"""
import torch

from . import _lib as L


def zigzag_shard(x, world: int, rank: int, dim: int = 1):
    """The rows of x (whole sequence along `dim`) that rank `rank` of a `world`-rank zigzag ring holds, in its
    local order (a copy)."""
    s_total = x.shape[dim]
    seg = L.ea_zigzag_segments(s_total, world, rank)
    parts = [x.narrow(dim, seg[i], seg[i + 1]) for i in range(0, len(seg), 2) if seg[i + 1] > 0]
    return torch.cat(parts, dim=dim)


def ulysses_shard(x, world: int, rank: int, dim: int = 2):
    """The heads of x ([B, S, H, D], whole sequence) that rank `rank` of a `world`-way Ulysses split holds after
    the sequence-to-head all-to-all: heads [rank * H / world, (rank + 1) * H / world), every token (a copy)."""
    H = x.shape[dim]
    if H % world:
        raise ValueError("the head count must be a multiple of the world size")
    hw = H // world
    return x.narrow(dim, rank * hw, hw).contiguous()


def ulysses_unshard(parts, dim: int = 2):
    """Inverse of `ulysses_shard` (the head-to-sequence all-to-all gathered on one device)."""
    return torch.cat(list(parts), dim=dim)


def zigzag_unshard(parts, world: int, dim: int = 1):
    """Inverse of `zigzag_shard`: the whole sequence from the `world` ranks' local tensors (rank order)."""
    if len(parts) != world:
        raise ValueError("one local tensor per rank")
    local = parts[0].shape[dim]
    s_total = local * world
    shape = list(parts[0].shape)
    shape[dim] = s_total
    out = parts[0].new_empty(shape)
    for r, x in enumerate(parts):
        seg = L.ea_zigzag_segments(s_total, world, r)
        off = 0
        for i in range(0, len(seg), 2):
            out.narrow(dim, seg[i], seg[i + 1]).copy_(x.narrow(dim, off, seg[i + 1]))
            off += seg[i + 1]
    return out


def _zero(stream, *ts):
    """Zero fp32 accumulators on the stream the library calls use (torch's fill kernel, no memset)."""
    if stream is None:
        for t in ts:
            t.zero_()
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(int(stream))
    with torch.cuda.stream(s):
        for t in ts:
            t.zero_()


def capture_step(driver, do):
    """Record one whole ``driver.step(do)`` (rotations, forward, merges, zeroing, backward) as a HIP graph.

    Returns a ``torch.cuda.CUDAGraph``; ``replay()`` reruns every launch of the step on the current stream.  The
    graph holds the driver's buffers and ``do`` by address: to run on new inputs, copy them into the same tensors
    (the driver's inputs and ``do``) before replaying.  Nothing in the step allocates or clears memory with a
    memset, so the recorded step is the eager one launch for launch."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        driver.step(do)
    return g


class DenseCausal:
    """Dense (whole-sequence) attention of one GPU: forward, then backward into fp32 gradients."""

    def __init__(self, q, k, v, causal=True, scale=None, o_dtype=torch.float32, rope_theta=None):
        B, S, H, D = q.shape
        self.rope_theta = rope_theta
        self.q_in, self.k_in = q, k
        if rope_theta is None:
            self.q, self.k = q, k
        else:  # rotated copies, refreshed by every forward
            self.q, self.k = torch.empty_like(q), torch.empty_like(k)
        self.v = v
        self.causal = causal
        self.scale = D ** -0.5 if scale is None else scale
        dev = q.device
        self.o = torch.empty((B, S, H, D), dtype=o_dtype, device=dev)
        self.lse = torch.empty((B, S, H), dtype=torch.float32, device=dev)
        self.delta = torch.empty((B, S, H), dtype=torch.float32, device=dev)
        self.dq = torch.empty((B, S, H, D), dtype=torch.float32, device=dev)
        self.dk = torch.empty((B, k.shape[1], H, D), dtype=torch.float32, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.q_seg = [0, S]
        self.k_seg = [0, k.shape[1]]

    def forward(self, stream=None):
        if self.rope_theta is None:
            L.ea_attn_fwd(self.q, self.k, self.v, self.o, self.lse, self.q_seg, self.k_seg, self.causal, self.scale,
                          stream)
            return
        L.ea_rope(self.k_in, self.k, self.k_seg, self.rope_theta, stream=stream)
        L.ea_attn_fwd_rope(self.q_in, self.k, self.v, self.o, self.lse, self.q_seg, self.k_seg, self.rope_theta,
                           q_rot=self.q, causal=self.causal, scale=self.scale, stream=stream)

    def backward(self, do, stream=None):
        _zero(stream, self.dq, self.dk, self.dv)
        args = (self.q, self.k, self.v, self.o, do, self.lse, self.delta, self.dq, self.dk, self.dv, self.q_seg,
                self.k_seg)
        if self.rope_theta is None:
            L.ea_attn_bwd(*args, self.causal, self.scale, delta_ready=False, stream=stream)
        else:
            L.ea_attn_bwd_rope(*args, self.rope_theta, self.causal, self.scale, delta_ready=False, stream=stream)

    def step(self, do, stream=None):
        self.forward(stream)
        self.backward(do, stream)


class ZigzagRingRank:
    """One rank of a W-rank zigzag ring.

    q, do: [B, 2C, H, D] bf16, the rank's local rows (chunk r then chunk 2W-1-r).
    k, v:  [B, W*2C, H, D] bf16, the W ranks' shares side by side: rows
           [2C*s, 2C*(s+1)) are rank s's local keys/values.
    fused_merge: steps after the first merge their partial result into (o, lse)
           inside the forward launch (``ea_attn_fwd_merge``); False writes each
           partial to its own buffers and merges it with ``ea_lse_merge``.
    """

    def __init__(self, q, k, v, world, rank, scale=None, rope_theta=None, fused_merge=True):
        B, sq, H, D = q.shape
        if sq % 2 or k.shape[1] != world * sq:
            raise ValueError("q must hold 2C rows and k/v W*2C rows")
        self.rope_theta = rope_theta
        self.q_in, self.k_in = q, k
        if rope_theta is None:
            self.q, self.k = q, k
        else:
            self.q, self.k = torch.empty_like(q), torch.empty_like(k)
        self.v = v
        self.W, self.r = world, rank
        self.C = sq // 2
        self.s_total = world * sq
        self.scale = D ** -0.5 if scale is None else scale
        dev = q.device
        self.o = torch.empty((B, sq, H, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, sq, H), dtype=torch.float32, device=dev)
        self.fused_merge = fused_merge
        if not fused_merge:
            self.o_part = torch.empty_like(self.o)
            self.lse_part = torch.empty_like(self.lse)
        self.delta = torch.empty_like(self.lse)
        self.dq = torch.empty_like(self.o)
        self.dk = torch.empty((B, k.shape[1], H, D), dtype=torch.float32, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.q_seg = L.ea_zigzag_segments(self.s_total, world, rank)
        self.sources = [L.ea_ring_source(rank, t, world) for t in range(world)]
        self.k_segs = [L.ea_zigzag_segments(self.s_total, world, s) for s in self.sources]
        self.share_segs = [L.ea_zigzag_segments(self.s_total, world, s) for s in range(world)]

    def _share(self, s, x):
        return x[:, 2 * self.C * s: 2 * self.C * (s + 1)]

    def _block(self, t, x):
        s = self.sources[t]
        return x[:, 2 * self.C * s: 2 * self.C * (s + 1)]

    def _fwd(self, t, kb, vb, o, lse, merge, stream):
        """One ring step's forward: a partial into (o, lse), or merged into that accumulator."""
        if self.rope_theta is not None:
            # q turned in the kernel; the turned rows are written once, at the first step
            L.ea_attn_fwd_rope(self.q_in, kb, vb, o, lse, self.q_seg, self.k_segs[t], self.rope_theta,
                               q_rot=self.q if t == 0 else None, merge=merge, causal=True, scale=self.scale,
                               stream=stream)
        elif merge:
            L.ea_attn_fwd_merge(self.q, kb, vb, o, lse, self.q_seg, self.k_segs[t], True, self.scale, stream)
        else:
            L.ea_attn_fwd(self.q, kb, vb, o, lse, self.q_seg, self.k_segs[t], True, self.scale, stream)

    def forward(self, stream=None):
        if self.rope_theta is not None:
            # each rank's share carries that rank's zigzag positions
            for s in range(self.W):
                L.ea_rope(self._share(s, self.k_in), self._share(s, self.k), self.share_segs[s], self.rope_theta,
                          stream=stream)
        for t in range(self.W):
            kb, vb = self._block(t, self.k), self._block(t, self.v)
            if t == 0:
                self._fwd(t, kb, vb, self.o, self.lse, False, stream)
            elif self.fused_merge:
                self._fwd(t, kb, vb, self.o, self.lse, True, stream)
            else:
                self._fwd(t, kb, vb, self.o_part, self.lse_part, False, stream)
                L.ea_lse_merge(self.o, self.lse, self.o_part, self.lse_part, stream)

    def backward(self, do, stream=None):
        _zero(stream, self.dq, self.dk, self.dv)
        for t in range(self.W):
            kb, vb = self._block(t, self.k), self._block(t, self.v)
            args = (self.q, kb, vb, self.o, do, self.lse, self.delta, self.dq, self._block(t, self.dk),
                    self._block(t, self.dv), self.q_seg, self.k_segs[t])
            if self.rope_theta is None:
                L.ea_attn_bwd(*args, True, self.scale, delta_ready=(t > 0), stream=stream)
            else:
                L.ea_attn_bwd_rope(*args, self.rope_theta, True, self.scale, delta_ready=(t > 0), stream=stream)

    def step(self, do, stream=None):
        self.forward(stream)
        self.backward(do, stream)
