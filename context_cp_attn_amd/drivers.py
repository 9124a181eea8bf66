"""P context-parallel ranks simulated on one GPU: the ring and Ulysses shares.

Host-side sequencing only; every step is a libcp_attn kernel.

Ring (handbook "Context parallelism: Ring Attention and Ulysses", §"Ring
Attention"): rank r keeps its queries; at step s it holds the KV block of rank
src = (r - s) mod P, attends to it at the block's global positions and merges the
partial (out, lse) into its running result.  On one GPU the block "arriving" from
the left neighbour is a view of block src.  With the zigzag partition (§"The zigzag
partition") the inputs are first reordered so that rank r's share is the contiguous
slice r of the reordered sequence, holding chunks r and 2P-1-r.

Ulysses (§"Ulysses"): the sequence -> head relayout gives each rank the whole
sequence for H/P heads; attention runs per rank; the inverse relayout returns the
output to sequence order.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib, ops


LAYOUT_OF_STRATEGY = {ops.DUAL_CHUNK_SWAP: "zigzag", ops.STRIPED: "striped"}


def auto_strategy(packed: bool) -> int:
    """Reorder strategy chosen from the packing configuration.  The MaxText packing
    PR ("Add Packing Support for Context Parallelism (Ring Attention)",
    §Description) says only that the choice follows the packing configuration, not
    which strategy each configuration gets; the reading here is striped for packed
    sequences and dual-chunk-swap otherwise.  It is a policy, not a result: both
    strategies give the same attention.  Under packing, dual-chunk-swap leaves the
    ranks unequal (on the packed 8K workload of these kernels the heaviest rank holds
    1.5x the mean of the visible pairs) while striped gives every rank the same
    share; there the two tie on the slowest rank's time, which is what a step on P
    GPUs takes, and dual-chunk-swap is faster only summed over the ranks."""
    return ops.STRIPED if packed else ops.DUAL_CHUNK_SWAP


def padded_length(S: int, multiple: int) -> int:
    return -(-S // multiple) * multiple


def pad_sequence(x, multiple: int):
    """Pad x [B][S][...] at its end with zero rows to a multiple of ``multiple`` (the
    CP degree, or 2P for the zigzag chunks).  Pad tokens take positions S, S+1, ...;
    under a causal mask no real query sees them.  Returns (x_padded, S)."""
    S = x.shape[1]
    return ops.pad_rows(x, padded_length(S, multiple)), S


def pad_segments(seg, multiple: int, pad_id: int | None = None):
    """Pad int32 segment ids [B][S] to a multiple, the pad tokens in a segment of
    their own, so that no real query sees a pad key without a causal mask either.

    Segment ids must never decrease along a row (the attention kernels classify
    whole tiles from their first and last ids), so the pad segment, which comes
    last, needs an id above every real one: ``pad_id`` defaults to the largest id
    + 1 (one device-to-host read), and a given ``pad_id`` that is not above every
    real id raises ValueError."""
    top = int(seg.max().item())
    if pad_id is None:
        pad_id = top + 1
    elif pad_id <= top:
        raise ValueError(f"pad_id {pad_id} must exceed every real segment id (largest {top}): "
                         "segment ids may not decrease along the sequence")
    return ops.pad_rows(seg, padded_length(seg.shape[1], multiple), fill=pad_id)


def rank_positions(rank: int, P: int, S: int, layout: str = "zigzag", device="cuda") -> torch.Tensor:
    """int32 global positions of the tokens rank ``rank`` holds (increasing)."""
    if layout == "striped":
        if S % P:
            raise ValueError(f"sequence {S} not divisible by {P} ranks")
        return torch.arange(rank, S, P, dtype=torch.int32).to(device)
    if S % (2 * P):
        raise ValueError(f"sequence {S} not divisible into {2 * P} chunks")
    c = S // (2 * P)
    if layout == "zigzag":
        chunks = (rank, 2 * P - 1 - rank)
    elif layout == "contiguous":
        chunks = (2 * rank, 2 * rank + 1)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    pos = torch.cat([torch.arange(ch * c, (ch + 1) * c, dtype=torch.int32) for ch in chunks])
    return pos.to(device)


def _block(t, r, C):
    return None if t is None else t[:, r * C:(r + 1) * C]


class RingShare:
    """One rank's ring pass over P KV blocks, forward and backward.

    q, k, v, seg are the whole tensors in the partition's order: for ``zigzag`` /
    ``striped`` the output of ``ops.zigzag_reorder`` with that strategy; for
    ``contiguous`` the sequence order.  Rank
    r's rows (queries and its own KV block) are slice r of length S/P.
    """

    def __init__(self, q, k, v, P: int, rank: int, layout="zigzag", seg=None, causal=True,
                 window=0, scale=0.0, fused=None):
        self.q, self.k, self.v, self.seg = q, k, v, seg
        self.P, self.rank, self.layout = P, rank, layout
        # True: the merge inside the attention epilogue; False: attn_fwd + lse_merge;
        # None: the fused step unless the forward splits the block's keys over two
        # workgroups (small grids of long blocks), which only the unfused pair can use
        self.fused = fused
        self.S = q.shape[1]
        self.C = self.S // P
        self.mask = dict(causal=causal, window=window, scale=scale)
        self.pos = [rank_positions(r, P, self.S, layout, q.device) for r in range(P)]
        self.ws = None
        self._steps = None   # per-step C-ABI arguments of the pass, built on first use

    def _skip(self, src):
        # A contiguous causal block later than the rank's own sees nothing; the
        # handbook's loop skips it too.  Zigzag blocks always hold visible pairs.
        return self.layout == "contiguous" and self.mask["causal"] and src > self.rank

    def _mask(self, src):
        r, C = self.rank, self.C
        m = dict(self.mask, q_pos=self.pos[r], k_pos=self.pos[src])
        if self.seg is not None:
            m.update(q_seg=_block(self.seg, r, C).contiguous(), k_seg=_block(self.seg, src, C).contiguous())
        return m

    def _step_args(self, ql):
        """Per step of the pass: the validated argument struct, the key / value block
        pointers and the source block, built once (every array they point to is held
        here), so that a forward or backward pass costs its P library calls and no
        per-step host work."""
        if self._steps is None:
            steps = []
            for step in range(self.P):
                src = (self.rank - step) % self.P
                if self._skip(src):
                    continue
                kb, vb = _block(self.k, src, self.C), _block(self.v, src, self.C)
                m = self._mask(src)
                ops._check_qkv(ql, kb, vb)
                steps.append((ops.make_args(ql, kb, **m), kb.data_ptr(), vb.data_ptr(), src, m))
            self._steps = steps
        return self._steps

    def forward(self):
        """(out [B,S/P,Hq,D] float32, lse [B,Hq,S/P]) of this rank after P steps."""
        r, C, P = self.rank, self.C, self.P
        ql = _block(self.q, r, C)
        B, _, Hq, D = ql.shape
        acc = torch.zeros(B, C, Hq, D, device=ql.device, dtype=torch.float32)
        lse = torch.full((B, Hq, C), float("-inf"), device=ql.device, dtype=torch.float32)
        fused, ws = self.fused, False
        if fused is None:
            ws = split_workspace(ql, _block(self.k, r, C), **self._mask(r))
            fused = ws is False
        if fused and not ops.DEBUG:
            lib, stream = _lib.load(), ops._stream()
            qp, ap, lp = ql.data_ptr(), acc.data_ptr(), lse.data_ptr()
            for a, kp, vp, _, _ in self._step_args(ql):
                _lib.check(lib.cp_attn_fwd_merge(ctypes.byref(a), qp, kp, vp, ap, lp, stream))
            return acc, lse
        if not fused:
            blk_o = torch.empty(B, C, Hq, D, device=ql.device, dtype=ql.dtype)
            blk_l = torch.empty(B, Hq, C, device=ql.device, dtype=torch.float32)
        for step in range(P):
            src = (r - step) % P
            if self._skip(src):
                continue
            kb, vb = _block(self.k, src, C), _block(self.v, src, C)
            if fused:
                ops.attn_fwd_merge(ql, kb, vb, acc, lse, **self._mask(src))
            else:
                ops.attn_fwd(ql, kb, vb, out=blk_o, lse=blk_l, workspace=None if ws is False else ws,
                             **self._mask(src))
                ops.lse_merge(acc, lse, blk_o, blk_l)
        return acc, lse

    def forward_graph(self):
        """This rank's ring forward captured as one HIP graph, for passes whose steps
        are short enough that launching them costs time: returns (replay, out, lse).
        ``replay()`` enqueues the whole pass on the current stream and leaves its
        result in ``out`` / ``lse``, buffers owned by the graph; it reads the share's
        q, k, v tensors at replay time.  One eager pass on a side stream runs first
        (it fills the share's cached launch arguments, which capture must not create).
        Not with CP_ATTN_DEBUG, whose checks synchronise the stream."""
        if ops.DEBUG:
            raise RuntimeError("forward_graph: the CP_ATTN_DEBUG checks cannot run under graph capture")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self.forward()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            out, lse = self.forward()
        return graph.replay, out, lse

    def backward(self, out, lse, dout, dq, dk, dv):
        """Accumulate this rank's gradients: dq [B,S/P,..] of its queries, and the
        partial dk/dv of every block into the whole-sequence dk/dv buffers."""
        r, C, P = self.rank, self.C, self.P
        ql = _block(self.q, r, C)
        # every step uses the rows' same out, lse and dout: the first call derives the
        # per-row values into the workspace, the later ones reuse them
        ws = ops.bwd_workspace(ql, _block(self.k, r, C), **self._mask(r))
        if not ops.DEBUG and ql.shape[0] == 1:
            # the pass's cached arguments; the buffers are checked once per call
            B, _, Hq, D = ql.shape
            for t, n, dt in ((out, "out", ql.dtype), (dout, "dout", ql.dtype), (dq, "dq", torch.float32),
                             (lse, "lse", torch.float32), (dk, "dk", torch.float32), (dv, "dv", torch.float32)):
                ops._dev(t, n, dt)
            if out.shape != ql.shape or dout.shape != ql.shape or dq.shape != ql.shape or \
                    lse.shape != (B, Hq, C) or dk.shape != self.k.shape or dv.shape != self.v.shape:
                raise ValueError("backward buffers do not match the rank's shapes")
            lib, stream = _lib.load(), ops._stream()
            blk = C * self.k.shape[2] * D * 4   # bytes of one rank's block of dk / dv
            fn = lib.cp_attn_bwd
            for a, kp, vp, src, _ in self._step_args(ql):
                _lib.check(fn(ctypes.byref(a), ql.data_ptr(), kp, vp, out.data_ptr(), lse.data_ptr(),
                              dout.data_ptr(), dq.data_ptr(), dk.data_ptr() + src * blk, dv.data_ptr() + src * blk,
                              1, ws.data_ptr(), ws.numel(), stream))
                fn = lib.cp_attn_bwd_rows_ready
            return dq, dk, dv
        ready = False
        for step in range(P):
            src = (r - step) % P
            if self._skip(src):
                continue
            ops.attn_bwd(ql, _block(self.k, src, C), _block(self.v, src, C), out, lse, dout,
                         dq=dq, dk=_block(dk, src, C), dv=_block(dv, src, C), accumulate=True,
                         workspace=ws, rows_ready=ready, **self._mask(src))
            ready = True
        return dq, dk, dv


def split_workspace(q, k, **mask):
    """The forward's workspace when it splits each query tile's keys over two
    workgroups for this block shape (the size does not depend on positions or
    segment ids), else False."""
    ws = ops.fwd_workspace(q, k, **mask)
    return False if ws is None else ws


def ring_forward_all(q, k, v, P, layout="zigzag", seg=None, **mask):
    """Every rank's ring forward; returns per-rank (out fp32, lse).  mask may hold
    ``fused`` (default None: the fused step unless the forward's key split applies)."""
    return [RingShare(q, k, v, P, r, layout, seg, **mask).forward() for r in range(P)]


def _kv_relayout(x_stack, P, kv_rep):
    if kv_rep == 1:
        return ops.ulysses_relayout(x_stack, P)
    return ops.ulysses_relayout_ex(x_stack.unsqueeze(0), P, rep=kv_rep)[0]


def ulysses_forward(q_stack, k_stack, v_stack, P, kv_rep=1, **mask):
    """q_stack [P][B][S/P][Hq][D], k/v [P][B][S/P][Hkv][D] (rank s holds sequence slice s).

    Returns (out_stack [P][B][S/P][Hq][D], lse [P][B][Hq/P][S], the relayouted q, k, v
    and per-rank outputs): rank p attends over the whole sequence with q heads
    [p*Hq/P, (p+1)*Hq/P).  kv_rep > 1 replicates every kv head by group before the
    exchange, for a degree up to Hkv * kv_rep.
    """
    ql = ops.ulysses_relayout(q_stack, P)
    kl = _kv_relayout(k_stack, P, kv_rep)
    vl = _kv_relayout(v_stack, P, kv_rep)
    outs, lses = [], []
    for p in range(P):
        o, l = ops.attn_fwd(ql[p], kl[p], vl[p], **mask)
        outs.append(o)
        lses.append(l)
    out_l = torch.stack(outs)
    return ops.ulysses_relayout_inv(out_l, P), torch.stack(lses), (ql, kl, vl, out_l)


def ulysses_backward(relayouted, lse, dout_stack, P, kv_rep=1, **mask):
    """Gradients through Ulysses, from ``ulysses_forward``'s relayouted tensors and lse.

    Returns (dq, dk, dv) stacks [P][B][S/P][H][D] float32 in the sequence-sharded
    layout; with kv_rep > 1 each kv head's gradient is the sum over its copies.
    """
    ql, kl, vl, out_l = relayouted
    gl = ops.ulysses_relayout(dout_stack, P)
    ws = ops.bwd_workspace(ql[0], kl[0], **mask)
    grads = [ops.attn_bwd(ql[p], kl[p], vl[p], out_l[p], lse[p], gl[p], workspace=ws, **mask) for p in range(P)]
    dql, dkl, dvl = (torch.stack([g[i] for g in grads]) for i in range(3))
    dq = ops.ulysses_relayout_inv(dql, P)
    if kv_rep == 1:
        return dq, ops.ulysses_relayout_inv(dkl, P), ops.ulysses_relayout_inv(dvl, P)
    inv = lambda t: ops.ulysses_relayout_ex(t.unsqueeze(0), P, rep=kv_rep, inverse=True)[0]
    return dq, inv(dkl), inv(dvl)


class UlyssesStep:
    """One Ulysses forward + backward pass of all P ranks with every buffer
    allocated once, so that repeated passes allocate nothing.

    qkv_stack [3][P][B][S/P][H][D] bf16 holds q, k and v in one buffer (rank s holds
    sequence slice s, all heads; MHA, so the three have the same shape), dout_stack
    [P][B][S/P][H][D].  ``run`` relayouts q, k and v to [3][P][B][S][H/P][D] in one
    launch (three groups of the general relayout), runs rank p's attention forward on
    its H/P heads over the whole sequence, returns the output to the sequence layout
    (``out``), relayouts dout, runs every rank's backward into one [3][P][B][S][H/P][D]
    float32 buffer and returns dq, dk, dv to the sequence layout in one launch
    (``dqkv`` [3][P][B][S/P][H][D]).  ``lse`` [P][B][H/P][S] keeps each rank's row
    log-sum-exp.  The same sequence of calls as ``ulysses_forward`` +
    ``ulysses_backward``, with the buffers reused and q / k / v exchanged together.
    """

    def __init__(self, qkv_stack, dout_stack, P: int, **mask):
        if qkv_stack.dim() != 6 or qkv_stack.shape[0] != 3:
            raise ValueError("qkv_stack must be [3][P][B][S/P][H][D]")
        _, P_, B, Sl, H, D = qkv_stack.shape
        if P_ != P or H % P:
            raise ValueError(f"stack of {P_} ranks and {H} heads for degree {P}")
        if tuple(dout_stack.shape) != tuple(qkv_stack.shape[1:]):
            raise ValueError("dout_stack must be shaped like q")
        self.P, self.mask = P, mask
        self.qkv, self.dout_stack = qkv_stack, dout_stack
        dev, bf, f32 = qkv_stack.device, qkv_stack.dtype, torch.float32
        S = Sl * P
        sh = (P, B, S, H // P, D)
        self.qkvl = torch.empty((3,) + sh, device=dev, dtype=bf)
        self.gl, self.ol = (torch.empty(sh, device=dev, dtype=bf) for _ in range(2))
        self.lse = torch.empty(P, B, H // P, S, device=dev, dtype=f32)
        self.out = torch.empty(dout_stack.shape, device=dev, dtype=bf)
        self.dqkvl = torch.empty((3,) + sh, device=dev, dtype=f32)
        self.dqkv = torch.empty(qkv_stack.shape, device=dev, dtype=f32)
        ql, kl = self.qkvl[0, 0], self.qkvl[1, 0]
        self.ws = ops.bwd_workspace(ql, kl, **mask)
        self.fws = ops.fwd_workspace(ql, kl, **mask)   # None when the forward does not split

    def forward(self):
        P, (ql, kl, vl) = self.P, self.qkvl
        ops.ulysses_relayout_ex(self.qkv, P, groups=3, out=self.qkvl)
        for p in range(P):
            ops.attn_fwd(ql[p], kl[p], vl[p], out=self.ol[p], lse=self.lse[p], workspace=self.fws, **self.mask)
        ops.ulysses_relayout_inv(self.ol, P, out=self.out)

    def backward(self):
        P, (ql, kl, vl), (dql, dkl, dvl) = self.P, self.qkvl, self.dqkvl
        ops.ulysses_relayout(self.dout_stack, P, out=self.gl)
        for p in range(P):
            ops.attn_bwd(ql[p], kl[p], vl[p], self.ol[p], self.lse[p], self.gl[p],
                         dq=dql[p], dk=dkl[p], dv=dvl[p], workspace=self.ws, **self.mask)
        ops.ulysses_relayout_ex(self.dqkvl, P, groups=3, inverse=True, out=self.dqkv)

    def run(self):
        self.forward()
        self.backward()


def usp_forward(q, k, v, Pr, Pu, kv_rep=1, seg=None, causal=True, window=0, scale=0.0, keep=False):
    """Ulysses within groups of Pu ranks x ring attention across Pr groups, all
    Pr*Pu ranks on one GPU.  q [1,S,Hq,D], k/v [1,S,Hkv,D] in sequence order.

    The sequence is zigzag-reordered for the Pr groups; group r's share is split
    contiguously over its Pu ranks and exchanged inside the group (heads slice u to
    rank (r, u)); rank (r, u) then runs the ring over the groups' blocks of its head
    slice with the fused step (or attn_fwd + lse_merge where the forward splits the
    blocks' keys over two workgroups).  Returns (out [1,S,Hq,D] float32 in sequence order,
    lse [Pr][Pu][1][Hq/Pu][S/Pr] per rank), and with ``keep`` also the state
    ``usp_backward`` needs (the exchanged q, k, v and every rank's final output).
    """
    if q.shape[0] != 1:
        raise ValueError("usp_forward takes batch 1")
    S = q.shape[1]
    Sr, Sl = S // Pr, S // (Pr * Pu)
    stack = lambda t: ops.zigzag_reorder(t, Pr).view(Pr, Pu, 1, Sl, t.shape[2], t.shape[3])
    ql = ops.ulysses_relayout_ex(stack(q), Pu, groups=Pr)
    kl = ops.ulysses_relayout_ex(stack(k), Pu, groups=Pr, rep=kv_rep)
    vl = ops.ulysses_relayout_ex(stack(v), Pu, groups=Pr, rep=kv_rep)
    pos = [rank_positions(r, Pr, S, "zigzag", q.device) for r in range(Pr)]
    sz = None if seg is None else ops.zigzag_reorder(seg, Pr)
    Hl = ql.shape[4]
    acc = torch.zeros(ql.shape, device=q.device, dtype=torch.float32)
    lse = torch.full((Pr, Pu, 1, Hl, Sr), float("-inf"), device=q.device, dtype=torch.float32)
    # the fused step, unless the forward splits the blocks' keys (as in RingShare)
    ws = split_workspace(ql[0, 0], kl[0, 0], causal=causal, window=window, scale=scale, q_pos=pos[0],
                         k_pos=pos[0], q_seg=None if sz is None else sz[:, :Sr].contiguous(),
                         k_seg=None if sz is None else sz[:, :Sr].contiguous())
    if ws is not False:
        blk_o = torch.empty(ql.shape[2:], device=q.device, dtype=ql.dtype)
        blk_l = torch.empty(1, Hl, Sr, device=q.device, dtype=torch.float32)
    for r in range(Pr):
        for u in range(Pu):
            for step in range(Pr):
                src = (r - step) % Pr
                m = dict(causal=causal, window=window, scale=scale, q_pos=pos[r], k_pos=pos[src])
                if sz is not None:
                    m.update(q_seg=sz[:, r * Sr:(r + 1) * Sr].contiguous(), k_seg=sz[:, src * Sr:(src + 1) * Sr].contiguous())
                if ws is False:
                    ops.attn_fwd_merge(ql[r, u], kl[src, u], vl[src, u], acc[r, u], lse[r, u], **m)
                else:
                    ops.attn_fwd(ql[r, u], kl[src, u], vl[src, u], out=blk_o, lse=blk_l, workspace=ws, **m)
                    ops.lse_merge(acc[r, u], lse[r, u], blk_o, blk_l)
    back = ops.ulysses_relayout_ex(acc, Pu, groups=Pr, inverse=True)   # [Pr][Pu][1][Sl][Hq][D]
    out = ops.zigzag_reorder(back.view(1, S, back.shape[4], back.shape[5]), Pr, inverse=True)
    if keep:
        mask = dict(causal=causal, window=window, scale=scale)
        return out, lse, dict(ql=ql, kl=kl, vl=vl, acc=acc, pos=pos, sz=sz, Pr=Pr, Pu=Pu, kv_rep=kv_rep, mask=mask)
    return out, lse


def usp_backward(state, lse, dout):
    """Gradients through the Ulysses x ring hybrid of ``usp_forward(..., keep=True)``.

    dout [1,S,Hq,D] in sequence order (the forward's input dtype).  dout takes the
    forward's path (zigzag reorder for the Pr groups, Ulysses exchange inside each
    group); rank (r, u) runs the ring backward over the groups' blocks with its final
    output and lse (dq accumulated over the steps, the partial dk / dv of block src
    added onto that block); dq, dk, dv then take the inverse path (the exchange back,
    the copies of replicated kv heads summed, the inverse reorder).  Returns (dq, dk,
    dv) float32 [1,S,H,D] in sequence order.
    """
    ql, kl, vl, acc, pos, sz = (state[n] for n in ("ql", "kl", "vl", "acc", "pos", "sz"))
    Pr, Pu, rep, mask = state["Pr"], state["Pu"], state["kv_rep"], state["mask"]
    S = dout.shape[1]
    Sr, Sl = S // Pr, S // (Pr * Pu)
    gl = ops.ulysses_relayout_ex(ops.zigzag_reorder(dout, Pr).view(Pr, Pu, 1, Sl, dout.shape[2], dout.shape[3]),
                                 Pu, groups=Pr)
    out_l = acc.to(ql.dtype)   # every rank's final output, in the dtype the backward takes
    dql = torch.zeros(ql.shape, device=dout.device, dtype=torch.float32)
    dkl = torch.zeros(kl.shape, device=dout.device, dtype=torch.float32)
    dvl = torch.zeros(vl.shape, device=dout.device, dtype=torch.float32)
    for r in range(Pr):
        for u in range(Pu):
            ws, ready = None, False
            for step in range(Pr):
                src = (r - step) % Pr
                m = dict(mask, q_pos=pos[r], k_pos=pos[src])
                if sz is not None:
                    m.update(q_seg=sz[:, r * Sr:(r + 1) * Sr].contiguous(),
                             k_seg=sz[:, src * Sr:(src + 1) * Sr].contiguous())
                if ws is None:
                    ws = ops.bwd_workspace(ql[r, u], kl[src, u], **m)
                ops.attn_bwd(ql[r, u], kl[src, u], vl[src, u], out_l[r, u], lse[r, u], gl[r, u], dq=dql[r, u],
                             dk=dkl[src, u], dv=dvl[src, u], accumulate=True, workspace=ws, rows_ready=ready, **m)
                ready = True

    def back(t, rep_):
        y = ops.ulysses_relayout_ex(t, Pu, groups=Pr, rep=rep_, inverse=True)   # [Pr][Pu][1][Sl][H][D]
        return ops.zigzag_reorder(y.view(1, S, y.shape[4], y.shape[5]), Pr, inverse=True)

    return back(dql, 1), back(dkl, rep), back(dvl, rep)
