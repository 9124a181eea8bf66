"""Ring attention for P simulated ranks: forward with LSE merge, blockwise backward.

Definition followed: handbook "Context parallelism: Ring Attention and Ulysses",
§"Ring Attention: passing the KV once around a ring": each rank keeps its queries;
at step s it holds the KV block of rank src = (rank - s) mod P, computes the partial
(out, lse) of its queries against that block at the block's global positions, and
merges it into its running result with the log-sum-exp merge.  With the zigzag
partition (§"The zigzag partition") a rank's queries and KV blocks are its two
chunks.  Here every block is computed: a block with no visible pair gives lse = -inf
rows, which the merge treats as the identity (the handbook skips such blocks
instead; the result is the same).

Backward (not on the pages; the plain reading): per (rank, step) block, the
attention gradient evaluated with the rows' final (out, lse); dq sums over steps,
dk/dv partials are summed back onto the positions of block src.

Pins (tests/test_oracle.py): ring equals full attention for contiguous and zigzag
partitions; the contiguous ring computes [1, 2, 3, 4] blocks per rank at P = 4; ring
backward equals full backward.
"""

from __future__ import annotations

import numpy as np

from .attention import attn_fwd, attn_bwd, visible_mask
from .merge import lse_merge
from .zigzag import rank_positions


def _gather(t, pos):
    return None if t is None else np.asarray(t)[:, pos]


def ring_fwd(q, k, v, P, layout="zigzag", causal=True, seg=None, window=0, scale=None):
    """q/k/v global [B,S,H*,D] in sequence order.  Returns per rank
    (positions, out [B,S/P,Hq,D], lse [B,Hq,S/P])."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    S = q.shape[1]
    res = []
    for r in range(P):
        qpos = rank_positions(r, P, S, layout)
        out = lse = None
        for s in range(P):
            src = (r - s) % P
            kpos = rank_positions(src, P, S, layout)
            o, l = attn_fwd(q[:, qpos], k[:, kpos], v[:, kpos], causal=causal,
                            q_pos=qpos, k_pos=kpos, q_seg=_gather(seg, qpos),
                            k_seg=_gather(seg, kpos), window=window, scale=scale)
            if out is None:
                out, lse = o, l
            else:
                out, lse = lse_merge(out, lse, o, l)
        res.append((qpos, out, lse))
    return res


def ring_bwd(q, k, v, dout, P, layout, finals, causal=True, seg=None, window=0, scale=None):
    """finals: per rank (positions, out, lse) from ``ring_fwd``.  dout global
    [B,S,Hq,D].  Returns global (dq, dk, dv)."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    S = q.shape[1]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for r in range(P):
        qpos, out, lse = finals[r]
        for s in range(P):
            src = (r - s) % P
            kpos = rank_positions(src, P, S, layout)
            gq, gk, gv = attn_bwd(q[:, qpos], k[:, kpos], v[:, kpos], out, lse, dout[:, qpos],
                                  causal=causal, q_pos=qpos, k_pos=kpos,
                                  q_seg=_gather(seg, qpos), k_seg=_gather(seg, kpos),
                                  window=window, scale=scale)
            dq[:, qpos] += gq
            dk[:, kpos] += gk
            dv[:, kpos] += gv
    return dq, dk, dv


def ring_block_counts(P, S, layout, causal=True):
    """Per rank, how many of its P ring steps hold a block with a visible pair."""
    counts = []
    for r in range(P):
        qpos = rank_positions(r, P, S, layout)
        n = 0
        for s in range(P):
            kpos = rank_positions((r - s) % P, P, S, layout)
            n += int(visible_mask(qpos, kpos, causal).any())
        counts.append(n)
    return counts
