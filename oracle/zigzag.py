"""Load-balancing partitions and reorders: zigzag (dual-chunk-swap) and striped;
causal work counts.

Definition followed: handbook "Context parallelism: Ring Attention and Ulysses",
§"The zigzag partition": the sequence is cut into 2P chunks and rank r takes chunk r
and chunk 2P-1-r; in the in-order partition rank r takes chunks 2r and 2r+1.  The
MaxText PR "Add Packing Support for Context Parallelism (Ring Attention)" names the
same permutation DualChunkSwap (reorder strategy 0) and applies it to the batch
before contiguous sharding, so the reordered sequence is the ranks' shares in rank
order: for P = 4 the chunk order is 0,7,1,6,2,5,3,4.

``work`` restates the handbook's causal cost of a set of query chunks: a query chunk
needs every earlier KV chunk in full and its own chunk (the diagonal) half.

Striped (reorder strategy 1 of the same MaxText PR, left undefined there beyond its
name; the handbook mentions a striped partition as the alternative): token t goes to
rank t mod P, so rank r holds positions r, r+P, r+2P, ...; as for the zigzag the
reordered sequence is the ranks' shares in rank order.  (The PR's automatic choice
between the two strategies is a host policy, not arithmetic of the method; it is
not part of this oracle.)

Pins (tests/test_oracle.py, tests/golden/): work = [2,6,10,14] in order and
[8,8,8,8] zigzag at P = 4; the exact visible-pair count of every zigzag rank at every
ring step; reorder_inv(reorder(x)) = x.  Striped: every rank's positions have stride
P and cover the sequence once; the exact pair count of rank r against block src is
c(c-1)/2 + c*[src <= r] (c = S/P), summing to S(S+1)/2; ring attention over striped
shares equals full attention, forward and backward.
"""

from __future__ import annotations

import numpy as np

DUAL_CHUNK_SWAP = 0
STRIPED = 1


def rank_chunks(rank, P, layout):
    if layout == "contiguous":
        return [2 * rank, 2 * rank + 1]
    if layout == "zigzag":
        return [rank, 2 * P - 1 - rank]
    raise ValueError(f"unknown layout {layout!r}")


def chunk_order(P):
    """Chunk index placed at each position of the reordered sequence."""
    return [c for r in range(P) for c in rank_chunks(r, P, "zigzag")]


def _chunks(x, n, axis):
    if x.shape[axis] % n:
        raise ValueError(f"sequence {x.shape[axis]} not divisible into {n} chunks")
    return np.split(x, n, axis=axis)


def reorder(x, P, axis=1):
    """Sequence order -> zigzag order (rank shares concatenated in rank order)."""
    x = np.asarray(x)
    ch = _chunks(x, 2 * P, axis)
    return np.concatenate([ch[c] for c in chunk_order(P)], axis=axis)


def reorder_inv(y, P, axis=1):
    """Zigzag order -> sequence order."""
    y = np.asarray(y)
    ch = _chunks(y, 2 * P, axis)
    out = [None] * (2 * P)
    for slot, c in enumerate(chunk_order(P)):
        out[c] = ch[slot]
    return np.concatenate(out, axis=axis)


def striped_order(P, S):
    """Sequence position placed at each row of the striped order."""
    if S % P:
        raise ValueError(f"sequence {S} not divisible by {P} ranks")
    return np.concatenate([np.arange(r, S, P) for r in range(P)])


def reorder_striped(x, P, axis=1):
    """Sequence order -> striped order (rank r's tokens r, r+P, ... in rank order)."""
    x = np.asarray(x)
    return np.take(x, striped_order(P, x.shape[axis]), axis=axis)


def reorder_striped_inv(y, P, axis=1):
    """Striped order -> sequence order."""
    y = np.asarray(y)
    order = striped_order(P, y.shape[axis])
    out = np.empty_like(y)
    idx = [slice(None)] * y.ndim
    for row, t in enumerate(order):
        idx[axis] = t
        src = [slice(None)] * y.ndim
        src[axis] = row
        out[tuple(idx)] = y[tuple(src)]
    return out


def rank_positions(rank, P, S, layout):
    """Global token positions held by ``rank`` (increasing)."""
    if layout == "striped":
        if S % P:
            raise ValueError(f"sequence {S} not divisible by {P} ranks")
        return np.arange(rank, S, P)
    if S % (2 * P):
        raise ValueError(f"sequence {S} not divisible into {2 * P} chunks")
    c = S // (2 * P)
    return np.concatenate([np.arange(ch * c, (ch + 1) * c) for ch in rank_chunks(rank, P, layout)])


def work(query_chunks):
    """Causal KV chunks a set of query chunks needs, the diagonal counted as half."""
    return float(sum(query_chunks)) + 0.5 * len(query_chunks)


def visible_pairs(qpos, kpos, causal=True, qseg=None, kseg=None, window=0):
    """Exact number of visible (query, key) pairs of one head."""
    from .attention import visible_mask
    return int(visible_mask(qpos, kpos, causal, qseg, kseg, window).sum())
