"""Ulysses sequence<->head exchange, simulated for all P ranks at once.  float64.

Definition followed: handbook "Context parallelism: Ring Attention and Ulysses",
§"Ulysses: transposing between the sequence and the heads" (``seq_to_head`` and
``head_to_seq`` around an all-to-all).  Restated here as three explicit steps per
rank — split into per-destination groups, exchange (destination p receives group p
from every source, in source-rank order), then reassemble — with a leading batch
dimension added to the handbook's [S/P, H, D] per-rank tensors.

seq_to_head: rank r holds [B, S/P, H, D] (its slice of the sequence, all heads) and
ends with [B, S, H/P, D] (the whole sequence, heads [r·H/P, (r+1)·H/P)).
head_to_seq is its inverse.

Pins (tests/test_oracle.py): head_to_seq(seq_to_head(x)) = x exactly; Ulysses
attention equals full attention; toy per-rank shapes (8, 8, 16) -> (32, 2, 16) as
the handbook's script prints them; a degree above the KV head count is refused.
"""

from __future__ import annotations

import numpy as np

from .attention import attn_fwd


def _exchange(send):
    """send[r][p] is what rank r sends to rank p; returns recv[p][r] = send[r][p]."""
    P = len(send)
    return [[send[r][p] for r in range(P)] for p in range(P)]


def seq_to_head(xs):
    """xs: list over ranks of [B, S/P, H, D] arrays -> list of [B, S, H/P, D]."""
    P = len(xs)
    B, Sp, H, D = xs[0].shape
    if H % P:
        raise ValueError(f"heads {H} not divisible by the Ulysses degree {P}")
    # group p of rank r = heads [p*H/P, (p+1)*H/P) of its sequence slice
    send = [[x.reshape(B, Sp, P, H // P, D)[:, :, p] for p in range(P)] for x in xs]
    recv = _exchange(send)
    # received groups come in source-rank order = sequence order
    return [np.concatenate(recv[p], axis=1) for p in range(P)]


def head_to_seq(ys):
    """ys: list over ranks of [B, S, H/P, D] arrays -> list of [B, S/P, H, D]."""
    P = len(ys)
    B, S, Hp, D = ys[0].shape
    if S % P:
        raise ValueError(f"sequence {S} not divisible by the Ulysses degree {P}")
    Sp = S // P
    # group s of rank p = sequence slice s of its heads
    send = [[y[:, s * Sp:(s + 1) * Sp] for s in range(P)] for y in ys]
    recv = _exchange(send)
    # rank s reassembles its slice with the heads in source-rank order
    return [np.concatenate(recv[s], axis=2) for s in range(P)]


def ulysses_relayout(stack):
    """[P][B][S/P][H][D] -> [P][B][S][H/P][D] (all ranks' seq_to_head)."""
    stack = np.asarray(stack)
    return np.stack(seq_to_head(list(stack)))


def ulysses_relayout_inv(stack):
    """[P][B][S][H/P][D] -> [P][B][S/P][H][D] (all ranks' head_to_seq)."""
    stack = np.asarray(stack)
    return np.stack(head_to_seq(list(stack)))


def ulysses_attn(q, k, v, P, **mask):
    """Full Ulysses forward for P ranks: seq_to_head(q, k, v), per-rank attention on
    its heads over the whole sequence, head_to_seq(out).

    q [B,S,Hq,D], k/v [B,S,Hkv,D] global (sequence order).  Returns the global
    output [B,S,Hq,D] and lse [B,Hq,S] reassembled from the ranks.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hkv % P or Hq % P:
        raise ValueError(f"Ulysses degree {P} must divide the kv head count {Hkv}")
    if S % P:
        raise ValueError(f"sequence {S} not divisible by the Ulysses degree {P}")
    Sp = S // P
    split = lambda t: [t[:, r * Sp:(r + 1) * Sp] for r in range(P)]
    ql, kl, vl = seq_to_head(split(q)), seq_to_head(split(k)), seq_to_head(split(v))
    outs, lses = [], []
    for p in range(P):
        o, l = attn_fwd(ql[p], kl[p], vl[p], **mask)
        outs.append(o)
        lses.append(l)
    out = np.concatenate(head_to_seq(outs), axis=1)
    lse = np.concatenate(lses, axis=1)  # rank p holds heads [p*Hq/P, (p+1)*Hq/P)
    return out, lse, (ql, kl, vl)
