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

Beyond the kv head count (same handbook, §Exercises): either replicate each kv head
onto several ranks by group before the exchange — head j of the replicated set is kv
head j // rep, so a contiguous split of the heads gives every rank one whole kv
head; the gradient of the copies is their sum — or run Ulysses within groups of Pu
ranks and ring attention across the Pr groups (the Ulysses x ring hybrid, USP, that
the handbook's comparison and the MaxText Ulysses PR describe): the sequence is
zigzag-partitioned over the groups, each group's share split over its Pu ranks,
exchanged within the group, and the groups' KV blocks passed round a ring.

Pins (tests/test_oracle.py): head_to_seq(seq_to_head(x)) = x exactly; Ulysses
attention equals full attention; toy per-rank shapes (8, 8, 16) -> (32, 2, 16) as
the handbook's script prints them; a degree above the KV head count is refused
without replication.  With replication (degree 2x and 4x the kv heads) and as USP,
forward and gradients equal full attention's.
"""

from __future__ import annotations

import numpy as np

from .attention import attn_fwd, attn_bwd
from .merge import lse_merge
from .zigzag import rank_positions, reorder, reorder_inv


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


def replicate_heads(x, rep):
    """[..., H, D] -> [..., H*rep, D]: head j of the result is head j // rep."""
    return np.repeat(np.asarray(x), rep, axis=-2)


def sum_replicas(x, rep):
    """[..., H*rep, D] -> [..., H, D]: the sum over each head's rep copies (the
    gradient of ``replicate_heads``)."""
    x = np.asarray(x)
    *lead, H, D = x.shape
    return x.reshape(*lead, H // rep, rep, D).sum(axis=-2)


def ulysses_relayout_rep(stack, rep):
    """[P][B][S/P][H][D] -> [P][B][S][H*rep/P][D]: heads replicated, then exchanged."""
    return ulysses_relayout(replicate_heads(stack, rep))


def ulysses_relayout_inv_sum(stack, rep):
    """[P][B][S][H*rep/P][D] -> [P][B][S/P][H][D]: exchanged back, copies summed."""
    return sum_replicas(ulysses_relayout_inv(stack), rep)


def usp_relayout(stack):
    """[Pr][Pu][B][Sl][H][D] -> [Pr][Pu][B][Pu*Sl][H/Pu][D]: the Ulysses exchange
    within each of the Pr groups."""
    return np.stack([ulysses_relayout(g) for g in np.asarray(stack)])


def usp_relayout_inv(stack):
    return np.stack([ulysses_relayout_inv(g) for g in np.asarray(stack)])


def ulysses_attn(q, k, v, P, kv_rep=1, **mask):
    """Full Ulysses forward for P ranks: seq_to_head(q, k, v), per-rank attention on
    its heads over the whole sequence, head_to_seq(out).  kv_rep > 1 replicates the
    kv heads first (degree up to kv heads x kv_rep).

    q [B,S,Hq,D], k/v [B,S,Hkv,D] global (sequence order).  Returns the global
    output [B,S,Hq,D] and lse [B,Hq,S] reassembled from the ranks.
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if kv_rep > 1:
        k, v = replicate_heads(k, kv_rep), replicate_heads(v, kv_rep)
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


def ulysses_attn_bwd(q, k, v, dout, P, kv_rep=1, **mask):
    """Gradients through Ulysses: exchange q, k, v (kv replicated) and dout, per-rank
    attention gradients, exchange dq, dk, dv back, sum the kv copies."""
    q, k, v, dout = (np.asarray(t, dtype=np.float64) for t in (q, k, v, dout))
    kr, vr = replicate_heads(k, kv_rep), replicate_heads(v, kv_rep)
    S = q.shape[1]
    Sp = S // P
    split = lambda t: [t[:, r * Sp:(r + 1) * Sp] for r in range(P)]
    ql, kl, vl, gl = (seq_to_head(split(t)) for t in (q, kr, vr, dout))
    dqs, dks, dvs = [], [], []
    for p in range(P):
        o, l = attn_fwd(ql[p], kl[p], vl[p], **mask)
        a, b, c = attn_bwd(ql[p], kl[p], vl[p], o, l, gl[p], **mask)
        dqs.append(a)
        dks.append(b)
        dvs.append(c)
    back = lambda ys: np.concatenate(head_to_seq(ys), axis=1)
    return back(dqs), sum_replicas(back(dks), kv_rep), sum_replicas(back(dvs), kv_rep)


def usp_attn(q, k, v, Pr, Pu, kv_rep=1, causal=True, seg=None, **mask):
    """Ulysses within groups of Pu ranks x ring across Pr groups, for all Pr*Pu ranks.

    The sequence is zigzag-reordered for the Pr groups; group r's share is split
    contiguously over its Pu ranks; the Ulysses exchange inside the group gives rank
    (r, u) group r's share with heads slice u; rank (r, u) then runs the ring over
    the groups' blocks of heads slice u (step s: block (r - s) mod Pr) and merges.
    seg [B,S] (sequence order): segment ids of packed documents; every row keeps its
    own id through the reorder.  Returns the global output [B,S,Hq,D] (sequence
    order) and lse [B,Hq,S].
    """
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    if kv_rep > 1:
        k, v = replicate_heads(k, kv_rep), replicate_heads(v, kv_rep)
    B, S, Hq, D = q.shape
    segs = None if seg is None else np.asarray(seg)
    if k.shape[2] % Pu or Hq % Pu:
        raise ValueError(f"Ulysses degree {Pu} must divide the kv head count {k.shape[2]}")
    Sr = S // Pr
    Sl = Sr // Pu
    qz, kz, vz = (reorder(t, Pr) for t in (q, k, v))
    # stacks [Pr][Pu][B][Sl][H][D]: group r, rank u holds rows r*Sr + u*Sl ...
    stack = lambda t: np.stack([np.stack([t[:, r * Sr + u * Sl:r * Sr + (u + 1) * Sl] for u in range(Pu)])
                                for r in range(Pr)])
    ql, kl, vl = (usp_relayout(stack(t)) for t in (qz, kz, vz))
    pos = [rank_positions(r, Pr, S, "zigzag") for r in range(Pr)]
    outs = np.zeros((Pr, Pu, B, Sr, Hq // Pu, D))
    lse = np.zeros((B, Hq, S))
    for r in range(Pr):
        for u in range(Pu):
            acc = None
            for s in range(Pr):
                src = (r - s) % Pr
                sm = {} if segs is None else dict(q_seg=segs[:, pos[r]], k_seg=segs[:, pos[src]])
                o, l = attn_fwd(ql[r, u], kl[src, u], vl[src, u], causal=causal, q_pos=pos[r], k_pos=pos[src],
                                **sm, **mask)
                acc = (o, l) if acc is None else lse_merge(acc[0], acc[1], o, l)
            outs[r, u] = acc[0]
            lse[:, u * Hq // Pu:(u + 1) * Hq // Pu][:, :, pos[r]] = acc[1]
    back = usp_relayout_inv(outs)  # [Pr][Pu][B][Sl][Hq][D]
    seq = np.concatenate([np.concatenate(list(back[r]), axis=1) for r in range(Pr)], axis=1)
    return reorder_inv(seq, Pr), lse
