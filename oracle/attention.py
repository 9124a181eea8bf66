"""Blockwise softmax attention with (out, lse), and its gradient.  float64.

Definition followed: handbook "Context parallelism: Ring Attention and Ulysses",
§"Which operations partition directly", the shared ``attention(q, k, v, causal,
q_offset, k_offset)``: scores are q·k scaled by 1/sqrt(D); with the causal mask a
key whose global index exceeds the query's global index gets -inf; lse is the
log-sum-exp of a row's scores; out is exp(scores - lse) applied to v.

Extensions (readings where the pages are silent):

* Per-token global positions (``q_pos``/``k_pos``) replace ``offset + index`` so a
  zigzag rank's two chunks can be described; they must be increasing.
* Segment ids (packing, MaxText PR "Add Packing Support for Context Parallelism
  (Ring Attention)", §Description and the ``segment_pos`` commit): a key is visible
  only to queries of the same document.
* Sliding window (HF PR "[distributed] Context parallel module, with Ulysses",
  §Tests names it without defining it): a key is visible iff
  0 <= qpos - kpos < window, the window most recent positions up to the query's own
  (window 0 = none).  The lower bound holds with or without the causal flag, so a
  window implies the causal rule.
* Grouped query heads (handbook §Ulysses, degree bounded by the KV head count):
  query head h uses kv head h // (Hq / Hkv).
* A row with no visible key: out = 0 and lse = -inf (the handbook's code would give
  NaN; it never meets the case because it skips later blocks).

Layouts: q [B,Sq,Hq,D], k/v [B,Sk,Hkv,D], out [B,Sq,Hq,D], lse [B,Hq,Sq].

Pins (tests/test_oracle.py): q = 0 closed form (lse = log #visible, out = mean of
visible v) for causal, packed and windowed masks; causal row 0 gives v_0; window 1
gives v_i; non-causal equals torch's scaled_dot_product_attention; explicit-loop
brute force on tiny inputs; GQA equals MHA on repeated K/V; packed equals separate
per-document attention; the gradient equals central finite differences, and
sum_j dK_j = 0, sum_j dV_j = sum_i dO_i.
"""

from __future__ import annotations

import numpy as np


def _f64(x):
    if hasattr(x, "detach"):  # torch tensor: widen exactly (bf16 -> fp32 -> fp64)
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x, dtype=np.int64)


def visible_mask(qpos, kpos, causal=True, qseg=None, kseg=None, window=0):
    """Boolean [Sq, Sk]: which keys each query may attend to (one batch row)."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    vis = np.ones((qpos.shape[0], kpos.shape[0]), dtype=bool)
    if causal:
        vis &= kpos[None, :] <= qpos[:, None]
    if qseg is not None:
        vis &= np.asarray(qseg)[:, None] == np.asarray(kseg)[None, :]
    if window:
        d = qpos[:, None] - kpos[None, :]
        vis &= (d >= 0) & (d < window)
    return vis


def _positions(n, offset, pos):
    if pos is None:
        return offset + np.arange(n, dtype=np.int64)
    pos = _i64(pos)
    assert pos.shape == (n,), "positions must have one entry per token"
    return pos


def attn_fwd(q, k, v, *, causal=True, q_offset=0, k_offset=0, q_pos=None, k_pos=None,
             q_seg=None, k_seg=None, window=0, scale=None, row_block=512):
    """Returns (out [B,Sq,Hq,D], lse [B,Hq,Sq]) in float64."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    assert Hq % Hkv == 0, "query heads must be a multiple of kv heads"
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    qpos = _positions(Sq, q_offset, q_pos)
    kpos = _positions(Sk, k_offset, k_pos)
    qseg, kseg = _i64(q_seg), _i64(k_seg)
    out = np.zeros((B, Sq, Hq, D))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for i0 in range(0, Sq, row_block):
            i1 = min(Sq, i0 + row_block)
            vis = visible_mask(qpos[i0:i1], kpos, causal,
                               None if qseg is None else qseg[b, i0:i1],
                               None if kseg is None else kseg[b], window)
            has = vis.any(axis=1)
            for h in range(Hq):
                g = h // G
                s = (q[b, i0:i1, h, :] @ k[b, :, g, :].T) * scale
                s = np.where(vis, s, -np.inf)
                m = np.where(has, s.max(axis=1, initial=-np.inf), 0.0)
                e = np.exp(s - m[:, None])  # exp(-inf) = 0 on masked keys
                l = np.where(has, m + np.log(np.where(has, e.sum(axis=1), 1.0)), -np.inf)
                p = np.where(has[:, None], np.exp(s - np.where(has, l, 0.0)[:, None]), 0.0)
                out[b, i0:i1, h, :] = p @ v[b, :, g, :]
                lse[b, h, i0:i1] = l
    return out, lse


def attn_bwd(q, k, v, out, lse, dout, *, causal=True, q_offset=0, k_offset=0, q_pos=None,
             k_pos=None, q_seg=None, k_seg=None, window=0, scale=None, row_block=512):
    """Gradient of sum(dout * out) w.r.t. q, k, v, given the rows' final (out, lse).

    The textbook softmax-attention VJP: with P = exp(s - lse) on visible pairs,
    Delta_i = sum_d dO_id O_id, dV = P^T dO, dP = dO V^T, dS = P * (dP - Delta),
    dQ = scale dS K, dK = scale dS^T Q; dK, dV summed over each query-head group.
    When ``out``/``lse`` are the final values of rows whose keys are split into
    blocks, the per-block results sum to the full gradient (ring backward).
    Returns (dq [B,Sq,Hq,D], dk [B,Sk,Hkv,D], dv [B,Sk,Hkv,D]) float64.
    """
    q, k, v, out, dout = _f64(q), _f64(k), _f64(v), _f64(out), _f64(dout)
    lse = _f64(lse)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    qpos = _positions(Sq, q_offset, q_pos)
    kpos = _positions(Sk, k_offset, k_pos)
    qseg, kseg = _i64(q_seg), _i64(k_seg)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for i0 in range(0, Sq, row_block):
            i1 = min(Sq, i0 + row_block)
            vis = visible_mask(qpos[i0:i1], kpos, causal,
                               None if qseg is None else qseg[b, i0:i1],
                               None if kseg is None else kseg[b], window)
            for h in range(Hq):
                g = h // G
                l = lse[b, h, i0:i1]
                ok = vis & np.isfinite(l)[:, None]
                lsafe = np.where(np.isfinite(l), l, 0.0)
                s = (q[b, i0:i1, h, :] @ k[b, :, g, :].T) * scale
                p = np.where(ok, np.exp(np.where(ok, s, 0.0) - lsafe[:, None]), 0.0)
                do = dout[b, i0:i1, h, :]
                delta = (do * out[b, i0:i1, h, :]).sum(axis=1)
                dv[b, :, g, :] += p.T @ do
                dp = do @ v[b, :, g, :].T
                ds = p * (dp - delta[:, None])
                dq[b, i0:i1, h, :] += scale * (ds @ k[b, :, g, :])
                dk[b, :, g, :] += scale * (ds.T @ q[b, i0:i1, h, :])
    return dq, dk, dv
