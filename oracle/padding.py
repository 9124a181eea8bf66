"""Padding a sequence at its end to a multiple of the context-parallel degree.

Definition followed: transformers PR "[distributed] Context parallel module, with
Ulysses", "What this PR brings" (ModelContextParallel) and the later note on it.
In short: each sequence is padded at its end up to a multiple of the CP degree
before any mask exists; the padded embedding and mask entries are zero, pad
positions carry on from the last document, and pad tokens are excluded from what
is counted.

Here: ``pad_rows`` appends zero (or ``fill``) rows along the sequence axis, or
truncates; pad tokens sit at positions S, S+1, ... (the sequence simply continues);
``pad_segments`` gives the pad tokens a segment id of their own, so that no real
query sees a pad key even without the causal mask (under the causal mask a pad key,
later than every real query, is never visible anyway).

Pins (tests/test_oracle.py): attention of the real rows is unchanged by end
padding — causal without segment ids, non-causal and packed with the pad segment,
for plain, ring (zigzag) and Ulysses partitions of the padded sequence.
"""

from __future__ import annotations

import numpy as np


def padded_length(S, multiple):
    return -(-S // multiple) * multiple


def pad_rows(x, S_out, fill=0, axis=1):
    """Copy the first min(S, S_out) rows along ``axis``; rows beyond S are ``fill``."""
    x = np.asarray(x)
    S = x.shape[axis]
    if S_out <= S:
        return np.take(x, np.arange(S_out), axis=axis)
    shape = list(x.shape)
    shape[axis] = S_out - S
    return np.concatenate([x, np.full(shape, fill, dtype=x.dtype)], axis=axis)


def pad_segments(seg, S_out):
    """[B, S] segment ids -> [B, S_out]; the pad tokens get max id + 1."""
    seg = np.asarray(seg)
    return pad_rows(seg, S_out, fill=int(seg.max()) + 1)
