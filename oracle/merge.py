"""Log-sum-exp merge of two partial attentions over disjoint key sets.  float64.

Definition: handbook "Context parallelism: Ring Attention and Ulysses", self-test
answers and §"Ring Attention": lse = log(e^lse1 + e^lse2), and
o = o1·e^(lse1 - lse) + o2·e^(lse2 - lse).

Reading for empty parts (a row that saw no key in a block has lse = -inf): its
weight is 0, so merge(x, (0, -inf)) = x, and two empty parts give (0, -inf).

Pins (tests/test_oracle.py): merging the attention of any two halves of a key set
reproduces attention over the whole set, in either order; the empty part is the
identity.

Layouts: o [B,S,H,D], lse [B,H,S].
"""

from __future__ import annotations

import numpy as np


def lse_merge(o1, lse1, o2, lse2):
    o1, o2 = np.asarray(o1, dtype=np.float64), np.asarray(o2, dtype=np.float64)
    lse1, lse2 = np.asarray(lse1, dtype=np.float64), np.asarray(lse2, dtype=np.float64)
    lse = np.logaddexp(lse1, lse2)  # -inf only if both are -inf
    fin = np.isfinite(lse)
    safe = np.where(fin, lse, 0.0)
    w1 = np.where(np.isfinite(lse1), np.exp(np.where(np.isfinite(lse1), lse1, 0.0) - safe), 0.0)
    w2 = np.where(np.isfinite(lse2), np.exp(np.where(np.isfinite(lse2), lse2, 0.0) - safe), 0.0)
    # [B,H,S] weights -> [B,S,H,1]
    w1 = np.transpose(w1, (0, 2, 1))[..., None]
    w2 = np.transpose(w2, (0, 2, 1))[..., None]
    return o1 * w1 + o2 * w2, lse
