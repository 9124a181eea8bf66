"""CPU oracle for context-parallel attention (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The library under ``context_cp_attn_amd/`` never imports it, and it imports
nothing from the library: the two share no code.  The only module both sides use
is ``cp_inputs`` (seeded random inputs, no arithmetic of the method).

Everything is a plain, slow restatement of what the pages define, in float64:

* ``attention`` — blockwise causal softmax attention returning (out, lse) at given
  query/key offsets or positions, with segment ids, a sliding window and grouped
  query heads; and its gradient (closed-form VJP).
* ``merge`` — the log-sum-exp merge of two partial attentions.
* ``ulysses`` — the sequence<->head exchange of Ulysses, as the reshape /
  transpose / exchange steps of the handbook, for all ranks at once; kv-head
  replication beyond the kv head count and the Ulysses x ring hybrid (USP).
* ``zigzag`` — the 2P-chunk zigzag (dual-chunk-swap) and the striped partitions,
  their reorders and the causal work counts.
* ``ring`` — ring attention per rank (forward and blockwise backward).
* ``padding`` — padding a sequence at its end to a multiple of the CP degree.

Pins (checked by ``tests/test_oracle.py`` against facts other than the oracle's
own formulas) are listed in each module's docstring.
"""

from .attention import attn_fwd, attn_bwd, visible_mask  # noqa: F401
from .merge import lse_merge  # noqa: F401
from .ulysses import (seq_to_head, head_to_seq, ulysses_relayout, ulysses_relayout_inv,  # noqa: F401
                      ulysses_attn, ulysses_attn_bwd, replicate_heads, sum_replicas, ulysses_relayout_rep,
                      ulysses_relayout_inv_sum, usp_relayout, usp_relayout_inv, usp_attn)
from .zigzag import (chunk_order, reorder, reorder_inv, rank_positions, rank_chunks,  # noqa: F401
                     work, visible_pairs, striped_order, reorder_striped, reorder_striped_inv,
                     DUAL_CHUNK_SWAP, STRIPED)
from .ring import ring_fwd, ring_bwd, ring_block_counts  # noqa: F401
from .padding import padded_length, pad_rows, pad_segments  # noqa: F401
