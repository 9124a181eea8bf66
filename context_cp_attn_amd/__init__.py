"""context_cp_attn_amd — context-parallel attention hot path on one MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (include/cp_attn.h, libcp_attn.so):

* ``attn_fwd`` / ``attn_bwd`` — blockwise causal attention returning (out, lse) at
  given query/key positions, with segment ids, a sliding window and grouped kv heads;
* ``lse_merge`` — the ring step's log-sum-exp merge; ``attn_fwd_merge`` — the ring
  step fused: attention whose epilogue merges into the running (out, lse);
* ``ulysses_relayout`` / ``ulysses_relayout_inv`` — the sequence<->head exchange of
  all simulated ranks as one local permute; ``ulysses_relayout_ex`` adds groups
  (Ulysses x ring, USP) and kv-head replication beyond the kv head count;
* ``zigzag_reorder`` — the zigzag / dual-chunk-swap (or striped) load-balancing
  reorder; ``pad_rows`` — end padding of a sequence to a multiple of the CP degree.

``drivers`` simulates the P ranks' ring and Ulysses shares on one GPU.
torch provides device memory and the stream; nothing here computes on the CPU.
"""

from ._lib import CpError, load as load_library  # noqa: F401
from .ops import (attn_fwd, attn_fwd_merge, attn_bwd, attn_bwd_noalloc, lse_merge, ulysses_relayout,  # noqa: F401
                  ulysses_relayout_inv, ulysses_relayout_ex, zigzag_reorder, pad_rows, bwd_workspace,
                  check_attn_args, fwd_workspace)
from . import drivers  # noqa: F401
