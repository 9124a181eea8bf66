"""Seeded synthetic inputs for the context-parallel attention workloads.

This module is shared by the tests, the benchmark and the smoke check, and is the
only code the CPU oracle and the HIP path have in common. It draws random numbers
and lays out workload shapes; it holds none of the attention, merge, relayout or
reorder arithmetic.

Recipe (stated once, used everywhere):

* Toy workload: the handbook "Context parallelism: Ring Attention and Ulysses",
  §"Which operations partition directly" (``make_qkv``): ``torch.manual_seed(0)``,
  then ``torch.randn(S, H, D)`` three times for q, k, v with S=32, H=8, D=16, fp32.
  A leading batch dimension of 1 is added.
* Every other workload: ``torch.manual_seed(seed)`` (0 unless stated), then
  ``torch.randn`` in fp32 on the CPU, one tensor at a time in the order the caller
  lists them (q, k, v, dout), multiplied by ``scale`` (0.5) and rounded to bf16
  (round-to-nearest-even, torch's cast).
* Packed documents: lengths drawn with ``torch.randint(lo, hi + 1, ())`` from a
  generator seeded ``seed`` (1) until their sum reaches the sequence length; the
  last document is cut to fit.  A token's segment id is the index of its document.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import torch


def toy_qkv(S: int = 32, H: int = 8, D: int = 16):
    """q, k, v of shape [1, S, H, D] fp32, drawn exactly as the handbook's toy data."""
    torch.manual_seed(0)
    q = torch.randn(S, H, D)
    k = torch.randn(S, H, D)
    v = torch.randn(S, H, D)
    return q[None].contiguous(), k[None].contiguous(), v[None].contiguous()


def normal_tensors(shapes, seed: int = 0, scale: float = 0.5, dtype=torch.bfloat16):
    """One tensor per shape, ~N(0,1)*scale drawn in fp32 in list order, then cast."""
    torch.manual_seed(seed)
    out = []
    for shp in shapes:
        t = torch.randn(*shp, dtype=torch.float32)
        if scale != 1.0:
            t.mul_(scale)
        out.append(t.to(dtype))
    return out


def doc_lengths(total: int, lo: int = 256, hi: int = 4096, seed: int = 1):
    """Document lengths uniform in [lo, hi] until they cover ``total`` tokens."""
    g = torch.Generator().manual_seed(seed)
    lens = []
    while sum(lens) < total:
        lens.append(int(torch.randint(lo, hi + 1, (), generator=g)))
    lens[-1] -= sum(lens) - total
    return lens


def segment_ids(lengths, batch: int = 1) -> torch.Tensor:
    """[batch, sum(lengths)] int32 document index of every token."""
    ids = torch.cat([torch.full((n,), i, dtype=torch.int32) for i, n in enumerate(lengths)])
    return ids[None].expand(batch, -1).contiguous()


def random_segment_ids(S: int, lo: int, hi: int, seed: int, batch: int = 1) -> torch.Tensor:
    """Segment ids of uniformly drawn document lengths, for small parity cases."""
    return segment_ids(doc_lengths(S, lo, hi, seed), batch)


@dataclass(frozen=True)
class Workload:
    """Shapes of one named workload.  Sizes only: no arithmetic of the method."""

    name: str
    batch: int
    seqlen: int           # full (global) sequence length
    heads_q: int
    heads_kv: int
    head_dim: int
    cp: int               # number of simulated context-parallel ranks
    dtype: torch.dtype
    causal: bool = True
    window: int = 0
    packed: bool = False
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    # Toy: S=32, H=8, D=16 fp32, P=4.
    "toy": Workload("toy", 1, 32, 8, 8, 16, 4, torch.float32),
    # Ulysses share of llama2-7b (MHA, 32 heads), 32K context, cp=16: one rank holds
    # the full 32768-token sequence for 2 of the 32 heads.
    "ulysses_llama2_7b_32k_cp16": Workload(
        "ulysses_llama2_7b_32k_cp16", 1, 32768, 32, 32, 128, 16, torch.bfloat16),
    # Ring share of llama2-7b: 2048 local queries x 32 heads against 16 KV blocks.
    "ring_llama2_7b_32k_cp16": Workload(
        "ring_llama2_7b_32k_cp16", 1, 32768, 32, 32, 128, 16, torch.bfloat16),
    # Ulysses share of llama3.1-8b (GQA 32 q / 8 kv heads), 64K, cp=4: 8 q heads
    # sharing 2 kv heads per rank.
    "ulysses_llama31_8b_64k_cp4": Workload(
        "ulysses_llama31_8b_64k_cp4", 1, 65536, 32, 8, 128, 4, torch.bfloat16),
    # Packed + windowed ring share: 8K, 32 q / 8 kv heads, documents 256..4096,
    # window 4096, cp=4.
    "packed_window_8k_cp4": Workload(
        "packed_window_8k_cp4", 1, 8192, 32, 8, 128, 4, torch.bfloat16,
        window=4096, packed=True),
}
