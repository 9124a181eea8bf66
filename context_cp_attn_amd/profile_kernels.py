"""Run one attention kernel a few times on synthetic bf16 inputs, for profilers.

    python -m context_cp_attn_amd.profile_kernels {fwd|bwd|ring} [S,Hq,Hkv,D] [--iters N]

Intended under ``rocprofv3 --pmc ...`` or ``--kernel-trace``: the inputs are made
on the device, the chosen kernel runs ``iters`` times (default 2), and nothing
else of the library is launched in between.  ``fwd`` / ``bwd``: causal attention of
batch 1 at the given shape (the forward splits its keys over two workgroups where
cp_attn_fwd_workspace_size asks for it).  ``ring``: rank 0's pass of the fused ring
step over S tokens in zigzag order with P = 16 ranks (q [1,S/16,Hq,D] against the
16 key blocks), one pass per iteration.
"""

from __future__ import annotations

import argparse

import torch

from . import ops


def main() -> None:
    ap = argparse.ArgumentParser()
    ap.add_argument("which", choices=["fwd", "bwd", "ring"])
    ap.add_argument("shape", nargs="?", default="65536,8,2,128", help="S,Hq,Hkv,D (causal, batch 1)")
    ap.add_argument("--iters", type=int, default=2)
    a = ap.parse_args()
    S, Hq, Hkv, D = (int(x) for x in a.shape.split(","))
    g = torch.Generator(device="cuda").manual_seed(0)
    q = torch.randn(1, S, Hq, D, device="cuda", generator=g).mul_(0.5).bfloat16()
    k = torch.randn(1, S, Hkv, D, device="cuda", generator=g).mul_(0.5).bfloat16()
    v = torch.randn(1, S, Hkv, D, device="cuda", generator=g).mul_(0.5).bfloat16()
    if a.which == "ring":
        from . import drivers
        P = 16
        qz, kz, vz = (ops.zigzag_reorder(t, P) for t in (q, k, v))
        share = drivers.RingShare(qz, kz, vz, P, 0, fused=True)
        for i in range(a.iters):
            share.forward()
            torch.cuda.synchronize()
            print(f"ring {S},{Hq},{Hkv},{D} pass {i} done", flush=True)
        return
    out, lse = ops.attn_fwd(q, k, v)
    if a.which == "bwd":
        do = torch.randn(q.shape, device="cuda", generator=g).mul_(0.5).bfloat16()
        ws = ops.bwd_workspace(q, k)
        grads = [torch.empty(t.shape, device="cuda") for t in (q, k, v)]
    for i in range(a.iters):
        if a.which == "fwd":
            ops.attn_fwd(q, k, v, out=out, lse=lse)
        else:
            ops.attn_bwd(q, k, v, out, lse, do, dq=grads[0], dk=grads[1], dv=grads[2], workspace=ws)
        torch.cuda.synchronize()
        print(f"{a.which} {S},{Hq},{Hkv},{D} iteration {i} done", flush=True)


if __name__ == "__main__":
    main()
