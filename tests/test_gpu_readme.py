"""The README's Python usage example runs as written, and what it computes agrees:
the ring pass over P ranks and the Ulysses pass give the same output and gradients
as one attention call over the whole sequence (bf16 inputs, float32 results)."""
import os
import re

import pytest
import torch

README = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "README.md")


def _example() -> str:
    blocks = re.findall(r"```python\n(.*?)```", open(README).read(), re.S)
    assert len(blocks) == 1, "the README holds one Python example"
    return blocks[0]


def test_readme_example_is_present():
    code = _example()
    compile(code, "README.md", "exec")
    for name in ("attn_fwd", "attn_bwd", "RingShare", "ulysses_forward", "ulysses_backward"):
        assert name in code


@pytest.mark.gpu
def test_readme_example_runs_and_agrees():
    print("README example", flush=True)
    torch.manual_seed(0)
    ns = {}
    exec(compile(_example(), "README.md", "exec"), ns)
    cp, B, S, Hq, D, P = ns["cp"], ns["B"], ns["S"], ns["Hq"], ns["D"], ns["P"]
    out, dq, dk, dv = ns["out"], ns["dq"], ns["dk"], ns["dv"]

    def close(got, ref, what):
        err = (got.float() - ref.float()).abs().max().item()
        bound = 2e-2 * max(1.0, ref.float().abs().max().item())
        assert err <= bound, f"{what}: max error {err} > {bound}"

    close(ns["out_ring"], out, "ring out")
    close(cp.zigzag_reorder(ns["dk_z"], P, inverse=True), dk, "ring dk")
    close(cp.zigzag_reorder(ns["dv_z"], P, inverse=True), dv, "ring dv")
    close(ns["o_st"].reshape(B, S, Hq, D), out, "ulysses out")
    close(ns["dq_st"].reshape(B, S, Hq, D), dq, "ulysses dq")
    Hkv = ns["Hkv"]
    close(ns["dk_st"].reshape(B, S, Hkv, D), dk, "ulysses dk")
